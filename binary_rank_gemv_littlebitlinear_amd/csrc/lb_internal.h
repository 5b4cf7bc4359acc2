// Internal declarations shared by the host library and the kernels.
//
// Device layout of one layer (P paths, rank s, input width a, output
// width b).  The canonical host layout packs each factor row along s; the
// device layouts below are chosen for the kernels that read them.
//
//   L   = P * s            latent columns, path-major: column c = p*s + k
//   R1  = ceil(a / 32)     row groups of S_V
//   Wk  = ceil(s / 32)     words per S_U row and path
//
//   sv1[r * L + c]                 (uint32, R1 x L)
//       bit (i % 32) = S_V,p[i, k] for i = 32 r + bit, c = p*s + k.
//       Column-major bits over the input index: lane c of a wave reads
//       its own column's word, so a wave's load of one row group is one
//       contiguous, coalesced 4*64-byte segment.
//   su2[(p*Wk + q) * b16 + j]      (uint32, P*Wk x b16, b16 = b rounded up to 16)
//       bit (k % 32) = S_U,p[j, 32 q + bit].  Row j's words of one path
//       are b16 apart, so lane j of a wave reads consecutive addresses, and
//       the words of 16-row tiles start on 64-byte boundaries.
//   sv16[gi * Lp + c]              (uint16, T16a x Lp, Lp = L rounded up to 8)
//       bit (i % 16) = S_V,p[i, k] for i = 16 gi + bit, c = p*s + k: the
//       first product's bits by 16-row groups, so a workgroup owning whole
//       16-row tiles reads one contiguous, 16-byte aligned block.
//   h[p*b16 + j], g[p*a16 + i], l[p*s8 + k]   (fp16 bit patterns; padded
//       per-path pitches, s8 = s rounded up to 8, zero padding)
//
// Tile-major copies for the persistent sweep, where a workgroup owns whole
// 16-row tiles and stages them into LDS as one contiguous block each:
//   su2t[((tau * P + p) * Wk + q) * 16 + r]   (uint32) = su2 word q, path p,
//       row 16 tau + r
//   ht[(tau * P + p) * 16 + r] = h[p*b16 + 16 tau + r]   (fp16)
//   gt[(tau * P + p) * 16 + r] = g[p*a16 + 16 tau + r]   (fp16)
//
// Copies for the matrix-core path, same indexing as sv1 / su2 but with each
// word's bits inverted (1 = sign -1) and permuted: the sign of element
// 8 g + e (g = 0..3, e = 0..7) sits at bit 15 - e/2 - 4 g for even e and
// 31 - (e - 1)/2 - 4 g for odd e.  Shifting the word left by 4 g + j and
// masking 0x80008000 then gives the fp16 sign flips of elements 8 g + 2 j
// and 8 g + 2 j + 1, one 32-bit operand register of a lane's 8 values:
//   sv1m[r * L + c], su2m[(p*Wk + q) * b16 + j]
//
// Padding bits and padding scales are zero, so they contribute nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/lb.h"

namespace lbi {

struct DeviceInfo {
  int device = -1;
  int cu_count = 0;
  int coop = 0;           // cooperative launch supported
  int max_wg_per_cu = 0;  // for the persistent kernel (filled lazily)
};

struct Layer {
  int64_t a = 0, b = 0, s = 0;
  int P = 1;
  int device = 0;
  int64_t L = 0, R1 = 0, Wk = 0;
  bool signs_set[2] = {false, false};
  bool scales_set[2] = {false, false};
  uint32_t *sv1 = nullptr;  // R1 * L words
  uint32_t *su2 = nullptr;  // P * Wk * b16 words
  uint16_t *h = nullptr;    // P * b16
  uint16_t *g = nullptr;    // P * a16
  uint16_t *l = nullptr;    // P * s8
  int64_t a16 = 0, b16 = 0, s8 = 0, Lp = 0, T16a = 0, T16b = 0;
  uint16_t *sv16 = nullptr; // T16a * Lp
  uint32_t *su2t = nullptr; // T16b * P * Wk * 16
  uint16_t *ht = nullptr;   // T16b * P * 16
  uint16_t *gt = nullptr;   // T16a * P * 16
  uint32_t *sv1m = nullptr; // R1 * L words (matrix-core bit order)
  uint32_t *su2m = nullptr; // P * Wk * b16 words (matrix-core bit order)
  // workspace: stage-1 partials / latent vectors, sized at create time
  float *ws = nullptr;
  size_t ws_bytes = 0;
  bool ready() const {
    for (int p = 0; p < P; ++p)
      if (!signs_set[p] || !scales_set[p]) return false;
    return true;
  }
};

struct MfmaPlan;

}  // namespace lbi

// The C ABI's opaque layer handle.
struct lb_layer {
  lbi::Layer ly;
  void *ctx = nullptr;  // the device context (workspace owner)
  lbi::MfmaPlan *mplan = nullptr;  // the layer as a one-layer MFMA unit
};

namespace lbi {

// ------------------------------------------------------------- launchers
// All return hipError_t of the launch (no synchronisation).

// Wave path, M < 64.  ws must hold wave_ws_floats(L, M, nchunk) floats.
size_t wave_ws_floats(const Layer &Ly, int64_t M, int nchunk);
int wave_nchunk(const Layer &Ly, int64_t M, const DeviceInfo &dev);
hipError_t launch_wave_stage1(const Layer &Ly, const uint16_t *x, float *w_out, int64_t M,
                              int nchunk, float *ws, hipStream_t st);
hipError_t launch_wave_stage2(const Layer &Ly, const float *w, uint16_t *y, int64_t M,
                              hipStream_t st);

// MFMA path (used for M >= 64) over a unit: 1..kMaxUnitLayersM layers of
// one shape that read the same input.  Rows are processed kMfmaRows at a
// time.  ws must hold mfma_unit_ws_bytes() and cnt mfma_cnt_entries()
// counters that are zero before the first launch (the kernels leave them
// zero); zero points to >= 256 zero bytes of device memory.  direct: y_layers[0] = the layer's output; otherwise xout =
// fp16(c_out * sum_m fp16(y_m)) and each non-null y_layers[m] receives y_m.
constexpr int kMaxUnitLayersM = 8;
constexpr int kMaxUnitSegs = 2 * kMaxUnitLayersM;
constexpr int kMfmaRows = 256;
struct MfmaPlan;
MfmaPlan *mfma_plan_build(const Layer *const *layers, int n);  // null if unsupported
void mfma_plan_free(MfmaPlan *p);
size_t mfma_unit_ws_bytes(const MfmaPlan *p);
size_t mfma_cnt_entries(const MfmaPlan *p);
hipError_t launch_mfma_unit(const MfmaPlan *p, const uint16_t *x, int64_t M,
                            uint16_t *const *y_layers, uint16_t *xout, float c_out, bool direct,
                            void *ws, unsigned *cnt, const void *zero, const DeviceInfo &dev,
                            hipStream_t st);

// Initialisation of one path from real device factors U (b x s) and
// V (a x s), fp32 row-major.  ws holds init_ws_bytes(a, b, s) bytes; the
// results are device pointers into ws: canonical sign words su (b x Wk),
// sv (a x Wk), fp16 bits h (b), g (a), l (s), and sigma[0..1] (top singular
// values of |U| and |V|).  Synchronises st while iterating.
struct InitResult {
  uint32_t *su = nullptr, *sv = nullptr;
  uint16_t *h = nullptr, *g = nullptr, *l = nullptr;
  double *sigma = nullptr;
  int iters_u = 0, iters_v = 0;
  bool converged = false;
};
size_t init_ws_bytes(int64_t a, int64_t b, int64_t s);
hipError_t init_from_factors_dev(const float *U, const float *V, int64_t a, int64_t b, int64_t s,
                                 void *ws, hipStream_t st, InitResult *res);
// The same from fp64 factors (the rotated factors of Joint-ITQ).
hipError_t init_from_factors_dev(const double *U, const double *V, int64_t a, int64_t b, int64_t s,
                                 void *ws, hipStream_t st, InitResult *res);

// Joint-ITQ on the device.  Each returns 0 on success, otherwise an
// lb_status value with the reason in *msg.
//   joint_itq_dev: R (s x s, fp64 row-major, device) = the rotation after
//     `iters` steps on X = [U; V] (U b x s, V a x s, fp32 device), started
//     from R0 (device, fp64) or the identity when R0 is null.  Allocates its
//     temporaries; synchronises st.
//   rotate_factors_dev: out ((b + a) x s, fp64 device) = [U; V] R.
int joint_itq_dev(const float *U, const float *V, int64_t a, int64_t b, int64_t s, int iters,
                  const double *R0, double *R, hipStream_t st, std::string *msg);
int rotate_factors_dev(const float *U, const float *V, int64_t a, int64_t b, int64_t s,
                       const double *R, double *out, hipStream_t st, std::string *msg);

// fp16 out[M x n] = fp16(c * sum_u in_u[M x n]) for n_in inputs.
hipError_t launch_combine(const uint16_t *const *ins, int n_in, float c, uint16_t *out,
                          int64_t elems, hipStream_t st);

}  // namespace lbi
