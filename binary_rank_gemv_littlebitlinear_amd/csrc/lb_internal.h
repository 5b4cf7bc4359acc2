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
//   su2[(p*Wk + q) * b + j]        (uint32, P*Wk x b)
//       bit (k % 32) = S_U,p[j, 32 q + bit].  Row j's words of one path
//       are b apart, so lane j of a wave reads consecutive addresses.
//   h[p*b + j], g[p*a + i], l[p*s + k]   (fp16 bit patterns)
//
// Padding bits (i >= a in the last row group of sv1, k >= s in the last
// word of su2) are zero, so they contribute nothing.
//
// Lane-mask layouts for the wave-level kernels.  A 64-bit mask holds one
// bit per lane of a 64-lane wave; the kernels turn it into a per-lane
// predicate and add a broadcast value in the lanes whose bit is set
// (sign-flip identity).  Lanes are split 16 x 4: lane = 16*q + r.
//
//   T16a = ceil(a / 16), T16b = ceil(b / 16) row tiles of 16 rows
//   NCT  = ceil(L / 16)  column tiles of 16 latent columns
//   Q    = ceil(s / 4),  Qp = Q rounded up to a multiple of 4
//
//   m1[(tau * NCT + kap) * 4 + i]          (uint64, T16a x NCT x 4)
//       bit (16 q + cc) = S_V[16 tau + 4 q + i, column 16 kap + cc]
//       (columns of the concatenated latent c = p*s + k; lane 16q+cc of
//       the first product accumulates column 16kap+cc over rows 4q+i).
//   m2[((p * T16b + tau) * Qp) + i]         (uint64, P x T16b x Qp)
//       bit (16 q + r) = S_U,p[16 tau + r, q*Q + i]   (0 if q*Q+i >= s)
//       (lane 16q+r of the second product accumulates row 16tau+r over
//       the latent quarter q).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  uint32_t *su2 = nullptr;  // P * Wk * b words
  uint16_t *h = nullptr;    // P * b
  uint16_t *g = nullptr;    // P * a
  uint16_t *l = nullptr;    // P * s
  int64_t T16a = 0, T16b = 0, NCT = 0, Q = 0, Qp = 0;
  uint64_t *m1 = nullptr;   // T16a * NCT * 4
  uint64_t *m2 = nullptr;   // P * T16b * Qp
  // host copies of the canonical S_V words of each path, kept until every
  // path is packed (m1 interleaves the paths' columns)
  std::vector<uint32_t> sv_host[2];
  // workspace: stage-1 partials / latent vectors, sized at create time
  float *ws = nullptr;
  size_t ws_bytes = 0;
  bool ready() const {
    for (int p = 0; p < P; ++p)
      if (!signs_set[p] || !scales_set[p]) return false;
    return true;
  }
};

}  // namespace lbi

// The C ABI's opaque layer handle.
struct lb_layer {
  lbi::Layer ly;
  void *ctx = nullptr;  // the device context (workspace owner)
  void *plan = nullptr; // single-layer persistent plan (M = 1), may be null
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

// MFMA path, any M (used for M >= 64).  ws must hold mfma_ws_bytes().
size_t mfma_ws_bytes(const Layer &Ly, int64_t M);
hipError_t launch_mfma_forward(const Layer &Ly, const uint16_t *x, uint16_t *y, int64_t M,
                               void *ws, const DeviceInfo &dev, hipStream_t st);

// fp16 out[M x n] = fp16(c * sum_u in_u[M x n]) for n_in inputs.
hipError_t launch_combine(const uint16_t *const *ins, int n_in, float c, uint16_t *out,
                          int64_t elems, hipStream_t st);

}  // namespace lbi
