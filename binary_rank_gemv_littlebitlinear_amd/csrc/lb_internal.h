// Internal declarations shared by the host library and the kernels.
//
// Device storage of one layer (P paths, rank s, input width a, output
// width b; the sign layouts are defined in lb_layout.h):
//
//   L   = P * s            latent columns, path-major: column c = p*s + k
//   R1  = ceil(a / 32)     32-row groups of S_V;  T16v = 2 R1 16-row tiles
//   Wk  = ceil(s / 32)     words per S_U row and path
//
//   sv16, su2t     the signs, once: S_V by 16-row input tiles (column-major
//                  over latent columns, so lane c of a wave reads column c
//                  and a 16-row tile of all columns is one contiguous
//                  block), S_U by 16-row output tiles (one contiguous block
//                  of P * Wk * 16 words per tile).  Every M < 64 kernel and
//                  the stack sweep read these.
//   sv1m, su2m     the matrix-core copies (bits inverted and permuted for
//                  the fp16 operand sign flips), built on the first call
//                  with M >= 64 (null until then).
//   h[p*b16 + j], g[p*a16 + i], l[p*s8 + k]   (fp16 bit patterns; padded
//                  per-path pitches, s8 = s rounded up to 8, zero padding)
//   ht, gt         h and g by 16-row tiles (the sweep's staging blocks)
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
  uint16_t *h = nullptr;    // P * b16
  uint16_t *g = nullptr;    // P * a16
  uint16_t *l = nullptr;    // P * s8
  int64_t a16 = 0, b16 = 0, s8 = 0, Lp = 0, T16a = 0, T16v = 0, T16b = 0;
  uint16_t *sv16 = nullptr; // T16v * Lp
  uint32_t *su2t = nullptr; // T16b * P * Wk * 16
  uint16_t *ht = nullptr;   // T16b * P * 16
  uint16_t *gt = nullptr;   // T16a * P * 16
  uint32_t *sv1m = nullptr; // R1 * L words (matrix-core bit order), null until first needed
  uint32_t *su2m = nullptr; // P * Wk * b16 words (matrix-core bit order), null until first needed
  // The layer's own forward workspace (wave-path chunk partials and latent
  // rows, or the matrix-core latent T and split-K partials) and split-K
  // tile counters (zero between launches), allocated at create time and
  // kept until destroy: forward calls on different layers share nothing.
  float *ws = nullptr;
  size_t ws_bytes = 0;
  unsigned *cnt = nullptr;
  int wave_rows = 1;  // rows per wave-path launch pair (the partials fit ws)
  // state of the one-launch M = 1 forward (one 64-bit ticket-and-generation
  // word, then the tagged chunk partials), zeroed at create; null when the
  // layer is outside it
  void *f1state = nullptr;
  bool ready() const {
    for (int p = 0; p < P; ++p)
      if (!signs_set[p] || !scales_set[p]) return false;
    return true;
  }
};

struct MfmaPlan;
struct Forward1Plan {
  int G = 0, N1 = 0, N2 = 0, wpl = 0;
  size_t lds = 0, state_bytes = 0;
};

}  // namespace lbi

// The C ABI's opaque layer handle.
struct lb_layer {
  lbi::Layer ly;
  void *ctx = nullptr;  // the device context (device facts, zero block)
  lbi::MfmaPlan *mplan = nullptr;  // the layer as a one-layer MFMA unit
  bool f1 = false;                 // the one-launch M = 1 forward applies
  lbi::Forward1Plan *f1plan = nullptr;
};

namespace lbi {

// ------------------------------------------------------------- launchers
// All return hipError_t of the launch (no synchronisation).

// Wave path, M < 64.  ws must hold wave_ws_floats(L, M, nchunk) floats.
size_t wave_ws_floats(const Layer &Ly, int64_t M, int nchunk);
int wave_nchunk(const Layer &Ly, int64_t M, const DeviceInfo &dev);
hipError_t launch_wave_stage1(const Layer &Ly, const uint16_t *x, float *w_out, int64_t M,
                              int nchunk, float *ws, hipStream_t st);
// With cout: also cout = fp16(c * (cin[0] + .. + cin[ncin - 1] + y)), the
// unit's combine (ncin <= 7), when wave_stage2_combines(Ly).
hipError_t launch_wave_stage2(const Layer &Ly, const float *w, uint16_t *y, int64_t M,
                              const DeviceInfo &dev, hipStream_t st, const uint16_t *const *cin = nullptr,
                              int ncin = 0, float c = 0.f, uint16_t *cout = nullptr);
bool wave_stage2_combines(const Layer &Ly);

// One launch for M = 1 on small layers (a <= 4096 input rows, at most 256
// latent columns: first product, reduction and second product by workgroup
// role; see lb_wave.hip).  state: state_bytes of device memory,
// zero before the first launch, owned by the layer (launches on it must be
// stream-ordered); herr: a host-mapped word set when a wait gives up.
bool forward1_plan(const Layer &Ly, Forward1Plan *pl);
hipError_t launch_forward1(const Layer &Ly, const Forward1Plan &pl, void *state, unsigned *herr,
                           const uint16_t *x, uint16_t *y, hipStream_t st);

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

// The whole stack for M >= 64 in one launch per 256 rows (lb_mfma.hip):
// the unit tiles above as work items dealt round robin, each waiting only for
// the previous step of its own 32-row block.  Built from the stack's unit
// plans (null when a width is not a multiple of 8 or the device cannot
// hold the kernel).  ws and cnt as for launch_mfma_unit, sized by
// mstack_ws_bytes and mstack_cnt_entries; xb0, xb1 hold 256 rows of the
// widest unit width each.  Launches only once an argument set for the row
// count and these buffers exists (built on first use outside capture;
// LB_ENOTREADY under capture); LB_ETIMEOUT once after a launch gave up a
// wait (the next call resets).
struct MStackPlan;
MStackPlan *mstack_build(const std::vector<const MfmaPlan *> &units, float kappa, const DeviceInfo &dev);
void mstack_free(MStackPlan *p);
size_t mstack_ws_bytes(const MStackPlan *p);
size_t mstack_cnt_entries(const MStackPlan *p);
// Whether the argument sets of every 256-row chunk of M exist for these
// buffers (no side effects).
bool mstack_ready(const MStackPlan *p, int64_t M, void *ws, unsigned *cnt, uint16_t *xb0, uint16_t *xb1);
lb_status mstack_run(MStackPlan *p, const uint16_t *x0, uint16_t *y, int64_t M, void *ws, unsigned *cnt,
                     uint16_t *xb0, uint16_t *xb1, const void *zero, const DeviceInfo &dev,
                     hipStream_t st, std::string *msg);

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

// The forward of one layer with caller-chosen scratch (see lb_api.hip),
// the argument checks of lb_forward, and the thread-local error text.
// A unit's combine for the wave path's second product (see launch_wave_stage2).
struct CombineReq {
  const uint16_t *const *in;  // the unit's earlier layers' outputs, M x b each
  int n;
  float c;
  uint16_t *out;
};
lb_status forward_ws(const lb_layer *L, const uint16_t *x, uint16_t *y, int64_t M, hipStream_t st,
                     void *ws, size_t ws_bytes, unsigned *cnt, size_t cnt_entries, std::string *msg,
                     const CombineReq *comb = nullptr);
lb_status forward_checks(const lb_layer *L, const void *x, const void *y, int64_t M, const char *who);
lb_status set_error(lb_status st, const std::string &msg);
const void *device_zero(const lb_layer *L);
// The matrix-core sign copies of a layer, built if missing when may_alloc
// and the stream is not capturing (allocates, synchronises the device);
// LB_ENOTREADY otherwise.
lb_status ensure_mfma_copies(const lb_layer *L, hipStream_t st, bool may_alloc, const char *who);

// fp16 out[M x n] = fp16(c * sum_u in_u[M x n]) for n_in inputs.
hipError_t launch_combine(const uint16_t *const *ins, int n_in, float c, uint16_t *out,
                          int64_t elems, hipStream_t st);

}  // namespace lbi
