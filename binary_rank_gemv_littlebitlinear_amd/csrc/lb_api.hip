// Host side of the C ABI declared in include/lb.h: argument checks, the
// canonical -> device sign re-layout, device storage, dispatch by M, the
// effective-bit arithmetic of [LB2 column] Ch. 1 and the stack runner.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "lb_internal.h"
#include "lb_layout.h"
#include "lb_persist.h"

using namespace lbi;

// ------------------------------------------------------------ errors
static thread_local std::string g_last_error;

static lb_status fail(lb_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

#define LB_HIP(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess)                                                         \
      return fail(LB_EHIP, std::string(#call) + ": " + hipGetErrorString(e_));    \
  } while (0)

// ------------------------------------------------------------ devices
namespace {
// Per-device facts and one read-only block of zero bytes (the DMA source
// for padding).  Nothing here is written after it is set up, so layers and
// stacks on one device share it freely; every buffer a forward call writes
// belongs to its layer or stack.
struct DevCtx {
  DeviceInfo info;
  void *zero = nullptr;  // 256 zero bytes
  // pinned host word set by a one-launch M = 1 forward whose wait gave up
  // (reported by the next such lb_forward on the device), and its device address
  unsigned *herr = nullptr, *herr_dev = nullptr;
};
std::mutex g_mu;
std::map<int, DevCtx> g_dev;

lb_status get_dev(int device, DevCtx **out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(device);
  if (it == g_dev.end()) {
    DevCtx c;
    c.info.device = device;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    c.info.cu_count = prop.multiProcessorCount;
    c.info.coop = prop.cooperativeLaunch;
    e = hipMalloc(&c.zero, 256);
    if (e == hipSuccess) e = hipMemset(c.zero, 0, 256);
    if (e == hipSuccess) e = hipHostMalloc(&c.herr, 64, hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) e = hipHostGetDevicePointer((void **)&c.herr_dev, c.herr, 0);
    if (e != hipSuccess) return fail(LB_ENOMEM, std::string("device context allocation: ") + hipGetErrorString(e));
    *(volatile unsigned *)c.herr = 0u;
    it = g_dev.emplace(device, c).first;
  }
  *out = &it->second;
  return LB_OK;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

static inline DevCtx *ctx_of(const lb_layer *L) { return static_cast<DevCtx *>(L->ctx); }
static lbl::Dims dims_of(const Layer &Ly) { return lbl::dims(Ly.a, Ly.b, Ly.s, Ly.P); }

// --------------------------------------------------------- workspace need
// The wave path keeps one fp32 partial latent vector per input chunk and
// row; a layer's launches take at most wave_rows rows at a time, so these
// partials stay within kWavePartBudget bytes (at least one row).
constexpr size_t kWavePartBudget = (size_t)4 << 20;

static int wave_rows_for(const Layer &Ly, const DeviceInfo &dev) {
  const int nch = wave_nchunk(Ly, 1, dev);
  const size_t per_row = wave_ws_floats(Ly, 1, nch) * sizeof(float);
  const size_t r = kWavePartBudget / std::max<size_t>(per_row, 1);
  return (int)std::max<size_t>(1, std::min<size_t>(63, r));
}

static size_t layer_ws_need(const Layer &Ly, const MfmaPlan *mp, const DeviceInfo &dev) {
  const int Mw = Ly.wave_rows;
  const int nch = wave_nchunk(Ly, Mw, dev);
  size_t need = (wave_ws_floats(Ly, Mw, nch) + (size_t)Mw * Ly.L) * sizeof(float) + 512;
  need = std::max(need, mfma_unit_ws_bytes(mp));
  return need;
}

// ------------------------------------------------------------- layers
extern "C" lb_status lb_create(int64_t a, int64_t b, int64_t s, int residual, lb_layer **out) {
  if (!out) return fail(LB_EINVAL, "lb_create: out is NULL");
  if (a < 1 || b < 1 || s < 1) return fail(LB_EINVAL, "lb_create: a, b, s must be >= 1");
  if (a > (1 << 24) || b > (1 << 24) || s > 4096)
    return fail(LB_EINVAL, "lb_create: a, b must be <= 2^24 and s <= 4096");
  if (residual != 0 && residual != 1) return fail(LB_EINVAL, "lb_create: residual must be 0 or 1");
  int device = 0;
  LB_HIP(hipGetDevice(&device));
  DevCtx *dc = nullptr;
  lb_status st = get_dev(device, &dc);
  if (st != LB_OK) return st;

  lb_layer *L = new (std::nothrow) lb_layer();
  if (!L) return fail(LB_ENOMEM, "lb_create: host allocation");
  Layer &Ly = L->ly;
  Ly.a = a; Ly.b = b; Ly.s = s; Ly.P = residual ? 2 : 1; Ly.device = device;
  {
    const lbl::Dims d = lbl::dims(a, b, s, Ly.P);
    Ly.L = d.L; Ly.R1 = d.R1; Ly.Wk = d.Wk;
    Ly.T16a = d.T16a; Ly.T16v = d.T16v; Ly.T16b = d.T16b;
    Ly.a16 = d.a16; Ly.b16 = d.b16; Ly.Lp = d.Lp;
    Ly.s8 = (s + 7) / 8 * 8;
  }
  L->ctx = dc;
  // the signs are held once, in the tile layouts every batch-1 and
  // small-batch kernel reads; the matrix-core copies come with the first
  // call that needs them (ensure_mfma_copies)
  struct Alloc { void **p; size_t n; };
  Alloc allocs[] = {
      {(void **)&Ly.sv16, (size_t)Ly.T16v * Ly.Lp * 2},
      {(void **)&Ly.su2t, (size_t)Ly.T16b * Ly.P * Ly.Wk * 16 * 4},
      {(void **)&Ly.h, (size_t)Ly.P * Ly.b16 * 2},
      {(void **)&Ly.g, (size_t)Ly.P * Ly.a16 * 2},
      {(void **)&Ly.l, (size_t)Ly.P * Ly.s8 * 2},
      {(void **)&Ly.ht, (size_t)Ly.T16b * Ly.P * 16 * 2},
      {(void **)&Ly.gt, (size_t)Ly.T16a * Ly.P * 16 * 2}};
  for (auto &al : allocs) {
    hipError_t e = hipMalloc(al.p, al.n);
    if (e != hipSuccess) {
      lb_destroy(L);
      return fail(LB_ENOMEM, std::string("lb_create: hipMalloc: ") + hipGetErrorString(e));
    }
    e = hipMemset(*al.p, 0, al.n);
    if (e != hipSuccess) {
      lb_destroy(L);
      return fail(LB_EHIP, std::string("lb_create: hipMemset: ") + hipGetErrorString(e));
    }
  }
  {
    const Layer *one = &Ly;
    L->mplan = mfma_plan_build(&one, 1);
  }
  if (!L->mplan) {
    lb_destroy(L);
    return fail(LB_EUNSUPPORTED, "lb_create: shape not supported by the MFMA path");
  }
  Ly.wave_rows = wave_rows_for(Ly, dc->info);
  Ly.ws_bytes = layer_ws_need(Ly, L->mplan, dc->info);
  const size_t ncnt = std::max<size_t>(1, mfma_cnt_entries(L->mplan));
  hipError_t e = hipMalloc(&Ly.ws, Ly.ws_bytes);
  if (e == hipSuccess) e = hipMalloc(&Ly.cnt, ncnt * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemset(Ly.cnt, 0, ncnt * sizeof(unsigned));
  {
    Forward1Plan pl;
    if (e == hipSuccess && forward1_plan(Ly, &pl)) {
      L->f1plan = new (std::nothrow) Forward1Plan(pl);
      if (!L->f1plan) e = hipErrorOutOfMemory;
      if (e == hipSuccess) e = hipMalloc(&Ly.f1state, pl.state_bytes);
      if (e == hipSuccess) e = hipMemset(Ly.f1state, 0, pl.state_bytes);
      L->f1 = e == hipSuccess;
    }
  }
  if (e != hipSuccess) {
    lb_destroy(L);
    return fail(LB_ENOMEM, std::string("lb_create: workspace hipMalloc: ") + hipGetErrorString(e));
  }
  *out = L;
  return LB_OK;
}

extern "C" lb_status lb_destroy(lb_layer *L) {
  if (!L) return LB_OK;
  DeviceGuard g(L->ly.device);
  Layer &Ly = L->ly;
  void *ps[] = {Ly.h, Ly.g, Ly.l, Ly.sv16, Ly.su2t, Ly.ht, Ly.gt, Ly.sv1m, Ly.su2m,
                Ly.ws, Ly.cnt, Ly.f1state};
  for (void *p : ps)
    if (p) (void)hipFree(p);
  mfma_plan_free(L->mplan);
  delete L->f1plan;
  delete L;
  return LB_OK;
}

extern "C" lb_status lb_prepare(lb_layer *L, int64_t M) {
  if (!L || M < 0) return fail(LB_EINVAL, "lb_prepare: bad argument");
  if (M < 64) return LB_OK;
  DeviceGuard dg(L->ly.device);
  return ensure_mfma_copies(L, nullptr, true, "lb_prepare");
}

extern "C" lb_status lb_layer_device_bytes(const lb_layer *L, uint64_t *sign_bytes, uint64_t *total_bytes) {
  if (!L) return fail(LB_EINVAL, "lb_layer_device_bytes: NULL layer");
  const Layer &Ly = L->ly;
  const lbl::Dims d = dims_of(Ly);
  uint64_t sb = lbl::sv16_elems(d) * 2 + lbl::su2t_elems(d) * 4;
  if (Ly.sv1m) sb += lbl::sv1m_elems(d) * 4 + lbl::su2m_elems(d) * 4;
  uint64_t tb = sb;
  tb += (uint64_t)Ly.P * (Ly.b16 + Ly.a16 + Ly.s8) * 2;                    // h, g, l
  tb += (lbl::tile16_elems(Ly.b16, Ly.P) + lbl::tile16_elems(Ly.a16, Ly.P)) * 2;  // ht, gt
  tb += Ly.ws_bytes + std::max<size_t>(1, mfma_cnt_entries(L->mplan)) * sizeof(unsigned);
  if (L->f1plan) tb += L->f1plan->state_bytes;
  if (sign_bytes) *sign_bytes = sb;
  if (total_bytes) *total_bytes = tb;
  return LB_OK;
}

extern "C" lb_status lb_layer_shape(const lb_layer *L, int64_t *a, int64_t *b, int64_t *s,
                                    int *residual) {
  if (!L) return fail(LB_EINVAL, "lb_layer_shape: NULL layer");
  if (a) *a = L->ly.a;
  if (b) *b = L->ly.b;
  if (s) *s = L->ly.s;
  if (residual) *residual = L->ly.P == 2;
  return LB_OK;
}

// Build the matrix-core copies of the signs from host tile layouts of
// every path and upload them (allocating them on first use).
static lb_status upload_mfma_copies(Layer &Ly, const std::vector<uint16_t> &v16,
                                    const std::vector<uint32_t> &u2t) {
  const lbl::Dims d = dims_of(Ly);
  std::vector<uint32_t> v1m, u2m;
  try {
    v1m.resize(lbl::sv1m_elems(d));
    u2m.resize(lbl::su2m_elems(d));
  } catch (...) {
    return fail(LB_ENOMEM, "matrix-core sign copies: host allocation");
  }
  lbl::sv1m_from_sv16(d, v16.data(), v1m.data());
  lbl::su2m_from_su2t(d, u2t.data(), u2m.data());
  const bool fresh = !Ly.sv1m;
  uint32_t *pv = Ly.sv1m, *pu = Ly.su2m;
  if (fresh) {
    hipError_t e = hipMalloc(&pv, v1m.size() * 4);
    if (e == hipSuccess) e = hipMalloc(&pu, u2m.size() * 4);
    if (e != hipSuccess) {
      if (pv) (void)hipFree(pv);
      return fail(LB_ENOMEM, std::string("matrix-core sign copies: hipMalloc: ") + hipGetErrorString(e));
    }
  }
  hipError_t e = hipMemcpy(pv, v1m.data(), v1m.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(pu, u2m.data(), u2m.size() * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    if (fresh) {  // never publish copies whose contents are unknown
      (void)hipFree(pv);
      (void)hipFree(pu);
    }
    return fail(LB_EHIP, std::string("matrix-core sign copies: hipMemcpy: ") + hipGetErrorString(e));
  }
  Ly.sv1m = pv;
  Ly.su2m = pu;
  return LB_OK;
}

// Re-lay host canonical words of one path out for the device (the caller
// has checked the arguments and made the layer's device current).  The
// tile layouts interleave the paths, so each buffer is read back, has this
// path's part replaced and is written whole.  Returns once the device holds
// the new words (a later launch on any stream sees them).
static lb_status pack_signs_impl(Layer &Ly, int path, const uint32_t *su, const uint32_t *sv) {
  const lbl::Dims d = dims_of(Ly);
  std::vector<uint16_t> v16;
  std::vector<uint32_t> u2t;
  try {
    v16.assign(lbl::sv16_elems(d), 0);
    u2t.assign(lbl::su2t_elems(d), 0u);
  } catch (...) {
    return fail(LB_ENOMEM, "lb_pack_signs: host allocation");
  }
  if (Ly.P > 1) {
    LB_HIP(hipMemcpy(v16.data(), Ly.sv16, v16.size() * 2, hipMemcpyDeviceToHost));
    LB_HIP(hipMemcpy(u2t.data(), Ly.su2t, u2t.size() * 4, hipMemcpyDeviceToHost));
  }
  lbl::put_sv16(d, path, sv, v16.data());
  lbl::put_su2t(d, path, su, u2t.data());
  LB_HIP(hipMemcpy(Ly.sv16, v16.data(), v16.size() * 2, hipMemcpyHostToDevice));
  LB_HIP(hipMemcpy(Ly.su2t, u2t.data(), u2t.size() * 4, hipMemcpyHostToDevice));
  if (Ly.sv1m) {  // already built: keep them current
    lb_status st = upload_mfma_copies(Ly, v16, u2t);
    if (st != LB_OK) return st;
  }
  LB_HIP(hipDeviceSynchronize());
  Ly.signs_set[path] = true;
  return LB_OK;
}

// The matrix-core copies of the signs, built on the first call that needs
// them.  That call allocates and synchronises the device, so it must not be
// captured into a graph and cannot come from lb_forward_noalloc: those
// report LB_ENOTREADY instead (lb_prepare builds the copies ahead).
lb_status lbi::ensure_mfma_copies(const lb_layer *L, hipStream_t st, bool may_alloc, const char *who) {
  Layer &Ly = const_cast<lb_layer *>(L)->ly;
  if (Ly.sv1m) return LB_OK;
  const std::string pre = std::string(who) + ": ";
  const std::string hint = "the matrix-core copy of the signs (M >= 64) is not built yet; call lb_prepare "
                           "(or lb_stack_reserve) with M >= 64 first";
  if (!may_alloc) return fail(LB_ENOTREADY, pre + hint);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  LB_HIP(hipStreamIsCapturing(st, &cs));
  if (cs != hipStreamCaptureStatusNone) return fail(LB_ENOTREADY, pre + hint + " (the stream is capturing)");
  if (!Ly.ready()) return fail(LB_ENOTREADY, pre + "signs/scales not set for every path");
  const lbl::Dims d = dims_of(Ly);
  std::vector<uint16_t> v16;
  std::vector<uint32_t> u2t;
  try {
    v16.resize(lbl::sv16_elems(d));
    u2t.resize(lbl::su2t_elems(d));
  } catch (...) {
    return fail(LB_ENOMEM, pre + "host allocation");
  }
  LB_HIP(hipMemcpy(v16.data(), Ly.sv16, v16.size() * 2, hipMemcpyDeviceToHost));
  LB_HIP(hipMemcpy(u2t.data(), Ly.su2t, u2t.size() * 4, hipMemcpyDeviceToHost));
  lb_status s = upload_mfma_copies(Ly, v16, u2t);
  if (s != LB_OK) return fail(s, pre + g_last_error);
  LB_HIP(hipDeviceSynchronize());
  return LB_OK;
}

extern "C" lb_status lb_pack_signs(lb_layer *L, int path, const uint32_t *su, const uint32_t *sv) {
  if (!L || !su || !sv) return fail(LB_EINVAL, "lb_pack_signs: NULL argument");
  Layer &Ly = L->ly;
  if (path < 0 || path >= Ly.P) return fail(LB_EINVAL, "lb_pack_signs: path out of range");
  DeviceGuard dg(Ly.device);
  return pack_signs_impl(Ly, path, su, sv);
}

extern "C" lb_status lb_unpack_signs(const lb_layer *L, int path, uint32_t *su, uint32_t *sv) {
  if (!L || !su || !sv) return fail(LB_EINVAL, "lb_unpack_signs: NULL argument");
  const Layer &Ly = L->ly;
  if (path < 0 || path >= Ly.P) return fail(LB_EINVAL, "lb_unpack_signs: path out of range");
  DeviceGuard dg(Ly.device);
  const lbl::Dims d = dims_of(Ly);
  std::vector<uint16_t> v16;
  std::vector<uint32_t> u2t;
  try {
    v16.resize(lbl::sv16_elems(d));
    u2t.resize(lbl::su2t_elems(d));
  } catch (...) {
    return fail(LB_ENOMEM, "lb_unpack_signs: host allocation");
  }
  LB_HIP(hipMemcpy(v16.data(), Ly.sv16, v16.size() * 2, hipMemcpyDeviceToHost));
  LB_HIP(hipMemcpy(u2t.data(), Ly.su2t, u2t.size() * 4, hipMemcpyDeviceToHost));
  lbl::get_sv16(d, path, v16.data(), sv);
  lbl::get_su2t(d, path, u2t.data(), su);
  return LB_OK;
}

static lb_status set_scales_impl(Layer &Ly, int path, const uint16_t *h, const uint16_t *g,
                                 const uint16_t *l) {
  LB_HIP(hipMemcpy(Ly.h + (size_t)path * Ly.b16, h, Ly.b * 2, hipMemcpyHostToDevice));
  LB_HIP(hipMemcpy(Ly.g + (size_t)path * Ly.a16, g, Ly.a * 2, hipMemcpyHostToDevice));
  LB_HIP(hipMemcpy(Ly.l + (size_t)path * Ly.s8, l, Ly.s * 2, hipMemcpyHostToDevice));
  {
    // tile copies of h and g (the paths interleave per tile, so each buffer
    // is read back and written whole)
    const size_t nh = lbl::tile16_elems(Ly.b16, Ly.P), ng = lbl::tile16_elems(Ly.a16, Ly.P);
    std::vector<uint16_t> hb(nh, 0), gb(ng, 0);
    if (Ly.P > 1) {
      LB_HIP(hipMemcpy(hb.data(), Ly.ht, nh * 2, hipMemcpyDeviceToHost));
      LB_HIP(hipMemcpy(gb.data(), Ly.gt, ng * 2, hipMemcpyDeviceToHost));
    }
    lbl::put_tile16(Ly.b, Ly.b16, Ly.P, path, h, hb.data());
    lbl::put_tile16(Ly.a, Ly.a16, Ly.P, path, g, gb.data());
    LB_HIP(hipMemcpy(Ly.ht, hb.data(), nh * 2, hipMemcpyHostToDevice));
    LB_HIP(hipMemcpy(Ly.gt, gb.data(), ng * 2, hipMemcpyHostToDevice));
  }
  LB_HIP(hipDeviceSynchronize());
  Ly.scales_set[path] = true;
  return LB_OK;
}

extern "C" lb_status lb_set_scales(lb_layer *L, int path, const uint16_t *h, const uint16_t *g,
                                   const uint16_t *l) {
  if (!L || !h || !g || !l) return fail(LB_EINVAL, "lb_set_scales: NULL argument");
  Layer &Ly = L->ly;
  if (path < 0 || path >= Ly.P) return fail(LB_EINVAL, "lb_set_scales: path out of range");
  DeviceGuard dg(Ly.device);
  return set_scales_impl(Ly, path, h, g, l);
}

extern "C" lb_status lb_get_scales(const lb_layer *L, int path, uint16_t *h, uint16_t *g,
                                   uint16_t *l) {
  if (!L || !h || !g || !l) return fail(LB_EINVAL, "lb_get_scales: NULL argument");
  const Layer &Ly = L->ly;
  if (path < 0 || path >= Ly.P) return fail(LB_EINVAL, "lb_get_scales: path out of range");
  if (!Ly.scales_set[path]) return fail(LB_ENOTREADY, "lb_get_scales: scales of this path not set");
  DeviceGuard dg(Ly.device);
  LB_HIP(hipMemcpy(h, Ly.h + (size_t)path * Ly.b16, Ly.b * 2, hipMemcpyDeviceToHost));
  LB_HIP(hipMemcpy(g, Ly.g + (size_t)path * Ly.a16, Ly.a * 2, hipMemcpyDeviceToHost));
  LB_HIP(hipMemcpy(l, Ly.l + (size_t)path * Ly.s8, Ly.s * 2, hipMemcpyDeviceToHost));
  return LB_OK;
}

extern "C" lb_status lb_init_from_factors(lb_layer *L, int path, const float *U, const float *V,
                                          const double *R, void *stream) {
  if (!L || !U || !V) return fail(LB_EINVAL, "lb_init_from_factors: NULL argument");
  Layer &Ly = L->ly;
  if (path < 0 || path >= Ly.P) return fail(LB_EINVAL, "lb_init_from_factors: path out of range");
  if (((uintptr_t)U | (uintptr_t)V) & 3u)
    return fail(LB_EINVAL, "lb_init_from_factors: U and V must be 4-byte aligned");
  if ((uintptr_t)R & 7u) return fail(LB_EINVAL, "lb_init_from_factors: R must be 8-byte aligned");
  if (R && (Ly.a + Ly.b) * Ly.s > ((int64_t)1 << 31) - 1)
    return fail(LB_EINVAL, "lb_init_from_factors: with R, (a + b) * s must fit in 31 bits");
  DeviceGuard dg(Ly.device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t a = Ly.a, b = Ly.b, s = Ly.s, Wk = Ly.Wk;
  std::vector<uint32_t> su, sv;
  std::vector<uint16_t> h, g, l;
  try {
    su.resize((size_t)b * Wk);
    sv.resize((size_t)a * Wk);
    h.resize((size_t)b);
    g.resize((size_t)a);
    l.resize((size_t)s);
  } catch (...) {
    return fail(LB_ENOMEM, "lb_init_from_factors: host allocation");
  }
  // with a rotation: the fp64 factors [U R; V R] first
  double *rot = nullptr;
  if (R) {
    hipError_t e = hipMalloc(&rot, (size_t)(a + b) * s * sizeof(double));
    if (e != hipSuccess)
      return fail(LB_ENOMEM, std::string("lb_init_from_factors: hipMalloc: ") + hipGetErrorString(e));
    std::string msg;
    const int rc = rotate_factors_dev(U, V, a, b, s, R, rot, st, &msg);
    if (rc != 0) {
      (void)hipFree(rot);
      return fail((lb_status)rc, "lb_init_from_factors: " + msg);
    }
  }
  void *ws = nullptr;
  hipError_t e = hipMalloc(&ws, init_ws_bytes(a, b, s));
  if (e != hipSuccess) {
    if (rot) (void)hipFree(rot);
    return fail(LB_ENOMEM, std::string("lb_init_from_factors: hipMalloc: ") + hipGetErrorString(e));
  }
  InitResult r;
  e = rot ? init_from_factors_dev(rot, rot + (size_t)b * s, a, b, s, ws, st, &r)
          : init_from_factors_dev(U, V, a, b, s, ws, st, &r);
  if (e == hipSuccess) e = hipMemcpyAsync(su.data(), r.su, su.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(sv.data(), r.sv, sv.size() * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(h.data(), r.h, h.size() * 2, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(g.data(), r.g, g.size() * 2, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(l.data(), r.l, l.size() * 2, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  const hipError_t ef = hipFree(ws);
  if (rot) (void)hipFree(rot);
  if (e != hipSuccess)
    return fail(LB_EHIP, std::string("lb_init_from_factors: ") + hipGetErrorString(e));
  if (ef != hipSuccess)
    return fail(LB_EHIP, std::string("lb_init_from_factors: hipFree: ") + hipGetErrorString(ef));
  if (!r.converged)
    return fail(LB_EUNSUPPORTED,
                "lb_init_from_factors: power iteration did not settle (the top singular value "
                "of |U| or |V| is not separated from the next one); the layer is unchanged");
  lb_status sst = pack_signs_impl(Ly, path, su.data(), sv.data());
  if (sst != LB_OK) return sst;
  return set_scales_impl(Ly, path, h.data(), g.data(), l.data());
}

extern "C" lb_status lb_joint_itq(const float *U, const float *V, int64_t a, int64_t b, int64_t s,
                                  int iters, const double *R0, double *R, void *stream) {
  if (!U || !V || !R) return fail(LB_EINVAL, "lb_joint_itq: NULL argument");
  if (a < 1 || b < 1 || s < 1 || a > (1 << 24) || b > (1 << 24) || s > 4096 || iters < 0)
    return fail(LB_EINVAL, "lb_joint_itq: need 1 <= a, b <= 2^24, 1 <= s <= 4096, iters >= 0");
  if ((a + b) * s > ((int64_t)1 << 31) - 1)
    return fail(LB_EINVAL, "lb_joint_itq: (a + b) * s must fit in 31 bits");
  if ((((uintptr_t)U | (uintptr_t)V) & 3u) || (((uintptr_t)R | (uintptr_t)R0) & 7u))
    return fail(LB_EINVAL, "lb_joint_itq: misaligned pointer");
  std::string msg;
  const int rc = joint_itq_dev(U, V, a, b, s, iters, R0, R, static_cast<hipStream_t>(stream), &msg);
  if (rc != 0) return fail((lb_status)rc, "lb_joint_itq: " + msg);
  return LB_OK;
}

// ------------------------------------------------------------- forward
static bool overlaps(const void *p, size_t np, const void *q, size_t nq) {
  const char *a = (const char *)p, *b = (const char *)q;
  return a < b + nq && b < a + np;
}

static lb_status check_io(const Layer &Ly, const void *x, const void *y, int64_t M,
                          const char *who) {
  if (M < 0) return fail(LB_EINVAL, std::string(who) + ": M < 0");
  if (M == 0) return LB_OK;
  if (!x || !y) return fail(LB_EINVAL, std::string(who) + ": NULL x or y");
  if (((uintptr_t)x & 15) || ((uintptr_t)y & 15))
    return fail(LB_EINVAL, std::string(who) + ": x and y must be 16-byte aligned");
  if (!Ly.ready()) return fail(LB_ENOTREADY, std::string(who) + ": signs/scales not set for every path");
  return LB_OK;
}

// The forward of one layer with the scratch it needs taken from `ws`
// (ws_bytes) and `cnt` (cnt_entries split-K tile counters, zero on entry and
// left zero).  Wave-path launches take as many rows as the partials of ws
// allow (at most 63); LB_EUNSUPPORTED when not even one row, or the
// matrix-core path, fits.
lb_status lbi::forward_ws(const lb_layer *L, const uint16_t *x, uint16_t *y, int64_t M,
                          hipStream_t st, void *ws, size_t ws_bytes, unsigned *cnt,
                          size_t cnt_entries, std::string *msg, const CombineReq *comb) {
  const Layer &Ly = L->ly;
  DevCtx *dc = ctx_of(L);
  if (M < 64) {
    const int nch = wave_nchunk(Ly, 1, dc->info);
    const size_t per_row = (wave_ws_floats(Ly, 1, nch) + (size_t)Ly.L) * sizeof(float);
    const int64_t rows = std::min<int64_t>(63, (int64_t)(ws_bytes / per_row));
    if (rows < 1) {
      if (msg) *msg = "scratch too small for one row of the wave path (needs " + std::to_string(per_row) + " bytes)";
      return LB_EUNSUPPORTED;
    }
    for (int64_t m0 = 0; m0 < M; m0 += rows) {
      const int64_t Mc = std::min<int64_t>(rows, M - m0);
      float *part = reinterpret_cast<float *>(ws);
      float *w = part + wave_ws_floats(Ly, Mc, nch);
      hipError_t e = launch_wave_stage1(Ly, x + m0 * Ly.a, w, Mc, nch, part, st);
      if (e == hipSuccess && comb) {
        const uint16_t *cin[7];
        for (int u = 0; u < comb->n && u < 7; ++u) cin[u] = comb->in[u] + m0 * Ly.b;
        e = launch_wave_stage2(Ly, w, y + m0 * Ly.b, Mc, dc->info, st, cin, comb->n, comb->c,
                               comb->out + m0 * Ly.b);
      } else if (e == hipSuccess) {
        e = launch_wave_stage2(Ly, w, y + m0 * Ly.b, Mc, dc->info, st);
      }
      if (e != hipSuccess) {
        if (msg) *msg = std::string("wave path: ") + hipGetErrorString(e);
        return LB_EHIP;
      }
    }
    return LB_OK;
  }
  if (comb) {
    if (msg) *msg = "a fused combine is for the wave path only";
    return LB_EINVAL;
  }
  if (mfma_unit_ws_bytes(L->mplan) > ws_bytes || mfma_cnt_entries(L->mplan) > cnt_entries) {
    if (msg)
      *msg = "scratch too small for the matrix-core path (needs " +
             std::to_string(mfma_unit_ws_bytes(L->mplan)) + " bytes and " +
             std::to_string(mfma_cnt_entries(L->mplan)) + " counters)";
    return LB_EUNSUPPORTED;
  }
  // built by lb_prepare or by lb_forward's first M >= 64 call, never here:
  // this function allocates nothing
  if (!Ly.sv1m) {
    if (msg) *msg = "the matrix-core copy of the signs is not built yet (lb_prepare with M >= 64)";
    return LB_ENOTREADY;
  }
  uint16_t *ys[1] = {y};
  hipError_t e = launch_mfma_unit(L->mplan, x, M, ys, nullptr, 1.f, true, ws, cnt, dc->zero, dc->info, st);
  if (e != hipSuccess) {
    if (msg) *msg = std::string("mfma path: ") + hipGetErrorString(e);
    return LB_EHIP;
  }
  return LB_OK;
}

// The layer's own workspace (sized at create time for every M); one row
// takes the one-launch forward when the layer fits it.
static lb_status forward_impl(const lb_layer *L, const uint16_t *x, uint16_t *y, int64_t M,
                              hipStream_t st) {
  const Layer &Ly = L->ly;
  if (M == 1 && L->f1) {
    DevCtx *dc = ctx_of(L);
    if (*(volatile unsigned *)dc->herr != 0u) {
      *(volatile unsigned *)dc->herr = 0u;
      return fail(LB_ETIMEOUT, "lb_forward: an earlier one-row forward on this device gave up a "
                               "device-side wait (its output is undefined); this call did not run");
    }
    hipError_t e = launch_forward1(Ly, *L->f1plan, Ly.f1state, dc->herr_dev, x, y, st);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("lb_forward: one-row launch: ") + hipGetErrorString(e));
    return LB_OK;
  }
  if (M >= 64) {
    lb_status es = ensure_mfma_copies(L, st, true, "lb_forward");
    if (es != LB_OK) return es;
  }
  std::string msg;
  const lb_status r = forward_ws(L, x, y, M, st, Ly.ws, Ly.ws_bytes, Ly.cnt,
                                 std::max<size_t>(1, mfma_cnt_entries(L->mplan)), &msg);
  return r == LB_OK ? r : fail(r, "lb_forward: " + msg);
}

// Checks shared by lb_forward and its allocation-free variant.
lb_status lbi::forward_checks(const lb_layer *L, const void *x, const void *y, int64_t M,
                              const char *who) {
  if (!L) return fail(LB_EINVAL, std::string(who) + ": NULL layer");
  const Layer &Ly = L->ly;
  lb_status st = check_io(Ly, x, y, M, who);
  if (st != LB_OK || M == 0) return st;
  if (overlaps(x, (size_t)M * Ly.a * 2, y, (size_t)M * Ly.b * 2))
    return fail(LB_EINVAL, std::string(who) + ": x and y overlap");
  return LB_OK;
}

lb_status lbi::set_error(lb_status st, const std::string &msg) { return fail(st, msg); }
const void *lbi::device_zero(const lb_layer *L) { return ctx_of(L)->zero; }

extern "C" lb_status lb_forward(const lb_layer *L, const void *x, void *y, int64_t M, void *stream) {
  lb_status st = forward_checks(L, x, y, M, "lb_forward");
  if (st != LB_OK || M == 0) return st;
  const Layer &Ly = L->ly;
  DeviceGuard dg(Ly.device);
  return forward_impl(L, (const uint16_t *)x, (uint16_t *)y, M, (hipStream_t)stream);
}

extern "C" lb_status lb_forward_stage1(const lb_layer *L, const void *x, float *w, int64_t M,
                                       void *stream) {
  if (!L) return fail(LB_EINVAL, "lb_forward_stage1: NULL layer");
  const Layer &Ly = L->ly;
  lb_status st = check_io(Ly, x, w, M, "lb_forward_stage1");
  if (st != LB_OK || M == 0) return st;
  DeviceGuard dg(Ly.device);
  DevCtx *dc = ctx_of(L);
  // rows in blocks of wave_rows so the chunk partials fit the layer's workspace
  for (int64_t m0 = 0; m0 < M; m0 += Ly.wave_rows) {
    const int64_t Mc = std::min<int64_t>(Ly.wave_rows, M - m0);
    const int nch = wave_nchunk(Ly, Mc, dc->info);
    hipError_t e = launch_wave_stage1(Ly, (const uint16_t *)x + m0 * Ly.a, w + m0 * Ly.L, Mc, nch,
                                      Ly.ws, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("stage 1: ") + hipGetErrorString(e));
  }
  return LB_OK;
}

extern "C" lb_status lb_forward_stage2(const lb_layer *L, const float *w, void *y, int64_t M,
                                       void *stream) {
  if (!L) return fail(LB_EINVAL, "lb_forward_stage2: NULL layer");
  const Layer &Ly = L->ly;
  lb_status st = check_io(Ly, w, y, M, "lb_forward_stage2");
  if (st != LB_OK || M == 0) return st;
  DeviceGuard dg(Ly.device);
  for (int64_t m0 = 0; m0 < M; m0 += 63) {
    const int64_t Mc = (M - m0) < 63 ? (M - m0) : 63;
    hipError_t e = launch_wave_stage2(Ly, w + m0 * Ly.L, (uint16_t *)y + m0 * Ly.b, Mc,
                                      ctx_of(L)->info, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("stage 2: ") + hipGetErrorString(e));
  }
  return LB_OK;
}

// ------------------------------------------------------------ bit count
// [LB2 column] Ch. 1: num_bits = P * (s*(a+b+16) + 16*(a+b)), den = a*b.
extern "C" lb_status lb_eff_bits(int64_t a, int64_t b, int64_t s, int residual, uint64_t *num_bits,
                                 uint64_t *den) {
  if (!num_bits || !den) return fail(LB_EINVAL, "lb_eff_bits: NULL output");
  if (a < 1 || b < 1 || s < 0 || (residual != 0 && residual != 1))
    return fail(LB_EINVAL, "lb_eff_bits: bad size");
  const unsigned __int128 P = residual ? 2 : 1;
  const unsigned __int128 ab = (unsigned __int128)a + (unsigned __int128)b;
  const unsigned __int128 n = P * ((unsigned __int128)s * (ab + 16) + 16 * ab);
  const unsigned __int128 d = (unsigned __int128)a * (unsigned __int128)b;
  if (n > UINT64_MAX || d > UINT64_MAX) return fail(LB_EINVAL, "lb_eff_bits: overflow");
  *num_bits = (uint64_t)n;
  *den = (uint64_t)d;
  return LB_OK;
}

extern "C" lb_status lb_rank_for_bpw(int64_t a, int64_t b, uint64_t bpw_num, uint64_t bpw_den,
                                     int residual, int64_t *s) {
  if (!s) return fail(LB_EINVAL, "lb_rank_for_bpw: NULL output");
  if (a < 1 || b < 1 || bpw_den == 0 || (residual != 0 && residual != 1))
    return fail(LB_EINVAL, "lb_rank_for_bpw: bad argument");
  // s = floor((bpw*a*b - 16 P (a+b)) / (P (a+b+16))), all scaled by bpw_den.
  const unsigned __int128 P = residual ? 2 : 1;
  const unsigned __int128 ab = (unsigned __int128)a + (unsigned __int128)b;
  const unsigned __int128 budget = (unsigned __int128)bpw_num * (unsigned __int128)a * (unsigned __int128)b;
  const unsigned __int128 scales = 16 * P * ab * bpw_den;
  if (budget < scales) return fail(LB_EINVAL, "lb_rank_for_bpw: scales alone exceed the budget");
  const unsigned __int128 q = (budget - scales) / (P * (ab + 16) * bpw_den);
  if (q > (unsigned __int128)INT64_MAX) return fail(LB_EINVAL, "lb_rank_for_bpw: overflow");
  *s = (int64_t)q;
  return LB_OK;
}

// --------------------------------------------------------------- stacks
struct lb_stack {
  std::vector<lb_layer *> layers;
  std::vector<int> unit_begin, unit_size;
  float kappa = 1.f;
  int device = 0;
  int mode = 0;
  int64_t cap_M = 0;      // rows the scratch buffers hold
  void *ybuf = nullptr;  // the running unit's layer outputs (cap_M x unit_out_max)
  void *xbuf[2] = {nullptr, nullptr};  // unit input ping-pong (cap_M x max a)
  // wave-path scratch of the stack's layers (chunk partials and latent rows
  // of up to min(cap_M, 63) rows; the layers run one after another), so a
  // small batch takes one launch pair per layer however large the layer
  void *wws = nullptr;
  size_t wws_bytes = 0;
  int64_t unit_out_max = 0;  // max over units of (layers x b)
  // scratch replaced by a larger reservation: kept until the stack is
  // destroyed, since launches captured earlier may still write it
  std::vector<void *> retired;
  int64_t max_width = 0;
  int64_t loop_rows = 2;  // automatic mode: rows run as batch-1 sweeps (see lb_stack_forward)
  PersistPlan *persist = nullptr;
  std::vector<MfmaPlan *> uplan;  // per unit, for M >= 64
  void *mws = nullptr;            // unit-path workspace (largest unit)
  unsigned *mcnt = nullptr;       // unit-path tile counters (kept zero)
  MStackPlan *mstack = nullptr;   // the one-launch M >= 64 stack (null if unsupported)
};

static void stack_free_scratch(lb_stack *S) {
  if (S->ybuf) (void)hipFree(S->ybuf);
  S->ybuf = nullptr;
  for (auto &p : S->xbuf)
    if (p) {
      (void)hipFree(p);
      p = nullptr;
    }
  if (S->wws) (void)hipFree(S->wws);
  S->wws = nullptr;
  S->wws_bytes = 0;
  for (void *p : S->retired)
    if (p) (void)hipFree(p);
  S->retired.clear();
  S->cap_M = 0;
}

// Grow the scratch to at least M rows (at least doubling, so a stack that
// grows step by step keeps few retired buffers).  The current buffers are
// retired, not freed: nothing a forward call used is released before
// lb_stack_destroy.  No device synchronisation.
static lb_status stack_reserve(lb_stack *S, int64_t M) {
  if (M <= S->cap_M) return LB_OK;
  const int64_t cap = std::max<int64_t>(M, 2 * S->cap_M);
  void *yb = nullptr;
  void *xb[2] = {nullptr, nullptr};
  auto undo = [&]() {
    if (yb) (void)hipFree(yb);
    for (void *p : xb)
      if (p) (void)hipFree(p);
    return fail(LB_ENOMEM, "stack scratch hipMalloc");
  };
  if (hipMalloc(&yb, (size_t)cap * S->unit_out_max * 2) != hipSuccess) return undo();
  for (auto &p : xb)
    if (hipMalloc(&p, (size_t)cap * S->max_width * 2) != hipSuccess) return undo();
  const int64_t R = std::min<int64_t>(cap, 63);
  size_t wneed = 0;
  for (const lb_layer *Lr : S->layers) {
    const Layer &Ly = Lr->ly;
    const int nch = wave_nchunk(Ly, 1, ctx_of(Lr)->info);
    wneed = std::max(wneed, (wave_ws_floats(Ly, R, nch) + (size_t)R * Ly.L) * sizeof(float) + 512);
  }
  void *wb = nullptr;
  if (wneed > S->wws_bytes && hipMalloc(&wb, wneed) != hipSuccess) return undo();
  if (S->ybuf) S->retired.push_back(S->ybuf);
  for (void *p : S->xbuf)
    if (p) S->retired.push_back(p);
  S->ybuf = yb;
  S->xbuf[0] = xb[0];
  S->xbuf[1] = xb[1];
  if (wb) {
    if (S->wws) S->retired.push_back(S->wws);
    S->wws = wb;
    S->wws_bytes = wneed;
  }
  S->cap_M = cap;
  return LB_OK;
}

extern "C" lb_status lb_stack_create(lb_layer *const *layers, int n_layers, const int32_t *unit_sizes,
                                     int n_units, float kappa, lb_stack **out) {
  if (!layers || !unit_sizes || !out || n_layers < 1 || n_units < 1)
    return fail(LB_EINVAL, "lb_stack_create: bad argument");
  int total = 0;
  for (int u = 0; u < n_units; ++u) {
    if (unit_sizes[u] < 1 || unit_sizes[u] > 8) return fail(LB_EINVAL, "lb_stack_create: unit size must be 1..8");
    total += unit_sizes[u];
  }
  if (total != n_layers) return fail(LB_EINVAL, "lb_stack_create: unit sizes do not sum to n_layers");
  if (!std::isfinite(kappa)) return fail(LB_EINVAL, "lb_stack_create: kappa not finite");
  lb_stack *S = new (std::nothrow) lb_stack();
  if (!S) return fail(LB_ENOMEM, "lb_stack_create: host allocation");
  S->kappa = kappa;
  S->device = layers[0] ? layers[0]->ly.device : 0;
  int idx = 0;
  for (int u = 0; u < n_units; ++u) {
    S->unit_begin.push_back(idx);
    S->unit_size.push_back(unit_sizes[u]);
    for (int k = 0; k < unit_sizes[u]; ++k, ++idx) {
      lb_layer *Lr = layers[idx];
      if (!Lr || !Lr->ly.ready() || Lr->ly.device != S->device) {
        delete S;
        return fail(LB_EINVAL, "lb_stack_create: layer NULL, not ready, or on another device");
      }
      const lb_layer *first = layers[S->unit_begin[u]];
      if (Lr->ly.a != first->ly.a || Lr->ly.b != first->ly.b) {
        delete S;
        return fail(LB_EINVAL, "lb_stack_create: layers of one unit differ in shape");
      }
      S->layers.push_back(Lr);
      if (Lr->ly.a > S->max_width) S->max_width = Lr->ly.a;
      if (Lr->ly.b > S->max_width) S->max_width = Lr->ly.b;
    }
    if (u > 0 && layers[S->unit_begin[u]]->ly.a != layers[S->unit_begin[u - 1]]->ly.b) {
      delete S;
      return fail(LB_EINVAL, "lb_stack_create: unit input width != previous unit output width");
    }
  }
  for (int u = 0; u < n_units; ++u)
    S->unit_out_max = std::max<int64_t>(S->unit_out_max,
                                        (int64_t)S->unit_size[u] * layers[S->unit_begin[u]]->ly.b);
  DeviceGuard dg(S->device);
  lb_status st = stack_reserve(S, 64);
  if (st != LB_OK) {
    delete S;
    return st;
  }
  {
    size_t wsb = 0, nc = 0;
    for (int u = 0; u < n_units; ++u) {
      std::vector<const Layer *> ls;
      for (int k = 0; k < S->unit_size[u]; ++k) ls.push_back(&S->layers[S->unit_begin[u] + k]->ly);
      MfmaPlan *mp = mfma_plan_build(ls.data(), (int)ls.size());
      S->uplan.push_back(mp);
      if (!mp) {
        lb_stack_destroy(S);
        return fail(LB_EUNSUPPORTED, "lb_stack_create: unit not supported by the MFMA path");
      }
      wsb = std::max(wsb, mfma_unit_ws_bytes(mp));
      nc = std::max(nc, mfma_cnt_entries(mp));
    }
    {
      std::vector<const MfmaPlan *> ups(S->uplan.begin(), S->uplan.end());
      S->mstack = mstack_build(ups, S->kappa, ctx_of(S->layers[0])->info);
      if (S->mstack) {
        wsb = std::max(wsb, mstack_ws_bytes(S->mstack));
        nc = std::max(nc, mstack_cnt_entries(S->mstack));
      }
    }
    hipError_t e = hipMalloc(&S->mws, wsb);
    if (e == hipSuccess) e = hipMalloc(&S->mcnt, nc * sizeof(unsigned));
    if (e == hipSuccess) e = hipMemset(S->mcnt, 0, nc * sizeof(unsigned));
    if (e != hipSuccess) {
      lb_stack_destroy(S);
      return fail(LB_ENOMEM, std::string("lb_stack_create: hipMalloc: ") + hipGetErrorString(e));
    }
  }
  st = persist_build(S->layers, S->unit_begin, S->unit_size, S->kappa, S->device, &S->persist);
  {
    // a batch-1 sweep costs about the same for any matrix size (it is
    // bound by its grid-wide exchanges), the per-layer kernels grow with
    // it: measured crossovers are about 4 rows for 4096 x 11008 matrices
    // and 7 for 8192 x 28672 ones, so the limit follows the mean size
    double elems = 0;
    for (const lb_layer *L : S->layers) elems += (double)L->ly.a * (double)L->ly.b;
    S->loop_rows = elems / (double)S->layers.size() >= (double)(1 << 27) ? 3 : 2;
  }
  if (st != LB_OK && st != LB_EUNSUPPORTED) {
    lb_stack_destroy(S);
    return fail(st, std::string("lb_stack_create: one-launch sweep setup: ") + hipGetErrorString(hipGetLastError()));
  }
  *out = S;
  return LB_OK;
}

extern "C" lb_status lb_stack_timeline(lb_stack *S, void *buf, int64_t capacity, int64_t *needed) {
  if (!S) return fail(LB_EINVAL, "lb_stack_timeline: NULL stack");
  if (!S->persist) return fail(LB_EUNSUPPORTED, "lb_stack_timeline: no persistent plan");
  const int64_t need =
      (int64_t)persist_grid(S->persist) * persist_phases(S->persist) * persist_stamps();
  if (needed) *needed = need;
  if (buf && capacity < need) return fail(LB_EINVAL, "lb_stack_timeline: buffer too small");
  if (((uintptr_t)buf) & 7) return fail(LB_EINVAL, "lb_stack_timeline: buffer not 8-byte aligned");
  persist_set_timeline(S->persist, (uint64_t *)buf);
  return LB_OK;
}

extern "C" lb_status lb_stack_test_wait_failure(lb_stack *S, int enable) {
  if (!S) return fail(LB_EINVAL, "lb_stack_test_wait_failure: NULL stack");
  if (!S->persist)
    return fail(LB_EUNSUPPORTED, "lb_stack_test_wait_failure: the stack has no persistent sweep");
  persist_set_fail_test(S->persist, enable != 0);
  return LB_OK;
}

extern "C" lb_status lb_stack_check(lb_stack *S) {
  if (!S) return fail(LB_EINVAL, "lb_stack_check: NULL stack");
  DeviceGuard dg(S->device);
  LB_HIP(hipDeviceSynchronize());
  if (S->persist) {
    std::string msg;
    lb_status st = persist_check(S->persist, &msg);
    if (st != LB_OK) return fail(st, msg);
  }
  return LB_OK;
}

extern "C" lb_status lb_stack_destroy(lb_stack *S) {
  if (!S) return LB_OK;
  DeviceGuard dg(S->device);
  stack_free_scratch(S);
  persist_free(S->persist);
  mstack_free(S->mstack);
  for (MfmaPlan *mp : S->uplan) mfma_plan_free(mp);
  if (S->mws) (void)hipFree(S->mws);
  if (S->mcnt) (void)hipFree(S->mcnt);
  delete S;
  return LB_OK;
}

extern "C" lb_status lb_stack_test_delay(lb_stack *S, uint32_t seed, uint32_t max_ticks) {
  if (!S) return fail(LB_EINVAL, "lb_stack_test_delay: NULL stack");
  if (max_ticks > 100000u) return fail(LB_EINVAL, "lb_stack_test_delay: max_ticks must be <= 100000 (1 ms)");
  if (!S->persist)
    return fail(LB_EUNSUPPORTED, "lb_stack_test_delay: the stack has no persistent sweep");
  persist_set_delay(S->persist, seed, max_ticks);
  return LB_OK;
}

extern "C" lb_status lb_stack_set_mode(lb_stack *S, int mode) {
  if (!S || mode < 0 || mode > 3) return fail(LB_EINVAL, "lb_stack_set_mode: bad argument");
  if (mode == 3 && !S->mstack)
    return fail(LB_EUNSUPPORTED, "lb_stack_set_mode: no one-launch M >= 64 plan (a width is not a multiple of 8)");
  if (mode == 2 && !S->persist) return fail(LB_EUNSUPPORTED, "lb_stack_set_mode: no persistent plan on this device");
  S->mode = mode;
  return LB_OK;
}

extern "C" lb_status lb_stack_trace_elems(const lb_stack *S, int64_t M, int64_t *elems) {
  if (!S || !elems || M < 0) return fail(LB_EINVAL, "lb_stack_trace_elems: bad argument");
  int64_t n = 0;
  for (auto *Lr : S->layers) n += Lr->ly.b;
  for (size_t u = 0; u < S->unit_begin.size(); ++u) n += S->layers[S->unit_begin[u]]->ly.a;
  *elems = n * M;
  return LB_OK;
}

// Rows that the automatic mode runs as one batch-1 sweep each (no trace).
static int64_t sweep_rows(const lb_stack *S) {
  if (!S->persist) return 0;
  return S->mstack ? std::min<int64_t>(S->loop_rows, 2) : S->loop_rows;
}
// Whether a call of M rows without a trace runs the one-launch stack (in
// the automatic mode and in mode 3): every M past the per-row sweeps.
static bool one_launch_rows(const lb_stack *S, int64_t M) {
  return S->mstack && M >= 2 && M > sweep_rows(S);
}

extern "C" lb_status lb_stack_reserve(lb_stack *S, int64_t M) {
  if (!S || M < 0) return fail(LB_EINVAL, "lb_stack_reserve: bad argument");
  DeviceGuard dg(S->device);
  lb_status st = stack_reserve(S, M);
  if (st != LB_OK || (M < 64 && !one_launch_rows(S, M))) return st;
  for (lb_layer *Lr : S->layers) {
    st = ensure_mfma_copies(Lr, nullptr, true, "lb_stack_reserve");
    if (st != LB_OK) return st;
  }
  return LB_OK;
}

extern "C" lb_status lb_stack_forward(lb_stack *S, const void *x0, void *y, void *trace, int64_t M,
                                      void *stream) {
  if (!S) return fail(LB_EINVAL, "lb_stack_forward: NULL stack");
  if (M < 0) return fail(LB_EINVAL, "lb_stack_forward: M < 0");
  if (M == 0) return LB_OK;
  if (!x0 || !y) return fail(LB_EINVAL, "lb_stack_forward: NULL x0 or y");
  if (((uintptr_t)x0 & 15) || ((uintptr_t)y & 15) || ((uintptr_t)trace & 15))
    return fail(LB_EINVAL, "lb_stack_forward: pointers must be 16-byte aligned");
  DeviceGuard dg(S->device);
  hipStream_t st = (hipStream_t)stream;
  const int U = (int)S->unit_begin.size();
  const int n = (int)S->layers.size();
  // trace offsets
  std::vector<uint16_t *> tY(n, nullptr), tX(U, nullptr);
  if (trace) {
    uint16_t *p = (uint16_t *)trace;
    for (int i = 0; i < n; ++i) { tY[i] = p; p += M * S->layers[i]->ly.b; }
    for (int u = 0; u < U; ++u) { tX[u] = p; p += M * S->layers[S->unit_begin[u]]->ly.a; }
  }
  const bool can_persist = S->persist && M <= persist_max_rows();
  if (S->mode == 2 && !can_persist)
    return fail(LB_EUNSUPPORTED, "lb_stack_forward: persistent mode cannot run this M");
  if (can_persist && S->mode != 1) {
    std::string msg;
    lb_status ps = persist_run(S->persist, (const uint16_t *)x0, (uint16_t *)y, (uint16_t *)trace, M,
                               st, &msg);
    if (ps != LB_OK) return fail(ps, msg);
    return LB_OK;
  }
  // a few rows without a trace: one batch-1 sweep per row (rows are
  // independent, so each row's result is exactly its batch-1 result); it
  // beats the per-layer kernels up to S->loop_rows rows, and the one-launch
  // stack up to 2
  if (S->persist && (S->mode == 0 || S->mode == 3) && !trace && M <= sweep_rows(S)) {
    const int64_t a0 = S->layers[0]->ly.a, bl = S->layers.back()->ly.b;
    for (int64_t m = 0; m < M; ++m) {
      std::string msg;
      lb_status ps = persist_run(S->persist, (const uint16_t *)x0 + m * a0, (uint16_t *)y + m * bl,
                                 nullptr, 1, st, &msg);
      if (ps != LB_OK) return fail(ps, msg);
    }
    return LB_OK;
  }
  lb_status rs = stack_reserve(S, M);
  if (rs != LB_OK) return rs;
  // past the per-row sweeps, without a trace: the one-launch stack (row
  // blocks pipeline through the units; measured faster than the per-layer
  // kernels from 3 rows, where the wave path has become ALU-bound).  In the
  // automatic mode, while the stream is being captured before the layers'
  // matrix-core sign copies or the launch's setup for this M exist, the
  // per-layer kernels below run instead (for M >= 64 the unit launches:
  // the same tiles in the same order)
  bool one_launch = (S->mode == 0 || S->mode == 3) && !trace && one_launch_rows(S, M);
  if (one_launch && S->mode == 0) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return fail(LB_EHIP, "lb_stack_forward: hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone) {
      bool copies = true;
      for (const lb_layer *Lr : S->layers) copies = copies && Lr->ly.sv1m && Lr->ly.su2m;
      if (!copies ||
          !mstack_ready(S->mstack, M, S->mws, S->mcnt, (uint16_t *)S->xbuf[0], (uint16_t *)S->xbuf[1]))
        one_launch = false;
    }
  }
  if (M >= 64 || one_launch) {
    for (lb_layer *Lr : S->layers) {
      lb_status es = ensure_mfma_copies(Lr, st, true, "lb_stack_forward");
      if (es != LB_OK) return es;
    }
  }
  if (one_launch) {
    std::string msg;
    DevCtx *dc = ctx_of(S->layers[0]);
    lb_status ms = mstack_run(S->mstack, (const uint16_t *)x0, (uint16_t *)y, M, S->mws, S->mcnt,
                              (uint16_t *)S->xbuf[0], (uint16_t *)S->xbuf[1], dc->zero, dc->info, st, &msg);
    if (ms != LB_OK) return fail(ms, "lb_stack_forward: " + msg);
    return LB_OK;
  }
  if (M >= 64 && S->mode != 1) {
    // one stage-1 and one stage-2 launch per unit; stage 2 also combines
    const uint16_t *cur = (const uint16_t *)x0;
    if (trace)
      LB_HIP(hipMemcpyAsync(tX[0], x0, (size_t)M * S->layers[0]->ly.a * 2, hipMemcpyDeviceToDevice, st));
    for (int u = 0; u < U; ++u) {
      const int b0 = S->unit_begin[u], nu = S->unit_size[u];
      uint16_t *next;
      if (u == U - 1)
        next = (uint16_t *)y;
      else if (trace)
        next = tX[u + 1];
      else
        next = (uint16_t *)S->xbuf[u & 1];
      hipError_t e = launch_mfma_unit(S->uplan[u], cur, M, trace ? &tY[b0] : nullptr, next,
                                      S->kappa / std::sqrt((float)nu), false, S->mws, S->mcnt,
                                      ctx_of(S->layers[b0])->zero, ctx_of(S->layers[b0])->info, st);
      if (e != hipSuccess) return fail(LB_EHIP, std::string("mfma unit: ") + hipGetErrorString(e));
      cur = next;
    }
    return LB_OK;
  }
  const uint16_t *cur = (const uint16_t *)x0;
  if (trace) {
    LB_HIP(hipMemcpyAsync(tX[0], x0, (size_t)M * S->layers[0]->ly.a * 2, hipMemcpyDeviceToDevice, st));
  }
  for (int u = 0; u < U; ++u) {
    const int b0 = S->unit_begin[u], nu = S->unit_size[u];
    uint16_t *next;
    if (u == U - 1)
      next = (uint16_t *)y;
    else
      next = trace ? tX[u + 1] : (uint16_t *)S->xbuf[u & 1];
    const float c = S->kappa / std::sqrt((float)nu);
    std::vector<const uint16_t *> outs;
    bool combined = false;
    for (int k = 0; k < nu; ++k) {
      lb_layer *Lr = S->layers[b0 + k];
      uint16_t *o = trace ? tY[b0 + k] : (uint16_t *)S->ybuf + (size_t)k * M * Lr->ly.b;
      lb_status fs;
      if (M > 1 && M < 64) {
        // the wave path with the stack's scratch: all rows in one launch
        // pair; up to 16 rows the unit's last layer also forms the combine
        // in its second product when its kernel can (one launch fewer; with
        // more rows the separate combine kernel was faster)
        std::string msg;
        const bool fuse = k == nu - 1 && M <= 16 && wave_stage2_combines(Lr->ly);
        const CombineReq cr{outs.data(), k, c, next};
        fs = forward_ws(Lr, cur, o, M, st, S->wws, S->wws_bytes, Lr->ly.cnt, 1, &msg, fuse ? &cr : nullptr);
        if (fs != LB_OK) return fail(fs, "lb_stack_forward: " + msg);
        combined = fuse;
      } else {
        fs = forward_impl(Lr, cur, o, M, st);
        if (fs != LB_OK) return fs;
      }
      outs.push_back(o);
    }
    if (!combined) {
      const int64_t elems = M * S->layers[b0]->ly.b;
      hipError_t e = launch_combine(outs.data(), nu, c, next, elems, st);
      if (e != hipSuccess) return fail(LB_EHIP, std::string("combine: ") + hipGetErrorString(e));
    }
    cur = next;
  }
  return LB_OK;
}

// ---------------------------------------------------------- diagnostics
extern "C" const char *lb_status_str(lb_status st) {
  switch (st) {
    case LB_OK: return "LB_OK";
    case LB_EINVAL: return "LB_EINVAL";
    case LB_ENOMEM: return "LB_ENOMEM";
    case LB_EHIP: return "LB_EHIP";
    case LB_ENOTREADY: return "LB_ENOTREADY";
    case LB_EUNSUPPORTED: return "LB_EUNSUPPORTED";
    case LB_ETIMEOUT: return "LB_ETIMEOUT";
  }
  return "LB_UNKNOWN";
}

extern "C" const char *lb_last_error(void) { return g_last_error.c_str(); }

extern "C" int lb_version(void) { return 100; }
