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
struct DevCtx {
  DeviceInfo info;
  void *ws = nullptr;  // shared forward workspace of this device
  size_t ws_bytes = 0;
  unsigned *cnt = nullptr;  // split-K tile counters of the MFMA path (kept zero)
  void *zero = nullptr;     // 256 zero bytes (copy source for padding)
};
constexpr size_t kDevCounters = 4096;
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
    e = hipMalloc(&c.cnt, kDevCounters * sizeof(unsigned) + 256);
    if (e == hipSuccess) e = hipMemset(c.cnt, 0, kDevCounters * sizeof(unsigned) + 256);
    c.zero = c.cnt + kDevCounters;
    if (e != hipSuccess) return fail(LB_ENOMEM, std::string("counter hipMalloc: ") + hipGetErrorString(e));
    it = g_dev.emplace(device, c).first;
  }
  *out = &it->second;
  return LB_OK;
}

// Grow the device workspace to at least `need` bytes (called at create
// time only, never from a forward call).
lb_status ensure_ws(DevCtx *c, size_t need) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (c->ws_bytes >= need) return LB_OK;
  if (c->ws) {
    (void)hipDeviceSynchronize();
    (void)hipFree(c->ws);
    c->ws = nullptr;
    c->ws_bytes = 0;
  }
  void *p = nullptr;
  hipError_t e = hipMalloc(&p, need);
  if (e != hipSuccess) return fail(LB_ENOMEM, std::string("workspace hipMalloc: ") + hipGetErrorString(e));
  c->ws = p;
  c->ws_bytes = need;
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

// Word in the matrix-core bit order (see lb_internal.h): bits inverted and
// permuted so that (w << (4 g + j)) & 0x80008000 holds the sign flips of
// elements 8 g + 2 j and 8 g + 2 j + 1.
// The permutation is bytewise: byte g of w fills its own bit positions, so
// a table per byte position gives the word in four lookups.
inline uint32_t mfma_bit_order_slow(uint32_t w) {
  uint32_t o = 0;
  for (int g = 0; g < 4; ++g)
    for (int e = 0; e < 8; ++e) {
      const uint32_t flip = ((w >> (8 * g + e)) & 1u) ^ 1u;
      const int pos = (e & 1) ? 31 - (e >> 1) - 4 * g : 15 - (e >> 1) - 4 * g;
      o |= flip << pos;
    }
  return o;
}

struct MfmaOrderTable {
  uint32_t t[4][256];
  MfmaOrderTable() {
    for (int g = 0; g < 4; ++g)
      for (uint32_t v = 0; v < 256; ++v)
        // the other bytes set to all ones contribute no flips
        t[g][v] = mfma_bit_order_slow((0xffffffffu & ~(0xffu << (8 * g))) | (v << (8 * g)));
  }
};
const MfmaOrderTable g_mfma_order;

inline uint32_t mfma_bit_order(uint32_t w) {
  return g_mfma_order.t[0][w & 0xff] | g_mfma_order.t[1][(w >> 8) & 0xff] |
         g_mfma_order.t[2][(w >> 16) & 0xff] | g_mfma_order.t[3][w >> 24];
}

inline uint32_t tail_mask(int64_t s, int64_t q) {
  const int64_t n = s - 32 * q;
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// In-place transpose of a 32 x 32 bit matrix: bit c of m[r] <-> bit r of m[c].
void transpose32(uint32_t m[32]) {
  uint32_t mask = 0x0000ffffu;
  for (int j = 16; j != 0; j >>= 1, mask ^= (mask << j)) {
    for (int k = 0; k < 32; k = ((k | j) + 1) & ~j) {
      const uint32_t t = ((m[k] >> j) ^ m[k | j]) & mask;
      m[k] ^= t << j;
      m[k | j] ^= t;
    }
  }
}

}  // namespace

static inline DevCtx *ctx_of(const lb_layer *L) { return static_cast<DevCtx *>(L->ctx); }

// --------------------------------------------------------- workspace need
static size_t layer_ws_need(const Layer &Ly, const MfmaPlan *mp, const DeviceInfo &dev) {
  size_t need = 0;
  for (int64_t M = 1; M < 64; ++M) {
    const int nch = wave_nchunk(Ly, M, dev);
    const size_t b = (wave_ws_floats(Ly, M, nch) + (size_t)M * Ly.L) * sizeof(float) + 512;
    if (b > need) need = b;
  }
  const size_t mf = mfma_unit_ws_bytes(mp);
  if (mf > need) need = mf;
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
  Ly.L = Ly.P * s; Ly.R1 = (a + 31) / 32; Ly.Wk = (s + 31) / 32;
  Ly.T16a = (a + 15) / 16; Ly.T16b = (b + 15) / 16;
  Ly.a16 = Ly.T16a * 16; Ly.b16 = Ly.T16b * 16; Ly.s8 = (s + 7) / 8 * 8;
  Ly.Lp = (Ly.L + 7) / 8 * 8;
  L->ctx = dc;
  struct Alloc { void **p; size_t n; };
  Alloc allocs[] = {
      {(void **)&Ly.sv1, (size_t)Ly.R1 * Ly.L * 4},
      {(void **)&Ly.su2, (size_t)Ly.P * Ly.Wk * Ly.b16 * 4},
      {(void **)&Ly.h, (size_t)Ly.P * Ly.b16 * 2},
      {(void **)&Ly.g, (size_t)Ly.P * Ly.a16 * 2},
      {(void **)&Ly.l, (size_t)Ly.P * Ly.s8 * 2},
      {(void **)&Ly.sv16, (size_t)Ly.T16a * Ly.Lp * 2},
      {(void **)&Ly.su2t, (size_t)Ly.T16b * Ly.P * Ly.Wk * 16 * 4},
      {(void **)&Ly.ht, (size_t)Ly.T16b * Ly.P * 16 * 2},
      {(void **)&Ly.gt, (size_t)Ly.T16a * Ly.P * 16 * 2},
      {(void **)&Ly.sv1m, (size_t)Ly.R1 * Ly.L * 4},
      {(void **)&Ly.su2m, (size_t)Ly.P * Ly.Wk * Ly.b16 * 4}};
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
  if (!L->mplan || mfma_cnt_entries(L->mplan) > kDevCounters) {
    lb_destroy(L);
    return fail(LB_EUNSUPPORTED, "lb_create: shape not supported by the MFMA path");
  }
  st = ensure_ws(dc, layer_ws_need(Ly, L->mplan, dc->info));
  if (st != LB_OK) {
    lb_destroy(L);
    return st;
  }
  *out = L;
  return LB_OK;
}

extern "C" lb_status lb_destroy(lb_layer *L) {
  if (!L) return LB_OK;
  DeviceGuard g(L->ly.device);
  Layer &Ly = L->ly;
  void *ps[] = {Ly.sv1, Ly.su2, Ly.h, Ly.g, Ly.l, Ly.sv16, Ly.su2t, Ly.ht, Ly.gt, Ly.sv1m, Ly.su2m};
  for (void *p : ps)
    if (p) (void)hipFree(p);
  mfma_plan_free(L->mplan);
  delete L;
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

// Re-lay host canonical words of one path out for the device (the caller
// has checked the arguments and made the layer's device current).
static lb_status pack_signs_impl(Layer &Ly, int path, const uint32_t *su, const uint32_t *sv) {
  const int64_t a = Ly.a, b = Ly.b, s = Ly.s, Wk = Ly.Wk, Lc = Ly.L;
  // S_U: su2[(p*Wk + q)*b16 + j] = su[j*Wk + q] (padding masked, rows >= b zero)
  const int64_t b16 = Ly.b16;
  std::vector<uint32_t> u2;
  std::vector<uint32_t> v1;
  std::vector<uint16_t> v16;
  try {
    u2.assign((size_t)Wk * b16, 0u);
    v1.resize((size_t)Ly.R1 * Lc);
    v16.assign((size_t)Ly.T16a * Ly.Lp, 0);
  } catch (...) {
    return fail(LB_ENOMEM, "lb_pack_signs: host allocation");
  }
  for (int64_t q = 0; q < Wk; ++q) {
    const uint32_t msk = tail_mask(s, q);
    for (int64_t j = 0; j < b; ++j) u2[(size_t)q * b16 + j] = su[j * Wk + q] & msk;
  }
  LB_HIP(hipMemcpy(Ly.su2 + (size_t)path * Wk * b16, u2.data(), u2.size() * 4, hipMemcpyHostToDevice));
  {
    std::vector<uint32_t> u2m(u2.size());
    for (size_t i = 0; i < u2.size(); ++i) u2m[i] = mfma_bit_order(u2[i]);
    LB_HIP(hipMemcpy(Ly.su2m + (size_t)path * Wk * b16, u2m.data(), u2m.size() * 4, hipMemcpyHostToDevice));
  }
  {
    // tile-major: for tile tau, this path's Wk x 16 words are one 64*Wk-byte
    // run.  The paths interleave per tile, so the whole buffer is rewritten
    // in one contiguous copy (after reading back the other path's runs).
    const size_t n = (size_t)Ly.T16b * Ly.P * Wk * 16;
    std::vector<uint32_t> u2t(n, 0u);
    if (Ly.P > 1) LB_HIP(hipMemcpy(u2t.data(), Ly.su2t, n * 4, hipMemcpyDeviceToHost));
    for (int64_t tau = 0; tau < Ly.T16b; ++tau)
      for (int64_t q = 0; q < Wk; ++q)
        for (int r = 0; r < 16; ++r)
          u2t[(((size_t)tau * Ly.P + path) * Wk + q) * 16 + r] = u2[(size_t)q * b16 + 16 * tau + r];
    LB_HIP(hipMemcpy(Ly.su2t, u2t.data(), n * 4, hipMemcpyHostToDevice));
  }
  // S_V: 32 x 32 bit transposes.  Block (row group r, word q) -> columns
  // p*s + 32q + kk of row group r.
  {
    // read back the other path's columns so this call only replaces its own
    LB_HIP(hipMemcpy(v1.data(), Ly.sv1, v1.size() * 4, hipMemcpyDeviceToHost));
    uint32_t blk[32];
    for (int64_t r = 0; r < Ly.R1; ++r) {
      for (int64_t q = 0; q < Wk; ++q) {
        const uint32_t msk = tail_mask(s, q);
        for (int e = 0; e < 32; ++e) {
          const int64_t i = r * 32 + e;
          blk[e] = i < a ? (sv[i * Wk + q] & msk) : 0u;
        }
        transpose32(blk);  // blk[kk] bit e = S_V[32r + e, 32q + kk]
        const int64_t nk = (s - 32 * q) < 32 ? (s - 32 * q) : 32;
        for (int64_t kk = 0; kk < nk; ++kk) v1[(size_t)r * Lc + path * s + 32 * q + kk] = blk[kk];
      }
    }
    LB_HIP(hipMemcpy(Ly.sv1, v1.data(), v1.size() * 4, hipMemcpyHostToDevice));
    {
      std::vector<uint32_t> v1m(v1.size());
      for (size_t i = 0; i < v1.size(); ++i) v1m[i] = mfma_bit_order(v1[i]);
      LB_HIP(hipMemcpy(Ly.sv1m, v1m.data(), v1m.size() * 4, hipMemcpyHostToDevice));
    }
    // sv16[gi*Lp + c]: the 16-row halves of the sv1 words
    for (int64_t gi = 0; gi < Ly.T16a; ++gi)
      for (int64_t c = 0; c < Lc; ++c)
        v16[(size_t)gi * Ly.Lp + c] = (uint16_t)(v1[(size_t)(gi / 2) * Lc + c] >> (16 * (gi % 2)));
    LB_HIP(hipMemcpy(Ly.sv16, v16.data(), v16.size() * 2, hipMemcpyHostToDevice));
  }
  Ly.signs_set[path] = true;
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
  const int64_t a = Ly.a, b = Ly.b, s = Ly.s, Wk = Ly.Wk, Lc = Ly.L;
  std::vector<uint32_t> u2((size_t)Wk * Ly.b16), v1((size_t)Ly.R1 * Lc);
  LB_HIP(hipMemcpy(u2.data(), Ly.su2 + (size_t)path * Wk * Ly.b16, u2.size() * 4, hipMemcpyDeviceToHost));
  LB_HIP(hipMemcpy(v1.data(), Ly.sv1, v1.size() * 4, hipMemcpyDeviceToHost));
  for (int64_t j = 0; j < b; ++j)
    for (int64_t q = 0; q < Wk; ++q) su[j * Wk + q] = u2[(size_t)q * Ly.b16 + j];
  uint32_t blk[32];
  for (int64_t r = 0; r < Ly.R1; ++r) {
    for (int64_t q = 0; q < Wk; ++q) {
      const int64_t nk = (s - 32 * q) < 32 ? (s - 32 * q) : 32;
      for (int kk = 0; kk < 32; ++kk) blk[kk] = kk < nk ? v1[(size_t)r * Lc + path * s + 32 * q + kk] : 0u;
      transpose32(blk);  // blk[e] bit kk = S_V[32r + e, 32q + kk]
      for (int e = 0; e < 32; ++e) {
        const int64_t i = r * 32 + e;
        if (i < a) sv[i * Wk + q] = blk[e];
      }
    }
  }
  return LB_OK;
}

static lb_status set_scales_impl(Layer &Ly, int path, const uint16_t *h, const uint16_t *g,
                                 const uint16_t *l) {
  LB_HIP(hipMemcpy(Ly.h + (size_t)path * Ly.b16, h, Ly.b * 2, hipMemcpyHostToDevice));
  LB_HIP(hipMemcpy(Ly.g + (size_t)path * Ly.a16, g, Ly.a * 2, hipMemcpyHostToDevice));
  LB_HIP(hipMemcpy(Ly.l + (size_t)path * Ly.s8, l, Ly.s * 2, hipMemcpyHostToDevice));
  {
    // tile-major copies of h and g: 16 values per (tile, path), zero padded;
    // the paths interleave per tile, so each buffer is rewritten whole
    const size_t nh = (size_t)Ly.T16b * Ly.P * 16, ng = (size_t)Ly.T16a * Ly.P * 16;
    std::vector<uint16_t> hb(nh, 0), gb(ng, 0);
    if (Ly.P > 1) {
      LB_HIP(hipMemcpy(hb.data(), Ly.ht, nh * 2, hipMemcpyDeviceToHost));
      LB_HIP(hipMemcpy(gb.data(), Ly.gt, ng * 2, hipMemcpyDeviceToHost));
    }
    for (int64_t j = 0; j < Ly.b16; ++j)
      hb[((size_t)(j >> 4) * Ly.P + path) * 16 + (j & 15)] = j < Ly.b ? h[j] : (uint16_t)0;
    for (int64_t i = 0; i < Ly.a16; ++i)
      gb[((size_t)(i >> 4) * Ly.P + path) * 16 + (i & 15)] = i < Ly.a ? g[i] : (uint16_t)0;
    LB_HIP(hipMemcpy(Ly.ht, hb.data(), nh * 2, hipMemcpyHostToDevice));
    LB_HIP(hipMemcpy(Ly.gt, gb.data(), ng * 2, hipMemcpyHostToDevice));
  }
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

static lb_status forward_impl(const lb_layer *L, const uint16_t *x, uint16_t *y, int64_t M,
                              hipStream_t st) {
  const Layer &Ly = L->ly;
  DevCtx *dc = ctx_of(L);
  if (M < 64) {
    const int nch = wave_nchunk(Ly, M, dc->info);
    float *part = reinterpret_cast<float *>(dc->ws);
    float *w = part + wave_ws_floats(Ly, M, nch);
    hipError_t e = launch_wave_stage1(Ly, x, w, M, nch, part, st);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("wave stage 1: ") + hipGetErrorString(e));
    e = launch_wave_stage2(Ly, w, y, M, st);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("wave stage 2: ") + hipGetErrorString(e));
    return LB_OK;
  }
  uint16_t *ys[1] = {y};
  hipError_t e = launch_mfma_unit(L->mplan, x, M, ys, nullptr, 1.f, true, dc->ws, dc->cnt, dc->zero,
                                 dc->info, st);
  if (e != hipSuccess) return fail(LB_EHIP, std::string("mfma path: ") + hipGetErrorString(e));
  return LB_OK;
}

extern "C" lb_status lb_forward(const lb_layer *L, const void *x, void *y, int64_t M, void *stream) {
  if (!L) return fail(LB_EINVAL, "lb_forward: NULL layer");
  const Layer &Ly = L->ly;
  lb_status st = check_io(Ly, x, y, M, "lb_forward");
  if (st != LB_OK || M == 0) return st;
  if (overlaps(x, (size_t)M * Ly.a * 2, y, (size_t)M * Ly.b * 2))
    return fail(LB_EINVAL, "lb_forward: x and y overlap");
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
  // Rows in blocks of 63 so the partial buffer stays within the workspace.
  for (int64_t m0 = 0; m0 < M; m0 += 63) {
    const int64_t Mc = (M - m0) < 63 ? (M - m0) : 63;
    const int nch = wave_nchunk(Ly, Mc, dc->info);
    hipError_t e = launch_wave_stage1(Ly, (const uint16_t *)x + m0 * Ly.a, w + m0 * Ly.L, Mc, nch,
                                      (float *)dc->ws, (hipStream_t)stream);
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
                                      (hipStream_t)stream);
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
  std::vector<void *> ybuf;  // per layer output scratch (cap_M x b)
  void *xbuf[2] = {nullptr, nullptr};  // unit input ping-pong (cap_M x max a)
  int64_t max_width = 0;
  int64_t loop_rows = 4;  // automatic mode: rows run as batch-1 sweeps (see lb_stack_forward)
  PersistPlan *persist = nullptr;
  std::vector<MfmaPlan *> uplan;  // per unit, for M >= 64
  void *mws = nullptr;            // unit-path workspace (largest unit)
  unsigned *mcnt = nullptr;       // unit-path tile counters (kept zero)
};

static void stack_free_scratch(lb_stack *S) {
  for (void *p : S->ybuf)
    if (p) (void)hipFree(p);
  S->ybuf.clear();
  for (auto &p : S->xbuf)
    if (p) {
      (void)hipFree(p);
      p = nullptr;
    }
  S->cap_M = 0;
}

static lb_status stack_reserve(lb_stack *S, int64_t M) {
  if (M <= S->cap_M) return LB_OK;
  (void)hipDeviceSynchronize();
  stack_free_scratch(S);
  S->ybuf.assign(S->layers.size(), nullptr);
  for (size_t i = 0; i < S->layers.size(); ++i) {
    hipError_t e = hipMalloc(&S->ybuf[i], (size_t)M * S->layers[i]->ly.b * 2);
    if (e != hipSuccess) {
      stack_free_scratch(S);
      return fail(LB_ENOMEM, "stack scratch hipMalloc");
    }
  }
  for (auto &p : S->xbuf) {
    hipError_t e = hipMalloc(&p, (size_t)M * S->max_width * 2);
    if (e != hipSuccess) {
      stack_free_scratch(S);
      return fail(LB_ENOMEM, "stack scratch hipMalloc");
    }
  }
  S->cap_M = M;
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
    S->loop_rows = elems / (double)S->layers.size() >= (double)(1 << 27) ? 7 : 4;
  }
  if (st != LB_OK && st != LB_EUNSUPPORTED) {
    stack_free_scratch(S);
    delete S;
    return st;
  }
  *out = S;
  return LB_OK;
}

extern "C" lb_status lb_stack_timeline(lb_stack *S, void *buf, int64_t capacity, int64_t *needed) {
  if (!S) return fail(LB_EINVAL, "lb_stack_timeline: NULL stack");
  if (!S->persist) return fail(LB_EUNSUPPORTED, "lb_stack_timeline: no persistent plan");
  const int64_t need = (int64_t)persist_grid(S->persist) * persist_phases(S->persist) * 4;
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
  for (MfmaPlan *mp : S->uplan) mfma_plan_free(mp);
  if (S->mws) (void)hipFree(S->mws);
  if (S->mcnt) (void)hipFree(S->mcnt);
  delete S;
  return LB_OK;
}

extern "C" lb_status lb_stack_set_mode(lb_stack *S, int mode) {
  if (!S || mode < 0 || mode > 2) return fail(LB_EINVAL, "lb_stack_set_mode: bad argument");
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

extern "C" lb_status lb_stack_reserve(lb_stack *S, int64_t M) {
  if (!S || M < 0) return fail(LB_EINVAL, "lb_stack_reserve: bad argument");
  DeviceGuard dg(S->device);
  return stack_reserve(S, M);
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
  // a few rows without a trace: one batch-1 sweep per row beats the
  // per-layer kernels up to S->loop_rows rows (rows are independent, so
  // each row's result is exactly its batch-1 result)
  if (S->persist && S->mode == 0 && !trace && M <= S->loop_rows) {
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
    std::vector<const uint16_t *> outs;
    for (int k = 0; k < nu; ++k) {
      lb_layer *Lr = S->layers[b0 + k];
      uint16_t *o = trace ? tY[b0 + k] : (uint16_t *)S->ybuf[b0 + k];
      lb_status fs = forward_impl(Lr, cur, o, M, st);
      if (fs != LB_OK) return fs;
      outs.push_back(o);
    }
    uint16_t *next;
    if (u == U - 1)
      next = (uint16_t *)y;
    else
      next = trace ? tX[u + 1] : (uint16_t *)S->xbuf[u & 1];
    const int64_t elems = M * S->layers[b0]->ly.b;
    hipError_t e = launch_combine(outs.data(), nu, S->kappa / std::sqrt((float)nu), next, elems, st);
    if (e != hipSuccess) return fail(LB_EHIP, std::string("combine: ") + hipGetErrorString(e));
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
