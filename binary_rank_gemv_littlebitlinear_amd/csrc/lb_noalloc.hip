// lb_forward_noalloc: the layer forward with its scratch in a fixed device
// array, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is the file-scope array `scratch` below (kScratchBytes per
// device, held until the process ends): the first kCntBytes hold the
// matrix-core path's split-K tile counters, the rest the forward's
// workspace (wave-path chunk partials and latent rows, or the matrix-core
// latent and split partials).  In host code `scratch` names a host-side
// stand-in, not device memory: its device address on each device comes
// from hipGetSymbolAddress, taken once per device with that device current
// and kept in g_scratch; only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>

#include "lb_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // per device
constexpr size_t kCntBytes = 16384;                  // 4096 tile counters

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
std::map<int, unsigned char *> g_scratch;  // device -> device address of `scratch`

__global__ void k_zero_u32(unsigned *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of `scratch` on `device` (current), set up on first
// use: the tile counters are cleared there (with a kernel on `st`, so this
// also works under capture); every later launch leaves them zero.
lb_status scratch_on(int device, hipStream_t st, unsigned char **out, std::string *msg) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(device);
  if (it != g_scratch.end()) {
    *out = it->second;
    return LB_OK;
  }
  unsigned char *ptr = nullptr;
  hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    *msg = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
    return LB_EHIP;
  }
  const int n = (int)(kCntBytes / sizeof(unsigned));
  hipLaunchKernelGGL(k_zero_u32, dim3((n + 255) / 256), dim3(256), 0, st,
                     reinterpret_cast<unsigned *>(ptr), n);
  e = hipGetLastError();
  if (e != hipSuccess) {
    *msg = std::string("clearing the scratch counters: ") + hipGetErrorString(e);
    return LB_EHIP;
  }
  g_scratch.emplace(device, ptr);
  *out = ptr;
  return LB_OK;
}

}  // namespace

extern "C" lb_status lb_forward_noalloc(const lb_layer *L, const void *x, void *y, int64_t M,
                                       void *stream) {
  lb_status st = lbi::forward_checks(L, x, y, M, "lb_forward_noalloc");
  if (st != LB_OK || M == 0) return st;
  const int dev = L->ly.device;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess)
    return lbi::set_error(LB_EHIP, "lb_forward_noalloc: hipGetDevice failed");
  if (prev != dev && hipSetDevice(dev) != hipSuccess)
    return lbi::set_error(LB_EHIP, "lb_forward_noalloc: hipSetDevice failed");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  unsigned char *base = nullptr;
  std::string msg;
  st = scratch_on(dev, hs, &base, &msg);
  if (st == LB_OK)
    st = lbi::forward_ws(L, static_cast<const uint16_t *>(x), static_cast<uint16_t *>(y), M, hs,
                         base + kCntBytes, kScratchBytes - kCntBytes, reinterpret_cast<unsigned *>(base),
                         kCntBytes / sizeof(unsigned), &msg);
  if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
  if (st != LB_OK) return lbi::set_error(st, "lb_forward_noalloc: " + msg);
  return LB_OK;
}
