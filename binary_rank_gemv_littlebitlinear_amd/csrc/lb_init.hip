// Initialisation of one path from real factors on the device ([LB news]
// Sec. 2, Dual-SVID): the signs of U (b x s) and V (a x s) become the
// binary factors, and the top singular pair of |U| and of |V| gives the
// scales (h and l_u from |U|, g and l_v from |V|, l = l_u * l_v, each
// singular value split evenly between its two vectors).
//
// Kernels
//   k_sign_words   one wave per factor row; each lane tests one element
//                  (f >= 0 counts as +1, so -0 and 0 are +1), a 64-lane
//                  ballot packs 64 columns, lanes 0 and 1 store the two
//                  canonical words.  Coalesced 256-byte reads per wave.
//   power iteration on A = |F| (n x s, fp32 in, fp64 arithmetic), started
//   from the all-ones direction, whose overlap with the nonnegative top
//   right singular vector of a nonnegative matrix is positive:
//     k_pow_fused   (s <= 1024) about 1024 workgroups of consecutive rows; a
//                   wave per row, lanes along k: x_r = sum_k A[r,k] v_k by a
//                   fixed-order shuffle tree, and with the same loaded values
//                   each lane adds A[r,k] x_r into its register share of A^T x;
//                   the block's share goes to part[block][k].  A is read once.
//     k_pow_block   (any s) 64 rows per workgroup, the same x_r, then the
//                   block's share of A^T x by a thread per column over the
//                   block's rows (a second, cache-served read).  Also gives
//                   x = A v for the final step.
//     k_pow_reduce  w_k = sum over blocks of part[.][k], 128 fixed ranges per
//                   column combined by a fixed pairwise tree.
//     k_pow_normalize  one workgroup: v = w / ||w||, and max |v_new - v_old|
//                   for the host's convergence test.
//   Every sum has a fixed order, so a call is deterministic.  After the
//   last step, x = A v and sigma = ||x||; then u sqrt(sigma) = x / sqrt(sigma)
//   and v sqrt(sigma) are the evenly split pair.
//   k_init_scales  h, g, l rounded once from fp64 to fp16 (nearest even).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "lb_internal.h"

namespace lbi {
namespace {

constexpr int kRowsPerBlock = 64;
constexpr int kCheckEvery = 8;

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// fp64 -> IEEE binary16 bits, round to nearest, ties to even, in one step
// (no intermediate fp32, which could round twice).  Overflow gives inf.
__device__ inline uint16_t f16_bits_rne(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int ex = (int)((u >> 52) & 0x7ff);
  const uint64_t man = u & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7ff) return sign | (man ? 0x7e00 : 0x7c00);
  if (ex == 0) return sign;  // fp64 subnormals are far below fp16's smallest step
  const int e = ex - 1023;
  if (e > 15) return sign | 0x7c00;
  const uint64_t m = man | (1ull << 52);
  // fp16 normals keep 10 fraction bits; below 2^-14 the step is 2^-24
  const int shift = e >= -14 ? 42 : 42 + (-14 - e);
  if (shift > 63) return sign;
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  // a carry out of the fraction moves into the exponent field by itself
  uint32_t bits = e >= -14 ? ((uint32_t)(e + 15) << 10) + (uint32_t)q - 1024u : (uint32_t)q;
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | (uint16_t)bits;
}

template <typename T>
__global__ void __launch_bounds__(256) k_sign_words(const T *__restrict__ F, int64_t rows,
                                                    int64_t s, int64_t Wk,
                                                    uint32_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T *row = F + (size_t)r * s;
  uint32_t *o = out + (size_t)r * Wk;
  for (int64_t c0 = 0; c0 < s; c0 += 64) {
    const int64_t k = c0 + lane;
    const bool bit = k < s && row[k < s ? k : 0] >= (T)0;
    const uint64_t m = __ballot(bit);
    const int64_t q = (c0 >> 5) + lane;
    if (lane < 2 && q < Wk) o[q] = (uint32_t)(m >> (32 * lane));
  }
}

template <typename T>
__global__ void __launch_bounds__(256) k_pow_block(const T *__restrict__ F, int64_t n,
                                                   int64_t s, const double *__restrict__ v,
                                                   double *__restrict__ part,
                                                   double *__restrict__ xout) {
  __shared__ double xs[kRowsPerBlock];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsPerBlock;
  const int rows = (int)((n - r0) < kRowsPerBlock ? (n - r0) : kRowsPerBlock);
  for (int rr = wave; rr < rows; rr += 4) {
    const T *row = F + (size_t)(r0 + rr) * s;
    double acc = 0.0;
    for (int64_t k = lane; k < s; k += 64) acc += fabs((double)row[k]) * v[k];
    acc = wave_sum(acc);
    if (lane == 0) {
      xs[rr] = acc;
      if (xout) xout[r0 + rr] = acc;
    }
  }
  if (!part) return;
  __syncthreads();
  const T *blk = F + (size_t)r0 * s;
  for (int64_t k = t; k < s; k += 256) {
    double acc = 0.0;
    for (int rr = 0; rr < rows; ++rr) acc += fabs((double)blk[(size_t)rr * s + k]) * xs[rr];
    part[(size_t)blockIdx.x * s + k] = acc;
  }
}

// Register-resident variant for s <= 64 KM: a lane keeps its KM columns of
// v and of the block's A^T x share in registers, so every element of A is
// loaded once: x_r = wave sum of |A[r, k]| v_k, then acc_k += |A[r, k]| x_r
// with the same loaded values.  The four waves' shares are added in wave
// order through LDS.
template <typename T, int KM>
__global__ void __launch_bounds__(256) k_pow_fused(const T *__restrict__ F, int64_t n, int s,
                                                   int rpb, const double *__restrict__ v,
                                                   double *__restrict__ part) {
  __shared__ double sh[3][KM * 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * rpb;
  const int rows = (int)((n - r0) < rpb ? (n - r0) : rpb);
  double vr[KM], acc[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int k = lane + 64 * j;
    vr[j] = k < s ? v[k] : 0.0;
    acc[j] = 0.0;
  }
  for (int rr = wave; rr < rows; rr += 4) {
    const T *row = F + (size_t)(r0 + rr) * s;
    double av[KM];
    double dot = 0.0;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int k = lane + 64 * j;
      av[j] = k < s ? fabs((double)row[k < s ? k : 0]) : 0.0;
      dot += av[j] * vr[j];
    }
    const double x = wave_sum(dot);
#pragma unroll
    for (int j = 0; j < KM; ++j) acc[j] += av[j] * x;
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) sh[wave - 1][lane + 64 * j] = acc[j];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int k = lane + 64 * j;
      const double sum = ((acc[j] + sh[0][lane + 64 * j]) + sh[1][lane + 64 * j]) + sh[2][lane + 64 * j];
      if (k < s) part[(size_t)blockIdx.x * s + k] = sum;
    }
  }
}

// w_k = sum over blocks of part[.][k]: 2 columns per workgroup, 128 fixed
// block ranges per column, combined by a fixed pairwise tree.
constexpr int kRedCols = 2;
__global__ void __launch_bounds__(256) k_pow_reduce(const double *__restrict__ part, int64_t nblk,
                                                    int64_t s, double *__restrict__ w) {
  constexpr int G = 256 / kRedCols;
  __shared__ double red[G][kRedCols];
  const int t = threadIdx.x, c = t % kRedCols, grp = t / kRedCols;
  const int64_t k = (int64_t)blockIdx.x * kRedCols + c;
  const int64_t q = (nblk + G - 1) / G;
  const int64_t b0 = grp * q, b1 = (b0 + q) < nblk ? (b0 + q) : nblk;
  double acc = 0.0;
  if (k < s)
    for (int64_t bi = b0; bi < b1; ++bi) acc += part[(size_t)bi * s + k];
  red[grp][c] = acc;
  __syncthreads();
  for (int o = G / 2; o >= 1; o >>= 1) {
    if (grp < o) red[grp][c] += red[grp + o][c];
    __syncthreads();
  }
  if (grp == 0 && k < s) w[k] = red[0][c];
}

// Fixed-order sum over a 1024-thread workgroup (tree over LDS).
__device__ inline double block_sum_1024(double v, double *sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

__device__ inline double block_max_1024(double v, double *sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (t < o) sh[t] = fmax(sh[t], sh[t + o]);
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(1024) k_pow_normalize(const double *__restrict__ w, int64_t s,
                                                        double *__restrict__ v,
                                                        double *__restrict__ diff) {
  __shared__ double sh[1024];
  const int t = threadIdx.x;
  double ss = 0.0;
  for (int64_t k = t; k < s; k += 1024) ss += w[k] * w[k];
  const double nrm = sqrt(block_sum_1024(ss, sh));
  double dm = 0.0;
  for (int64_t k = t; k < s; k += 1024) {
    const double vn = nrm > 0.0 ? w[k] / nrm : 0.0;
    dm = fmax(dm, fabs(vn - v[k]));
    v[k] = vn;
  }
  dm = block_max_1024(dm, sh);
  if (t == 0) *diff = dm;
}

__global__ void __launch_bounds__(1024) k_vec_norm(const double *__restrict__ x, int64_t n,
                                                   double *__restrict__ out) {
  __shared__ double sh[1024];
  double ss = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) ss += x[i] * x[i];
  const double r = sqrt(block_sum_1024(ss, sh));
  if (threadIdx.x == 0) *out = r;
}

__global__ void __launch_bounds__(256) k_fill(double *__restrict__ v, int64_t n, double val) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) v[i] = val;
}

__global__ void __launch_bounds__(256) k_init_scales(
    const double *__restrict__ xU, int64_t b, const double *__restrict__ vU,
    const double *__restrict__ xV, int64_t a, const double *__restrict__ vV, int64_t s,
    const double *__restrict__ sig, uint16_t *__restrict__ h, uint16_t *__restrict__ g,
    uint16_t *__restrict__ l) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const double sU = sig[0], sV = sig[1];
  const double rU = sqrt(sU), rV = sqrt(sV);
  if (i < b) h[i] = sU > 0.0 ? f16_bits_rne(xU[i] / rU) : 0;
  if (i < a) g[i] = sV > 0.0 ? f16_bits_rne(xV[i] / rV) : 0;
  if (i < s) l[i] = f16_bits_rne((vU[i] * rU) * (vV[i] * rV));
}

inline unsigned grid_of(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

// Rank-1 fit of |F| (n x s): v (s) the unit right vector, x = |F| v (n),
// *sigma = ||x||.  Returns the first HIP error; *converged is false when the
// iterate still moved by more than tol after max_iters steps.
// Rows per workgroup of the register-resident step: about four workgroups
// per compute unit over the matrix (enough waves to cover the load
// latency; more make the partial sums cost more), at least 8 rows.
constexpr int kFusedMaxKM = 16;
constexpr int kFusedBlocks = 1024;
inline int fused_rpb(int64_t n) {
  const int64_t r = (n + kFusedBlocks - 1) / kFusedBlocks;
  return (int)(r < 8 ? 8 : r);
}
inline int64_t fused_nblk(int64_t n) { return (n + fused_rpb(n) - 1) / fused_rpb(n); }

template <typename T, int KM>
void launch_fused_km(const T *F, int64_t n, int s, const double *v, double *part,
                     hipStream_t st) {
  const int rpb = fused_rpb(n);
  hipLaunchKernelGGL((k_pow_fused<T, KM>), dim3((unsigned)fused_nblk(n)), dim3(256), 0, st, F, n, s,
                     rpb, v, part);
}

// One step's A^T (A v) partials; returns the number of partial rows.
template <typename T>
int64_t launch_pow_step(const T *F, int64_t n, int64_t s, const double *v, double *part,
                        hipStream_t st) {
  const int64_t km = (s + 63) / 64;
  if (km > kFusedMaxKM) {
    const int64_t nblk = (n + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(k_pow_block<T>, dim3((unsigned)nblk), dim3(256), 0, st, F, n, s, v, part,
                       (double *)nullptr);
    return nblk;
  }
  switch (km) {
#define LB_KM(K) \
  case K:        \
    launch_fused_km<T, K>(F, n, (int)s, v, part, st); \
    break;
    LB_KM(1) LB_KM(2) LB_KM(3) LB_KM(4) LB_KM(5) LB_KM(6) LB_KM(7) LB_KM(8)
    LB_KM(9) LB_KM(10) LB_KM(11) LB_KM(12) LB_KM(13) LB_KM(14) LB_KM(15) LB_KM(16)
#undef LB_KM
  }
  return fused_nblk(n);
}

template <typename T>
hipError_t fit_rank1(const T *F, int64_t n, int64_t s, double *v, double *x, double *w,
                     double *part, double *diff, double *sigma, int max_iters, double tol,
                     hipStream_t st, bool *converged, int *iters) {
  const int64_t nblk = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  *converged = false;
  *iters = 0;
  hipLaunchKernelGGL(k_fill, dim3(grid_of(s, 256)), dim3(256), 0, st, v, s,
                     1.0 / std::sqrt((double)s));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  while (*iters < max_iters) {
    for (int i = 0; i < kCheckEvery; ++i) {
      const int64_t np = launch_pow_step(F, n, s, v, part, st);
      hipLaunchKernelGGL(k_pow_reduce, dim3(grid_of(s, kRedCols)), dim3(256), 0, st, part, np, s,
                         w);
      hipLaunchKernelGGL(k_pow_normalize, dim3(1), dim3(1024), 0, st, w, s, v, diff);
    }
    *iters += kCheckEvery;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    double d = 0.0;
    if ((e = hipMemcpyAsync(&d, diff, sizeof(double), hipMemcpyDeviceToHost, st)) != hipSuccess)
      return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    if (d <= tol) {
      *converged = true;
      break;
    }
  }
  hipLaunchKernelGGL(k_pow_block<T>, dim3((unsigned)nblk), dim3(256), 0, st, F, n, s, v,
                     (double *)nullptr, x);
  hipLaunchKernelGGL(k_vec_norm, dim3(1), dim3(1024), 0, st, x, n, sigma);
  return hipGetLastError();
}

}  // namespace

// Partial rows of either step kind, for the larger factor.
inline int64_t part_rows(int64_t nmax) {
  const int64_t a = (nmax + kRowsPerBlock - 1) / kRowsPerBlock, b = fused_nblk(nmax);
  return a > b ? a : b;
}

size_t init_ws_bytes(int64_t a, int64_t b, int64_t s) {
  const int64_t nmax = a > b ? a : b;
  const int64_t nblk = part_rows(nmax);
  const int64_t Wk = (s + 31) / 32;
  size_t d = (size_t)(4 * s + a + b + nblk * s + 4);  // doubles
  size_t bytes = d * 8;
  bytes += (size_t)(a + b) * Wk * 4;       // sign words
  bytes += (size_t)(a + b + s) * 2 + 256;  // fp16 scales
  return bytes;
}

template <typename T>
hipError_t init_dev_impl(const T *U, const T *V, int64_t a, int64_t b, int64_t s, void *ws,
                         hipStream_t st, InitResult *res) {
  const int64_t nmax = a > b ? a : b;
  const int64_t nblk = part_rows(nmax);
  const int64_t Wk = (s + 31) / 32;
  double *d = static_cast<double *>(ws);
  double *vU = d, *vV = vU + s, *w = vV + s, *xU = w + s, *xV = xU + b, *part = xV + a;
  double *scal = part + (size_t)nblk * s;  // [0] sigma_U, [1] sigma_V, [2] diff
  uint32_t *su = reinterpret_cast<uint32_t *>(scal + 4);
  uint32_t *sv = su + (size_t)b * Wk;
  uint16_t *h = reinterpret_cast<uint16_t *>(sv + (size_t)a * Wk);
  uint16_t *g = h + b, *l = g + a;
  res->su = su;
  res->sv = sv;
  res->h = h;
  res->g = g;
  res->l = l;
  res->sigma = scal;

  hipLaunchKernelGGL(k_sign_words<T>, dim3(grid_of(b, 4)), dim3(256), 0, st, U, b, s, Wk, su);
  hipLaunchKernelGGL(k_sign_words<T>, dim3(grid_of(a, 4)), dim3(256), 0, st, V, a, s, Wk, sv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int max_iters = 2048;
  const double tol = 1e-13;
  bool cu = false, cv = false;
  if ((e = fit_rank1(U, b, s, vU, xU, w, part, scal + 2, scal + 0, max_iters, tol, st, &cu,
                     &res->iters_u)) != hipSuccess)
    return e;
  if ((e = fit_rank1(V, a, s, vV, xV, w, part, scal + 2, scal + 1, max_iters, tol, st, &cv,
                     &res->iters_v)) != hipSuccess)
    return e;
  res->converged = cu && cv;
  const int64_t m = nmax > s ? nmax : s;
  hipLaunchKernelGGL(k_init_scales, dim3(grid_of(m, 256)), dim3(256), 0, st, xU, b, vU, xV, a, vV,
                     s, scal, h, g, l);
  return hipGetLastError();
}

hipError_t init_from_factors_dev(const float *U, const float *V, int64_t a, int64_t b, int64_t s,
                                 void *ws, hipStream_t st, InitResult *res) {
  return init_dev_impl<float>(U, V, a, b, s, ws, st, res);
}

hipError_t init_from_factors_dev(const double *U, const double *V, int64_t a, int64_t b, int64_t s,
                                 void *ws, hipStream_t st, InitResult *res) {
  return init_dev_impl<double>(U, V, a, b, s, ws, st, res);
}

}  // namespace lbi
