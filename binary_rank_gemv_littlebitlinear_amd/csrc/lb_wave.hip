// Wave-level binary GEMV path (M < 64 rows of x).
//
// [LB news] Sec. 2: inference is two small binary matrix products with
// elementwise scaling.  With S in {+-1} stored as bits (1 = +1), each
// product uses the sign-flip identity
//     sum_i s_i v_i = 2 * sum_{bit_i = 1} v_i - sum_i v_i,
// so the inner loop only adds the entries whose bit is set.
//
// Stage 1 (per chunk of input rows): partial t[c] over the chunk for every
// latent column c = p*s + k, with z = g_p * x kept in LDS.
// Reduce: t = sum of partials (fixed order), w = l * t.
// Stage 2: u_p[j] = 2 * sum_{bit} w_p[k] - sum_k w_p[k]; y = sum_p h_p u_p.
#include <hip/hip_fp16.h>

#include "lb_internal.h"

namespace lbi {

__device__ __forceinline__ float h2f(uint16_t v) {
  return __half2float(__ushort_as_half(v));
}
__device__ __forceinline__ uint16_t f2h(float v) {
  return __half_as_ushort(__float2half_rn(v));
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  // 64-lane wave reduction, then across waves through LDS.
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float tot = 0.f;
  const int nw = (blockDim.x + 63) >> 6;
  for (int w = 0; w < nw; ++w) tot += red[w];
  return tot;
}

constexpr int kS1Threads = 256;

// grid.x = nchunk; chunk c covers row groups [c*G, min(c*G+G, R1)).
// part[(c*M + m)*L + col] = 2 * sum_{bit} z - sum z over the chunk.
__global__ void __launch_bounds__(kS1Threads)
k_wave_stage1(const uint32_t *__restrict__ sv1, const uint16_t *__restrict__ g,
              const uint16_t *__restrict__ x, int64_t a, int64_t a16, int64_t s, int64_t L, int P,
              int64_t R1, int M, int G, float *__restrict__ part) {
  extern __shared__ float smem[];
  const int c = blockIdx.x;
  const int64_t r0 = (int64_t)c * G;
  const int64_t r1 = r0 + G < R1 ? r0 + G : R1;
  if (r0 >= r1) return;
  const int nrow = (int)(r1 - r0) * 32;
  const int zstride = G * 32;
  float *z = smem;                       // [M][P][G*32]
  float *sz = smem + (size_t)M * P * zstride;  // [M][P]
  float *red = sz + M * P;               // [waves]

  for (int idx = threadIdx.x; idx < M * P * nrow; idx += blockDim.x) {
    const int m = idx / (P * nrow);
    const int rem = idx - m * P * nrow;
    const int p = rem / nrow;
    const int il = rem - p * nrow;
    const int64_t i = r0 * 32 + il;
    float v = 0.f;
    if (i < a) v = h2f(g[p * a16 + i]) * h2f(x[(int64_t)m * a + i]);
    z[(m * P + p) * zstride + il] = v;
  }
  __syncthreads();
  for (int mp = 0; mp < M * P; ++mp) {
    float v = 0.f;
    for (int il = threadIdx.x; il < nrow; il += blockDim.x) v += z[mp * zstride + il];
    v = block_sum(v, red);
    if (threadIdx.x == 0) sz[mp] = v;
  }
  __syncthreads();

  for (int64_t col = threadIdx.x; col < L; col += blockDim.x) {
    const int p = (int)(col / s);
    for (int m = 0; m < M; ++m) {
      const float *zp = z + (m * P + p) * zstride;
      float acc = 0.f;
      for (int64_t r = r0; r < r1; ++r) {
        const uint32_t wd = sv1[r * L + col];
        const float *zr = zp + (r - r0) * 32;
#pragma unroll
        for (int bit = 0; bit < 32; ++bit) acc += ((wd >> bit) & 1u) ? zr[bit] : 0.f;
      }
      part[((int64_t)c * M + m) * L + col] = 2.f * acc - sz[m * P + p];
    }
  }
}

// w[m*L + col] = l[col] * sum_c part[(c*M + m)*L + col]
__global__ void k_wave_reduce(const float *__restrict__ part, const uint16_t *__restrict__ l,
                              int64_t s, int64_t s8, int64_t L, int M, int nchunk,
                              float *__restrict__ w) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * L) return;
  const int m = (int)(idx / L);
  const int64_t col = idx - (int64_t)m * L;
  float t = 0.f;
  for (int c = 0; c < nchunk; ++c) t += part[((int64_t)c * M + m) * L + col];
  const int64_t p = col / s;
  w[idx] = h2f(l[p * s8 + (col - p * s)]) * t;
}

constexpr int kS2Threads = 256;

// One thread per output row j.  LDS holds w for one row of x at a time.
__global__ void __launch_bounds__(kS2Threads)
k_wave_stage2(const uint32_t *__restrict__ su2, const uint16_t *__restrict__ h,
              const float *__restrict__ w, int64_t b, int64_t b16, int64_t s, int64_t L, int P,
              int64_t Wk, int M, uint16_t *__restrict__ y) {
  extern __shared__ float smem[];
  float *wl = smem;           // [L]
  float *ws = smem + L;       // [P]
  float *red = ws + 2;        // [waves]
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int m = 0; m < M; ++m) {
    __syncthreads();
    for (int64_t c = threadIdx.x; c < L; c += blockDim.x) wl[c] = w[(int64_t)m * L + c];
    __syncthreads();
    for (int p = 0; p < P; ++p) {
      float v = 0.f;
      for (int64_t k = threadIdx.x; k < s; k += blockDim.x) v += wl[p * s + k];
      v = block_sum(v, red);
      if (threadIdx.x == 0) ws[p] = v;
    }
    __syncthreads();
    if (j < b) {
      float out = 0.f;
      for (int p = 0; p < P; ++p) {
        const float *wp = wl + p * s;
        float acc = 0.f;
        for (int64_t q = 0; q < Wk; ++q) {
          const uint32_t wd = su2[(p * Wk + q) * b16 + j];
          const int64_t kb = q * 32;
          const int nb = (s - kb) < 32 ? (int)(s - kb) : 32;
          if (nb == 32) {
#pragma unroll
            for (int bit = 0; bit < 32; ++bit) acc += ((wd >> bit) & 1u) ? wp[kb + bit] : 0.f;
          } else {
            for (int bit = 0; bit < nb; ++bit) acc += ((wd >> bit) & 1u) ? wp[kb + bit] : 0.f;
          }
        }
        out += h2f(h[p * b16 + j]) * (2.f * acc - ws[p]);
      }
      y[(int64_t)m * b + j] = f2h(out);
    }
  }
}

// Row groups per chunk so that z for all M rows and paths fits in 48 KB.
static int wave_gmax(const Layer &Ly, int64_t M) {
  int64_t g = (48 * 1024 / 4 - 64) / (M * Ly.P * 32);
  return (int)(g < 1 ? 1 : (g > 64 ? 64 : g));
}

int wave_nchunk(const Layer &Ly, int64_t M, const DeviceInfo &dev) {
  // Enough chunks to cover the device twice, each at least one row group,
  // and few enough row groups per chunk for the LDS copy of z.
  int64_t want = 2LL * (dev.cu_count > 0 ? dev.cu_count : 256);
  if (want > Ly.R1) want = Ly.R1;
  const int64_t gmax = wave_gmax(Ly, M);
  const int64_t need = (Ly.R1 + gmax - 1) / gmax;
  if (want < need) want = need;
  return (int)(want < 1 ? 1 : want);
}

size_t wave_ws_floats(const Layer &Ly, int64_t M, int nchunk) {
  return (size_t)nchunk * (size_t)M * (size_t)Ly.L;
}

hipError_t launch_wave_stage1(const Layer &Ly, const uint16_t *x, float *w_out, int64_t M,
                              int nchunk, float *ws, hipStream_t st) {
  const int G = (int)((Ly.R1 + nchunk - 1) / nchunk);
  const int nch = (int)((Ly.R1 + G - 1) / G);
  const size_t lds = ((size_t)M * Ly.P * G * 32 + (size_t)M * Ly.P + 16) * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_wave_stage1, dim3(nch), dim3(kS1Threads), lds, st, Ly.sv1, Ly.g, x, Ly.a,
                     Ly.a16, Ly.s, Ly.L, Ly.P, Ly.R1, (int)M, G, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = M * Ly.L;
  hipLaunchKernelGGL(k_wave_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ws, Ly.l,
                     Ly.s, Ly.s8, Ly.L, (int)M, nch, w_out);
  return hipGetLastError();
}

hipError_t launch_wave_stage2(const Layer &Ly, const float *w, uint16_t *y, int64_t M,
                              hipStream_t st) {
  const size_t lds = ((size_t)Ly.L + 2 + 16) * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_wave_stage2, dim3((unsigned)((Ly.b + kS2Threads - 1) / kS2Threads)),
                     dim3(kS2Threads), lds, st, Ly.su2, Ly.h, w, Ly.b, Ly.b16, Ly.s, Ly.L, Ly.P,
                     Ly.Wk, (int)M, y);
  return hipGetLastError();
}

// out = fp16(c * sum of n_in fp16 inputs), in fp32.
struct CombineArgs {
  const uint16_t *in[8];
};

__global__ void k_combine(CombineArgs args, int n_in, float c, uint16_t *__restrict__ out,
                          int64_t elems) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= elems) return;
  float acc = 0.f;
  for (int u = 0; u < n_in; ++u) acc += h2f(args.in[u][i]);
  out[i] = f2h(c * acc);
}

hipError_t launch_combine(const uint16_t *const *ins, int n_in, float c, uint16_t *out,
                          int64_t elems, hipStream_t st) {
  if (n_in < 1 || n_in > 8) return hipErrorInvalidValue;
  CombineArgs args{};
  for (int u = 0; u < n_in; ++u) args.in[u] = ins[u];
  if (elems == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, st, args,
                     n_in, c, out, elems);
  return hipGetLastError();
}

}  // namespace lbi
