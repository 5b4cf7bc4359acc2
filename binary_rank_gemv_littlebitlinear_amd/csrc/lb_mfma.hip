// MFMA path (used for M >= 64 rows of x).
//
// With many rows of x the two binary products of [LB news] Sec. 2 are
// real dense contractions, so they run on the fp16 matrix cores:
//   stage 1: T[M x L]  = x[M x a] . B1[a x L],  B1[i][p*s+k] = S_V,p[i,k] * g_p[i]
//   stage 2: Y[M x b]  = sum_p h_p * ( fp16(T_p)[M x s] . B2_p[s x b] ),
//            B2_p[k][j] = S_U,p[j,k] * l_p[k]
// +-g and +-l are exact in fp16 (a sign flip), so the only rounding of an
// operand is T -> fp16, once.  Accumulation is fp32.  The bits are
// expanded to fp16 in LDS per K-tile, where the M rows of the tile
// amortise the expansion.
//
// Tiles: 64 x 64 output per workgroup of 4 waves (2 x 2 waves of 32 x 32),
// K-step 32, v_mfma_f32_16x16x16_f16.  Stage 1 splits K across
// workgroups; a reduce kernel sums the splits and rounds T to fp16 into a
// zero-padded [P][M][s_pad] buffer.
#include <hip/hip_fp16.h>

#include "lb_internal.h"

namespace lbi {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 64, BN = 64, BK = 32;
constexpr int kPadK = 8;  // LDS row padding (halfs) against bank conflicts
constexpr int kMfmaThreads = 256;
constexpr int kMChunk = 256;  // rows of x per pass (bounds the workspace)

__device__ __forceinline__ float mh2f(uint16_t v) { return __half2float(__ushort_as_half(v)); }
__device__ __forceinline__ uint16_t mf2h(float v) { return __half_as_ushort(__float2half_rn(v)); }

static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Load a BM x BK fp16 tile of A (row-major, lda) into As[BM][BK+pad].
__device__ __forceinline__ void load_a_tile(const uint16_t *__restrict__ A, int64_t lda, int64_t M,
                                            int64_t K, int64_t m0, int64_t k0,
                                            uint16_t (*As)[BK + kPadK]) {
  const int t = threadIdx.x;
  const int r = t >> 2;          // 0..63
  const int kseg = (t & 3) * 8;  // 0, 8, 16, 24
  const int64_t m = m0 + r;
  const int64_t k = k0 + kseg;
  uint16_t v[8];
  const uint16_t *src = A + m * lda + k;
  if (m < M && k + 8 <= K && (((uintptr_t)src) & 15) == 0) {
    const uint4 q = *reinterpret_cast<const uint4 *>(src);
    v[0] = q.x & 0xffff; v[1] = q.x >> 16; v[2] = q.y & 0xffff; v[3] = q.y >> 16;
    v[4] = q.z & 0xffff; v[5] = q.z >> 16; v[6] = q.w & 0xffff; v[7] = q.w >> 16;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (m < M && k + e < K) ? src[e] : (uint16_t)0;
  }
  uint4 o;
  o.x = v[0] | ((uint32_t)v[1] << 16); o.y = v[2] | ((uint32_t)v[3] << 16);
  o.z = v[4] | ((uint32_t)v[5] << 16); o.w = v[6] | ((uint32_t)v[7] << 16);
  *reinterpret_cast<uint4 *>(&As[r][kseg]) = o;
}

// One BK-step of MFMAs for a wave's 32 x 32 sub-tile.
__device__ __forceinline__ void mma_step(const uint16_t (*As)[BK + kPadK],
                                         const uint16_t (*Bs)[BK + kPadK], int wm, int wn,
                                         float4_t acc[2][2]) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lk = (lane >> 4) * 4;
#pragma unroll
  for (int kk = 0; kk < BK; kk += 16) {
    half4_t af[2], bf[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
      af[mi] = *reinterpret_cast<const half4_t *>(&As[wm * 32 + mi * 16 + li][kk + lk]);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      bf[ni] = *reinterpret_cast<const half4_t *>(&Bs[wn * 32 + ni * 16 + li][kk + lk]);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x16f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
  }
}

// Stage 1: part[split][m][col] = sum over this split's K range of x . B1.
// grid = (ceil(L/BN), ceil(Mc/BM), nsplit); K range per split is a
// multiple of BK.
__global__ void __launch_bounds__(kMfmaThreads)
k_mfma_stage1(const uint16_t *__restrict__ x, int64_t M, const uint32_t *__restrict__ sv1,
              const uint16_t *__restrict__ g, int64_t a, int64_t a16, int64_t s, int64_t L,
              int64_t kper, float *__restrict__ part) {
  __shared__ __align__(16) uint16_t As[BM][BK + kPadK];
  __shared__ __align__(16) uint16_t Bs[BN][BK + kPadK];
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
  const int64_t kbeg = (int64_t)blockIdx.z * kper;
  const int64_t kend = kbeg + kper < a ? kbeg + kper : a;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  float4_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = float4_t{0.f, 0.f, 0.f, 0.f};

  // B-tile expansion: thread -> column n = t / 4, 8 consecutive k
  const int bn = threadIdx.x >> 2, bk = (threadIdx.x & 3) * 8;
  const int64_t col = n0 + bn;
  const int p = col < L ? (int)(col / s) : 0;
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    load_a_tile(x, a, M, a, m0, k0, As);
    {
      uint16_t v[8];
      if (col < L) {
        const uint32_t wd = sv1[(k0 >> 5) * L + col];  // k0 is a multiple of 32
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t i = k0 + bk + e;
          const uint16_t gv = i < a ? g[p * a16 + i] : (uint16_t)0;
          const uint32_t bit = (wd >> (bk + e)) & 1u;
          v[e] = bit ? gv : (uint16_t)(gv ^ 0x8000u);
          if (i >= a) v[e] = 0;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0;
      }
      uint4 o;
      o.x = v[0] | ((uint32_t)v[1] << 16); o.y = v[2] | ((uint32_t)v[3] << 16);
      o.z = v[4] | ((uint32_t)v[5] << 16); o.w = v[6] | ((uint32_t)v[7] << 16);
      *reinterpret_cast<uint4 *>(&Bs[bn][bk]) = o;
    }
    __syncthreads();
    mma_step(As, Bs, wm, wn, acc);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  float *out = part + (int64_t)blockIdx.z * M * L;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 32 + mi * 16 + (lane >> 4) * 4 + r;
        const int64_t c = n0 + wn * 32 + ni * 16 + (lane & 15);
        if (m < M && c < L) out[m * L + c] = acc[mi][ni][r];
      }
}

// T16[p][m][k] = fp16(sum_split part[split][m][p*s+k]) for k < s, 0 up to s_pad.
__global__ void k_mfma_reduce(const float *__restrict__ part, int nsplit, int64_t M, int64_t s,
                              int64_t L, int P, int64_t s_pad, uint16_t *__restrict__ T16) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)P * M * s_pad;
  if (idx >= total) return;
  const int p = (int)(idx / (M * s_pad));
  const int64_t rem = idx - (int64_t)p * M * s_pad;
  const int64_t m = rem / s_pad, k = rem - m * s_pad;
  float t = 0.f;
  if (k < s)
    for (int z = 0; z < nsplit; ++z) t += part[((int64_t)z * M + m) * L + p * s + k];
  T16[idx] = k < s ? mf2h(t) : (uint16_t)0;
}

// Stage 2: y[m][j] = fp16( sum_p h_p[j] * sum_k T16_p[m][k] * B2_p[k][j] ).
// grid = (ceil(b/BN), ceil(Mc/BM)).
__global__ void __launch_bounds__(kMfmaThreads)
k_mfma_stage2(const uint16_t *__restrict__ T16, int64_t M, int64_t s_pad,
              const uint32_t *__restrict__ su2, const uint16_t *__restrict__ l,
              const uint16_t *__restrict__ h, int64_t b, int64_t b16, int64_t s, int64_t s8,
              int64_t Wk, int P, uint16_t *__restrict__ y) {
  __shared__ __align__(16) uint16_t As[BM][BK + kPadK];
  __shared__ __align__(16) uint16_t Bs[BN][BK + kPadK];
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  float4_t acc[2][2][2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[pp][mi][ni] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int bn = threadIdx.x >> 2, bk = (threadIdx.x & 3) * 8;
  const int64_t j = n0 + bn;
  for (int p = 0; p < P; ++p) {
    const uint16_t *Ap = T16 + (int64_t)p * M * s_pad;
    for (int64_t k0 = 0; k0 < s_pad; k0 += BK) {
      load_a_tile(Ap, s_pad, M, s_pad, m0, k0, As);
      {
        uint16_t v[8];
        if (j < b) {
          const uint32_t wd = su2[(p * Wk + (k0 >> 5)) * b16 + j];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + bk + e;
            const uint16_t lv = k < s ? l[p * s8 + k] : (uint16_t)0;
            const uint32_t bit = (wd >> (bk + e)) & 1u;
            v[e] = k < s ? (bit ? lv : (uint16_t)(lv ^ 0x8000u)) : (uint16_t)0;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0;
        }
        uint4 o;
        o.x = v[0] | ((uint32_t)v[1] << 16); o.y = v[2] | ((uint32_t)v[3] << 16);
        o.z = v[4] | ((uint32_t)v[5] << 16); o.w = v[6] | ((uint32_t)v[7] << 16);
        *reinterpret_cast<uint4 *>(&Bs[bn][bk]) = o;
      }
      __syncthreads();
      if (p == 0)
        mma_step(As, Bs, wm, wn, acc[0]);
      else
        mma_step(As, Bs, wm, wn, acc[1]);
      __syncthreads();
    }
  }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 32 + mi * 16 + (lane >> 4) * 4 + r;
        const int64_t c = n0 + wn * 32 + ni * 16 + (lane & 15);
        if (m < M && c < b) {
          float v = mh2f(h[c]) * acc[0][mi][ni][r];
          if (P > 1) v += mh2f(h[b16 + c]) * acc[1][mi][ni][r];
          y[m * b + c] = mf2h(v);
        }
      }
}

static int mfma_nsplit(const Layer &Ly, int64_t Mc, const DeviceInfo &dev) {
  const int64_t tiles = ((Ly.L + BN - 1) / BN) * ((Mc + BM - 1) / BM);
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  int64_t ns = (2 * cus + tiles - 1) / tiles;
  const int64_t ksteps = (Ly.a + BK - 1) / BK;
  if (ns > ksteps) ns = ksteps;
  if (ns > 16) ns = 16;
  return (int)(ns < 1 ? 1 : ns);
}

size_t mfma_ws_bytes(const Layer &Ly, int64_t M) {
  const int64_t Mc = M < kMChunk ? M : kMChunk;
  const int64_t s_pad = round_up(Ly.s, BK);
  return (size_t)16 * Mc * Ly.L * sizeof(float) + (size_t)Ly.P * Mc * s_pad * 2 + 256;
}

hipError_t launch_mfma_forward(const Layer &Ly, const uint16_t *x, uint16_t *y, int64_t M,
                               void *ws, const DeviceInfo &dev, hipStream_t st) {
  const int64_t s_pad = round_up(Ly.s, BK);
  for (int64_t mb = 0; mb < M; mb += kMChunk) {
    const int64_t Mc = (M - mb) < kMChunk ? (M - mb) : kMChunk;
    const int ns = mfma_nsplit(Ly, Mc, dev);
    const int64_t ksteps = (Ly.a + BK - 1) / BK;
    const int64_t kper = ((ksteps + ns - 1) / ns) * BK;
    const int nsr = (int)((Ly.a + kper - 1) / kper);
    float *part = reinterpret_cast<float *>(ws);
    uint16_t *T16 = reinterpret_cast<uint16_t *>(
        reinterpret_cast<char *>(ws) + (size_t)16 * Mc * Ly.L * sizeof(float));
    dim3 g1((unsigned)((Ly.L + BN - 1) / BN), (unsigned)((Mc + BM - 1) / BM), (unsigned)nsr);
    hipLaunchKernelGGL(k_mfma_stage1, g1, dim3(kMfmaThreads), 0, st, x + mb * Ly.a, Mc, Ly.sv1,
                       Ly.g, Ly.a, Ly.a16, Ly.s, Ly.L, kper, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nT = (int64_t)Ly.P * Mc * s_pad;
    hipLaunchKernelGGL(k_mfma_reduce, dim3((unsigned)((nT + 255) / 256)), dim3(256), 0, st, part,
                       nsr, Mc, Ly.s, Ly.L, Ly.P, s_pad, T16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2((unsigned)((Ly.b + BN - 1) / BN), (unsigned)((Mc + BM - 1) / BM));
    hipLaunchKernelGGL(k_mfma_stage2, g2, dim3(kMfmaThreads), 0, st, T16, Mc, s_pad, Ly.su2, Ly.l,
                       Ly.h, Ly.b, Ly.b16, Ly.s, Ly.s8, Ly.Wk, Ly.P, y + mb * Ly.b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lbi
