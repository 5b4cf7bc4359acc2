// Wave-level binary GEMV path (M < 64 rows of x).
//
// [LB news] Sec. 2: inference is two small binary matrix products with
// elementwise scaling.  With S in {+-1} stored as bits (1 = +1), each
// product uses the sign-flip identity
//     sum_i s_i v_i = 2 * sum_{bit_i = 1} v_i - sum_i v_i,
// and the sum over set bits is taken four bits at a time from 16-entry
// tables in LDS: for a group of four entries (v0..v3) of the vector,
// tab[n] = sum of the v_e whose bit e of n is set, so one word of 32 sign
// bits costs eight table reads.  All 64 lanes of a wave read the same
// table at a time (one group), so the reads are bank-conflict free.
//
// Stage 1 (k_wave_s1): one workgroup per chunk of input rows builds the
//   tables of z = g_p * x for its rows, then each thread takes latent
//   columns c = p*s + k: part[chunk][m][c] = 2 * sum_{bit} z - sum z over
//   the chunk (its words read once for all rows m).
// Reduce (k_wave_reduce): w = l * sum of the chunk partials, 16 fixed
//   chunk ranges per column combined by a fixed pairwise tree.
// Stage 2 (k_wave_s2): tables of w_p for a batch of rows m (as many as fit
//   in 48 KB, so one build and three barriers serve several rows); four
//   lanes per output row j split its words (kept in registers for every
//   row) and are summed by a fixed shuffle tree:
//   y[m][j] = fp16(sum_p h_p[j] (2 * sum_{bit} w_p - sum_k w_p[k])).
//   Layers whose tables would not fit (P * ceil(s/32) > 96) use
//   k_wave_s2_bits, one thread per row testing bits one by one.
// Every sum has a fixed order, so results are deterministic.
#include <hip/hip_fp16.h>

#include <algorithm>

#include "lb_internal.h"

namespace lbi {

__device__ __forceinline__ float h2f(uint16_t v) {
  return __half2float(__ushort_as_half(v));
}
__device__ __forceinline__ uint16_t f2h(float v) {
  return __half_as_ushort(__float2half_rn(v));
}

// 16 sums of subsets of (v0, v1, v2, v3): entry n sums the v_e with bit e of n set.
__device__ __forceinline__ void build_table(float *tab, float v0, float v1, float v2, float v3) {
  tab[0] = 0.f;
  tab[1] = v0;
  tab[2] = v1;
  tab[3] = v0 + v1;
  tab[4] = v2;
  tab[5] = v0 + v2;
  tab[6] = v1 + v2;
  tab[7] = (v0 + v1) + v2;
  tab[8] = v3;
  tab[9] = v0 + v3;
  tab[10] = v1 + v3;
  tab[11] = (v0 + v1) + v3;
  tab[12] = v2 + v3;
  tab[13] = (v0 + v2) + v3;
  tab[14] = (v1 + v2) + v3;
  tab[15] = ((v0 + v1) + v2) + v3;
}

// sum over the set bits of word: eight table reads, tables tab[g*16 + n]
__device__ __forceinline__ float lut_word(const float *tab, uint32_t wd) {
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) acc += tab[g * 16 + ((wd >> (4 * g)) & 15u)];
  return acc;
}

constexpr int kS1Threads = 256;
constexpr int kS1TabFloats = 12288;  // 48 KB of stage-1 tables per batch of rows

// Rows m processed together by one stage-1 workgroup (tables of every such
// row in LDS at once).
static int s1_mbatch(const Layer &Ly, int G) {
  const int per_row = Ly.P * G * 8 * 16;
  const int mb = kS1TabFloats / per_row;
  return mb < 1 ? 1 : mb;
}

// grid.x = nchunk; chunk c covers row groups [c*G, min(c*G+G, R1)).
// LDS: tab[mi][p][grp][16] (grp < 8 G), sz[mi][p].
__global__ void __launch_bounds__(kS1Threads)
k_wave_s1(const uint32_t *__restrict__ sv1, const uint16_t *__restrict__ g,
          const uint16_t *__restrict__ x, int64_t a, int64_t a16, int64_t s, int64_t L, int P,
          int64_t R1, int M, int G, int MB, float *__restrict__ part) {
  extern __shared__ float smem[];
  const int c = blockIdx.x, t = threadIdx.x;
  const int64_t r0 = (int64_t)c * G;
  const int64_t r1 = r0 + G < R1 ? r0 + G : R1;
  if (r0 >= r1) return;
  const int ng = (int)(r1 - r0) * 8;  // table groups of this chunk
  const int tabs = P * G * 8 * 16;    // floats per row m
  float *tab = smem;                  // [MB][P][G*8][16]
  float *sz = smem + (size_t)MB * tabs;  // [MB][P]
  for (int m0 = 0; m0 < M; m0 += MB) {
    const int mn = (M - m0) < MB ? (M - m0) : MB;
    __syncthreads();  // the previous batch's lookups are done
    for (int idx = t; idx < mn * P * ng; idx += kS1Threads) {
      const int mi = idx / (P * ng);
      const int rem = idx - mi * P * ng;
      const int p = rem / ng, gr = rem - p * ng;
      const int64_t i0 = r0 * 32 + 4 * gr;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        v[e] = i < a ? h2f(g[p * a16 + i]) * h2f(x[(int64_t)(m0 + mi) * a + i]) : 0.f;
      }
      build_table(tab + ((size_t)(mi * P + p) * G * 8 + gr) * 16, v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    for (int idx = t; idx < mn * P; idx += kS1Threads) {
      const float *tb = tab + (size_t)idx * G * 8 * 16;
      float acc = 0.f;
      for (int gr = 0; gr < ng; ++gr) acc += tb[gr * 16 + 15];
      sz[idx] = acc;
    }
    __syncthreads();
    // a thread per column: its words are loaded once, before the rows
    for (int64_t col = t; col < L; col += kS1Threads) {
      const int p = (int)((uint32_t)col / (uint32_t)s);  // col < L = P s <= 8192
      uint32_t wd[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wd[r] = (r0 + r < r1) ? sv1[(r0 + r) * L + col] : 0u;
      for (int mi = 0; mi < mn; ++mi) {
        const float *tb = tab + (size_t)(mi * P + p) * G * 8 * 16;
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r0 + r < r1) acc += lut_word(tb + r * 8 * 16, wd[r]);
        for (int r = 4; r < (int)(r1 - r0); ++r) acc += lut_word(tb + r * 8 * 16, sv1[(r0 + r) * L + col]);
        part[((int64_t)c * M + m0 + mi) * L + col] = 2.f * acc - sz[mi * P + p];
      }
    }
  }
}

// w[m*L + col] = l[col] * sum_c part[(c*M + m)*L + col]: 16 columns per
// workgroup, 16 fixed chunk ranges per column, a fixed pairwise tree.
__global__ void __launch_bounds__(256) k_wave_reduce(const float *__restrict__ part,
                                                     const uint16_t *__restrict__ l, int64_t s,
                                                     int64_t s8, int64_t L, int M, int nchunk,
                                                     float *__restrict__ w) {
  __shared__ float red[16][16];
  const int t = threadIdx.x, cl = t & 15, grp = t >> 4;
  const int64_t idx = (int64_t)blockIdx.x * 16 + cl;
  const bool live = idx < (int64_t)M * L;
  // M < 64 and L = P s <= 8192 here, so idx, col and s fit 32-bit divisions
  const int m = live ? (int)((uint32_t)idx / (uint32_t)L) : 0;
  const int64_t col = live ? idx - (int64_t)m * L : 0;
  const int q = (nchunk + 15) / 16;
  const int c0 = grp * q, c1 = (c0 + q) < nchunk ? (c0 + q) : nchunk;
  float acc = 0.f;
  if (live)
    for (int c = c0; c < c1; ++c) acc += part[((int64_t)c * M + m) * L + col];
  red[grp][cl] = acc;
  __syncthreads();
  for (int o = 8; o >= 1; o >>= 1) {
    if (grp < o) red[grp][cl] += red[grp + o][cl];
    __syncthreads();
  }
  if (grp == 0 && live) {
    const int64_t p = (uint32_t)col / (uint32_t)s;
    w[idx] = h2f(l[p * s8 + (col - p * s)]) * red[0][cl];
  }
}

constexpr int kS2Threads = 256;
constexpr int kS2Lanes = 4;                        // lanes per output row
constexpr int kS2Rows = kS2Threads / kS2Lanes;     // output rows per workgroup
constexpr int kS2MaxWords = 96;                    // P * Wk with tables (48 KB per row m)
constexpr int kS2TabFloats = 12288;                // 48 KB of tables per batch of rows m
constexpr int kS2MaxBatch = 16;

// Rows m whose tables (and w rows) share one build.
static int s2_mbatch(int nw, int64_t L) {
  const int64_t mb = kS2TabFloats / ((int64_t)nw * 128 + L);
  return mb < 1 ? 1 : (mb > kS2MaxBatch ? kS2MaxBatch : (int)mb);
}

// LDS: tab[mi][p*Wk + q][8][16] for a batch of MB rows, ws[mi][P], and the
// batch's w rows wl[mi][L] (one coalesced copy, so the table build reads LDS).
// WPL: words per lane (>= ceil(P * Wk / 4)).
template <int WPL>
__global__ void __launch_bounds__(kS2Threads)
k_wave_s2(const uint32_t *__restrict__ su2, const uint16_t *__restrict__ h,
          const float *__restrict__ w, int64_t b, int64_t b16, int64_t s, int64_t L, int P,
          int64_t Wk, int M, int MB, uint16_t *__restrict__ y) {
  extern __shared__ float smem[];
  const int t = threadIdx.x, part = t & (kS2Lanes - 1);
  const int nw = P * (int)Wk;
  float *tab = smem;                               // [MB][nw][8][16]
  float *ws = smem + (size_t)MB * nw * 128;        // [MB][2]
  float *wl = ws + (size_t)MB * 2;                 // [MB][L]
  const int64_t j = (int64_t)blockIdx.x * kS2Rows + (t >> 2);
  const int64_t jc = j < b ? j : b - 1;
  // this lane's words (the same for every row m): idx = part + 4 v
  uint32_t wd[WPL];
#pragma unroll
  for (int v = 0; v < WPL; ++v) {
    const int idx = part + kS2Lanes * v;
    wd[v] = idx < nw ? su2[(int64_t)idx * b16 + jc] : 0u;
  }
  float hv[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) hv[p] = p < P ? h2f(h[p * b16 + jc]) : 0.f;
  for (int m0 = 0; m0 < M; m0 += MB) {
    const int mn = (M - m0) < MB ? (M - m0) : MB;
    __syncthreads();  // the previous batch's lookups are done
    {
      const float *src = w + (int64_t)m0 * L;
      const int64_t n = (int64_t)mn * L;
#pragma unroll 4
      for (int64_t i = t; i < n; i += kS2Threads) wl[i] = src[i];
    }
    __syncthreads();
    for (int gi = t; gi < mn * nw * 8; gi += kS2Threads) {
      const int mi = gi / (nw * 8), rem = gi - mi * nw * 8;
      const int idx = rem >> 3, gg = rem & 7;
      const int p = idx / (int)Wk, q = idx - p * (int)Wk;
      const int64_t k0 = (int64_t)q * 32 + 4 * gg;
      const float *wm = wl + (int64_t)mi * L + p * s;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k0 + e < s) ? wm[k0 + e] : 0.f;
      build_table(tab + (size_t)gi * 16, v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    // sum_k w_p[k] of each row: the group totals (entry 15) in order
    if (t < mn * P) {
      const int mi = t / P, p = t - mi * P;
      const float *tb = tab + ((size_t)mi * nw + (size_t)p * Wk) * 128;
      float acc = 0.f;
      for (int gi = 0; gi < (int)Wk * 8; ++gi) acc += tb[gi * 16 + 15];
      ws[mi * 2 + p] = acc;
    }
    __syncthreads();
    for (int mi = 0; mi < mn; ++mi) {
      const float *tb = tab + (size_t)mi * nw * 128;
      float acc[2] = {0.f, 0.f};
#pragma unroll
      for (int v = 0; v < WPL; ++v) {
        const int idx = part + kS2Lanes * v;
        if (idx < nw) {
          const float sum = lut_word(tb + (size_t)idx * 128, wd[v]);
          if (idx < (int)Wk) acc[0] += sum; else acc[1] += sum;
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        acc[p] += __shfl_xor(acc[p], 1, 64);
        acc[p] += __shfl_xor(acc[p], 2, 64);
      }
      if (part == 0 && j < b) {
        float out = 0.f;
        for (int p = 0; p < P; ++p) out += hv[p] * (2.f * acc[p] - ws[mi * 2 + p]);
        y[(int64_t)(m0 + mi) * b + j] = f2h(out);
      }
    }
  }
}

// Fallback for layers whose tables do not fit: one thread per output row.
__global__ void __launch_bounds__(kS2Threads)
k_wave_s2_bits(const uint32_t *__restrict__ su2, const uint16_t *__restrict__ h,
               const float *__restrict__ w, int64_t b, int64_t b16, int64_t s, int64_t L, int P,
               int64_t Wk, int M, uint16_t *__restrict__ y) {
  extern __shared__ float smem[];
  float *wl = smem;           // [L]
  float *ws = smem + L;       // [P]
  float *red = ws + 2;        // [waves]
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int m = 0; m < M; ++m) {
    __syncthreads();
    for (int64_t c = threadIdx.x; c < L; c += blockDim.x) wl[c] = w[(int64_t)m * L + c];
    __syncthreads();
    for (int p = 0; p < P; ++p) {
      float v = 0.f;
      for (int64_t k = threadIdx.x; k < s; k += blockDim.x) v += wl[p * s + k];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0) red[wave] = v;
      __syncthreads();
      if (threadIdx.x == 0) ws[p] = ((red[0] + red[1]) + red[2]) + red[3];
      __syncthreads();
    }
    if (j < b) {
      float out = 0.f;
      for (int p = 0; p < P; ++p) {
        const float *wp = wl + p * s;
        float acc = 0.f;
        for (int64_t q = 0; q < Wk; ++q) {
          const uint32_t wd = su2[(p * Wk + q) * b16 + j];
          const int64_t kb = q * 32;
          const int nb = (s - kb) < 32 ? (int)(s - kb) : 32;
          for (int bit = 0; bit < nb; ++bit) acc += ((wd >> bit) & 1u) ? wp[kb + bit] : 0.f;
        }
        out += h2f(h[p * b16 + j]) * (2.f * acc - ws[p]);
      }
      y[(int64_t)m * b + j] = f2h(out);
    }
  }
}

int wave_nchunk(const Layer &Ly, int64_t M, const DeviceInfo &dev) {
  // Enough chunks to cover the device twice, each at least one row group,
  // and few enough row groups per chunk for one row's tables in LDS.
  (void)M;
  int64_t want = 2LL * (dev.cu_count > 0 ? dev.cu_count : 256);
  if (want > Ly.R1) want = Ly.R1;
  const int64_t gmax = kS1TabFloats / (Ly.P * 8 * 16);
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
  if (Ly.P * G * 8 * 16 > kS1TabFloats) return hipErrorInvalidValue;  // wave_nchunk keeps G small
  const int MB = (int)std::min<int64_t>(M, s1_mbatch(Ly, G));
  const size_t lds = ((size_t)MB * Ly.P * G * 8 * 16 + (size_t)MB * Ly.P + 16) * sizeof(float);
  hipLaunchKernelGGL(k_wave_s1, dim3(nch), dim3(kS1Threads), lds, st, Ly.sv1, Ly.g, x, Ly.a,
                     Ly.a16, Ly.s, Ly.L, Ly.P, Ly.R1, (int)M, G, MB, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = M * Ly.L;
  hipLaunchKernelGGL(k_wave_reduce, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, st, ws, Ly.l,
                     Ly.s, Ly.s8, Ly.L, (int)M, nch, w_out);
  return hipGetLastError();
}

hipError_t launch_wave_stage2(const Layer &Ly, const float *w, uint16_t *y, int64_t M,
                              hipStream_t st) {
  const int nw = (int)(Ly.P * Ly.Wk);
  if (nw <= kS2MaxWords) {
    const int MB = (int)std::min<int64_t>(M, s2_mbatch(nw, Ly.L));
    const size_t lds = ((size_t)MB * nw * 128 + (size_t)MB * 2 + (size_t)MB * Ly.L) * sizeof(float);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((Ly.b + kS2Rows - 1) / kS2Rows));
    const int wpl = (nw + kS2Lanes - 1) / kS2Lanes;
#define LB_S2(WPLV)                                                                       \
  hipLaunchKernelGGL(k_wave_s2<WPLV>, grid, dim3(kS2Threads), lds, st, Ly.su2, Ly.h, w, Ly.b, \
                     Ly.b16, Ly.s, Ly.L, Ly.P, Ly.Wk, (int)M, MB, y)
    if (wpl <= 2) LB_S2(2);
    else if (wpl <= 4) LB_S2(4);
    else if (wpl <= 8) LB_S2(8);
    else if (wpl <= 12) LB_S2(12);
    else LB_S2(24);
#undef LB_S2
    return hipGetLastError();
  }
  const size_t lds = ((size_t)Ly.L + 2 + 16) * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_wave_s2_bits, dim3((unsigned)((Ly.b + kS2Threads - 1) / kS2Threads)),
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
