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
//   tables of z = g_p * x for its rows, then each thread takes items of one
//   latent column c = p*s + k and four rows m:
//   part[chunk][m][c] = 2 * sum_{bit} z - sum z over the chunk (the
//   column's words read once per item).
// Reduce (k_wave_reduce): w = l * sum of the chunk partials, 16 fixed
//   chunk ranges per column combined by a fixed pairwise tree.
// Stage 2 (k_wave_s2): tables of w_p for a batch of rows m (as many as fit
//   the LDS the workgroup's CU can spare, so one build and three barriers
//   serve several rows); eight lanes per output row j split its words
//   (kept in registers for every row) and are summed by a fixed shuffle tree:
//   y[m][j] = fp16(sum_p h_p[j] (2 * sum_{bit} w_p - sum_k w_p[k])).
//   Layers whose tables would not fit (P * ceil(s/32) > 96) use
//   k_wave_s2_bits, one thread per row testing bits one by one.
// Every sum has a fixed order, so results are deterministic.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <atomic>

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

// Entries 4 h .. 4 h + 3 of build_table's table: entry k sums the v_e with
// bit e of k set, added in index order with the first taken as is (the
// same additions as build_table, so the same values bit for bit).
__device__ __forceinline__ float4 table_quarter(float v0, float v1, float v2, float v3, int h) {
  const float lo[4] = {0.f, v0, v1, v0 + v1};  // entries 0-3: the subsets of (v0, v1)
  float o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float acc = lo[j];
    bool any = j != 0;
    if (h & 1) {
      acc = any ? acc + v2 : v2;
      any = true;
    }
    if (h & 2) acc = any ? acc + v3 : v3;
    o[j] = acc;
  }
  return make_float4(o[0], o[1], o[2], o[3]);
}

// Sum of the totals (entry 15) of the first n tables, n a multiple of 8,
// added in table order; the reads go out eight at a time.
__device__ __forceinline__ float sum_totals(const float *tab, int n) {
  float acc = 0.f;
  for (int g0 = 0; g0 < n; g0 += 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tab[(g0 + e) * 16 + 15];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += v[e];
  }
  return acc;
}

// The 32-row sign word of S_V row group r, latent column col: the two
// 16-row tiles 2 r and 2 r + 1 of the tile layout joined.
__device__ __forceinline__ uint32_t sv_word(const uint16_t *__restrict__ sv16, int64_t Lp, int64_t r,
                                            int64_t col) {
  return (uint32_t)sv16[2 * r * Lp + col] | ((uint32_t)sv16[(2 * r + 1) * Lp + col] << 16);
}

// Index of word idx = p * Wk + q of S_U row j in the tile layout (nw = P Wk
// words per row): 16-row tiles of nw * 16 words, row j % 16 innermost.
__device__ __forceinline__ int64_t su_index(int64_t j, int nw, int idx) {
  return (((j >> 4) * nw + idx) << 4) + (j & 15);
}

constexpr int kS1Threads = 512;
constexpr int kS1RowBlock = 4;  // rows m one lookup item covers (its column's words reused)
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
// At most two workgroups of eight waves share a CU (nchunk <= 2 x CUs,
// wave_nchunk), so the compiler may use the registers of four waves per
// SIMD: with the default occupancy target it reused one register for all
// eight table reads of a word and waited for each in turn.
__global__ void __launch_bounds__(kS1Threads) __attribute__((amdgpu_waves_per_eu(1, 4)))
k_wave_s1(const uint16_t *__restrict__ sv16, const uint16_t *__restrict__ g,
          const uint16_t *__restrict__ x, int64_t a, int64_t a16, int64_t s, int64_t L, int64_t Lp, int P,
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
      const uint16_t *gp = g + p * a16, *xp = x + (int64_t)(m0 + mi) * a;
      // the eight loads go out together: indices past the input read its
      // last element and the product is replaced by 0
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e < a ? i0 + e : a - 1;
        v[e] = h2f(gp[i]) * h2f(xp[i]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e >= a) v[e] = 0.f;
      build_table(tab + ((size_t)(mi * P + p) * G * 8 + gr) * 16, v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    for (int idx = t; idx < mn * P; idx += kS1Threads) {
      const float *tb = tab + (size_t)idx * G * 8 * 16;
      sz[idx] = sum_totals(tb, ng);
    }
    __syncthreads();
    // a thread per (column, block of kS1RowBlock rows) item, columns
    // innermost (coalesced stores); the column's words are loaded once per
    // item, before its rows
    const int nrb = (mn + kS1RowBlock - 1) / kS1RowBlock;
    for (int64_t it = t; it < (int64_t)nrb * L; it += kS1Threads) {
      const int rb = (int)((uint64_t)it / (uint64_t)L);
      const int64_t col = it - (int64_t)rb * L;
      const int p = (int)((uint32_t)col / (uint32_t)s);  // col < L = P s <= 8192
      uint32_t wd[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wd[r] = (r0 + r < r1) ? sv_word(sv16, Lp, r0 + r, col) : 0u;
      const int mi1 = min(mn, (rb + 1) * kS1RowBlock);
      for (int mi = rb * kS1RowBlock; mi < mi1; ++mi) {
        const float *tb = tab + (size_t)(mi * P + p) * G * 8 * 16;
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r0 + r < r1) acc += lut_word(tb + r * 8 * 16, wd[r]);
        for (int r = 4; r < (int)(r1 - r0); ++r) acc += lut_word(tb + r * 8 * 16, sv_word(sv16, Lp, r0 + r, col));
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
  // the range's partials are loaded 16 at a time, then added in chunk order
  // (one load waited for at a time would make each add a memory round trip)
  constexpr int kBatch = 16;
  float acc = 0.f;
  if (live)
    for (int cb = c0; cb < c1; cb += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) v[k] = cb + k < c1 ? part[((int64_t)(cb + k) * M + m) * L + col] : 0.f;
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (cb + k < c1) acc += v[k];
    }
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

// The combine of a unit's outputs fused into its last layer's second
// product (k_wave_s2 only): out = fp16(c * (sum of in[u], then this layer)).
struct WaveCombine {
  const uint16_t *in[7];  // the unit's earlier layers' outputs, M x b each
  int n;
  float c;
  uint16_t *out;  // null: no combine
};

constexpr int kS2Threads = 256;
constexpr int kS2Lanes = 4;                        // lanes per output row
constexpr int kS2Rows = kS2Threads / kS2Lanes;     // output rows per workgroup
// k_wave_s2 itself: 8 waves, eight lanes per output row (two waves per
// SIMD hide each other's table-read latency; with four waves and four
// lanes per row the kernel was 7-12% slower on the MLP stacks).
constexpr int kW2Threads = 512, kW2Lanes = 8;
constexpr int kS2MaxWords = 96;                    // P * Wk with tables (48 KB per row m)
constexpr int kS2TabFloats = 12288;                // 48 KB: the least LDS a workgroup is given
constexpr int kS2MaxBatch = 32;
constexpr int kS2WordF = 8 * 16 + 16;  // a word's 8 tables plus a pad, so neighbouring words' tables
                                       // sit on different bank halves
constexpr int kS2LdsCU = 160 * 1024;               // LDS of one CU
constexpr int kS2LdsMax = 150 * 1024;              // the most one workgroup takes

// LDS: tab[mi][p*Wk + q][8][16] for a batch of MB rows, ws[mi][P], and w
// rows wl[.][L]: every row's, copied once at the start (wall), or the
// batch's, copied per batch; the copies are coalesced, so the table build
// reads LDS.  Each batch then costs a table build and three barriers, so
// the launcher gives a workgroup as much LDS as its CU can spare.
// WPL: words per lane (>= ceil(P * Wk / 4)).
template <int WPL>
__global__ void __launch_bounds__(kW2Threads)
k_wave_s2(const uint32_t *__restrict__ su2t, const uint16_t *__restrict__ h,
          const float *__restrict__ w, int64_t b, int64_t b16, int64_t s, int64_t L, int P,
          int64_t Wk, int M, int MB, int wall, uint16_t *__restrict__ y, WaveCombine cb) {
  extern __shared__ float smem[];
  const int t = threadIdx.x, part = t & (kW2Lanes - 1);
  const int nw = P * (int)Wk;
  float *tab = smem;                               // [MB][nw][kS2WordF]: a word's 8 tables, padded
  float *ws = smem + (size_t)MB * nw * kS2WordF;   // [MB][2]
  float *wl = ws + (size_t)MB * 2;                 // [wall ? M : MB][L]
  const int64_t j = (int64_t)blockIdx.x * kS2Rows + (t >> 3);
  const int64_t jc = j < b ? j : b - 1;
  // this lane's words (the same for every row m): idx = part + 4 v
  uint32_t wd[WPL];
#pragma unroll
  for (int v = 0; v < WPL; ++v) {
    const int idx = part + kW2Lanes * v;
    wd[v] = idx < nw ? su2t[su_index(jc, nw, idx)] : 0u;
  }
  float hv[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) hv[p] = p < P ? h2f(h[p * b16 + jc]) : 0.f;
  if (wall) {
    const int64_t n = (int64_t)M * L;
#pragma unroll 4
    for (int64_t i = t; i < n; i += kW2Threads) wl[i] = w[i];
  }
  for (int m0 = 0; m0 < M; m0 += MB) {
    const int mn = (M - m0) < MB ? (M - m0) : MB;
    __syncthreads();  // the previous batch's lookups are done (and the copy of every row landed)
    if (!wall) {
      const float *src = w + (int64_t)m0 * L;
      const int64_t n = (int64_t)mn * L;
#pragma unroll 4
      for (int64_t i = t; i < n; i += kW2Threads) wl[i] = src[i];
      __syncthreads();
    }
    const float *wb = wl + (wall ? (int64_t)m0 * L : 0);  // the batch's first row
    // four threads per table, each storing four entries at once: a wave's
    // stores are 1 KB contiguous (one thread per table put 64 lanes' stores
    // 64 bytes apart, on the same banks)
    for (int gq = t; gq < mn * nw * 8 * 4; gq += kW2Threads) {
      const int gi = gq >> 2, hq = gq & 3;
      const int mi = gi / (nw * 8), rem = gi - mi * nw * 8;
      const int idx = rem >> 3, gg = rem & 7;
      const int p = idx / (int)Wk, q = idx - p * (int)Wk;
      const int64_t k0 = (int64_t)q * 32 + 4 * gg;
      const float *wm = wb + (int64_t)mi * L + p * s;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k0 + e < s) ? wm[k0 + e] : 0.f;
      *reinterpret_cast<float4 *>(tab + ((size_t)mi * nw + idx) * kS2WordF + gg * 16 + 4 * hq) =
          table_quarter(v[0], v[1], v[2], v[3], hq);
    }
    __syncthreads();
    // sum_k w_p[k] of each row: the group totals (entry 15) in order
    if (t < mn * P) {
      const int mi = t / P, p = t - mi * P;
      const float *tb = tab + ((size_t)mi * nw + (size_t)p * Wk) * kS2WordF;
      float acc = 0.f;  // one running sum over every table, in order (as sum_totals)
      for (int q = 0; q < (int)Wk; ++q) {
        const float *tq = tb + (size_t)q * kS2WordF;
        float v8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v8[e] = tq[e * 16 + 15];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += v8[e];
      }
      ws[mi * 2 + p] = acc;
    }
    __syncthreads();
    for (int mi = 0; mi < mn; ++mi) {
      const float *tb = tab + (size_t)mi * nw * kS2WordF;
      float acc[2] = {0.f, 0.f};
#pragma unroll
      for (int v = 0; v < WPL; ++v) {
        const int idx = part + kW2Lanes * v;
        if (idx < nw) {
          const float sum = lut_word(tb + (size_t)idx * kS2WordF, wd[v]);
          if (idx < (int)Wk) acc[0] += sum; else acc[1] += sum;
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        acc[p] += __shfl_xor(acc[p], 1, 64);
        acc[p] += __shfl_xor(acc[p], 2, 64);
        acc[p] += __shfl_xor(acc[p], 4, 64);
      }
      if (part == 0 && j < b) {
        float out = 0.f;
        for (int p = 0; p < P; ++p) out += hv[p] * (2.f * acc[p] - ws[mi * 2 + p]);
        const int64_t o = (int64_t)(m0 + mi) * b + j;
        const uint16_t yv = f2h(out);
        y[o] = yv;
        if (cb.out) {
          // the unit's combine, as k_combine: the fp16 outputs of its layers
          // summed in layer order in fp32, this layer's last, one rounding
          float acc2 = 0.f;
          for (int u = 0; u < cb.n; ++u) acc2 += h2f(cb.in[u][o]);
          acc2 += h2f(yv);
          cb.out[o] = f2h(cb.c * acc2);
        }
      }
    }
  }
}

// Fallback for layers whose tables do not fit: one thread per output row.
__global__ void __launch_bounds__(kS2Threads)
k_wave_s2_bits(const uint32_t *__restrict__ su2t, const uint16_t *__restrict__ h,
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
          const uint32_t wd = su2t[su_index(j, P * (int)Wk, (int)(p * Wk + q))];
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
  hipLaunchKernelGGL(k_wave_s1, dim3(nch), dim3(kS1Threads), lds, st, Ly.sv16, Ly.g, x, Ly.a,
                     Ly.a16, Ly.s, Ly.L, Ly.Lp, Ly.P, Ly.R1, (int)M, G, MB, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = M * Ly.L;
  hipLaunchKernelGGL(k_wave_reduce, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, st, ws, Ly.l,
                     Ly.s, Ly.s8, Ly.L, (int)M, nch, w_out);
  return hipGetLastError();
}

// Stage-2 batching: the LDS a workgroup may take (its CU's share when the
// grid needs several workgroups per CU at once), then rows per batch, with
// every row's w copied once when that costs no extra batch.
static void s2_shape(int nw, int64_t L, int64_t M, int64_t grid, int cus, int *MB, int *wall,
                     size_t *lds) {
  const int64_t per_cu = (grid + cus - 1) / cus;
  const int64_t budget = std::max<int64_t>(kS2TabFloats * 4 + 2048,
                                           std::min<int64_t>(kS2LdsMax, kS2LdsCU / per_cu - 2048));
  const int64_t fl = budget / 4, tab = (int64_t)nw * kS2WordF + 2;
  const int64_t cap = std::min<int64_t>(M, kS2MaxBatch);
  const int64_t mb_b = std::max<int64_t>(1, std::min<int64_t>(cap, fl / (tab + L)));  // per-batch copies
  const int64_t mb_a = std::min<int64_t>(cap, (fl - M * L) / tab);                   // every row once
  if (mb_a >= 1 && (M + mb_a - 1) / mb_a <= (M + mb_b - 1) / mb_b) {
    *MB = (int)mb_a;
    *wall = 1;
    *lds = ((size_t)mb_a * tab + (size_t)M * L) * sizeof(float);
  } else {
    *MB = (int)mb_b;
    *wall = 0;
    *lds = ((size_t)mb_b * (tab + L)) * sizeof(float);
  }
}

// Stage-2 workgroups may take more than 64 KB of LDS: allowed once per
// device for every instance.
static hipError_t s2_lds_attr(int device) {
  static std::atomic<uint64_t> done{0};
  const uint64_t bit = device >= 0 && device < 64 ? (1ull << device) : 0;
  if (bit && (done.load() & bit)) return hipSuccess;
  const void *k[5] = {(const void *)k_wave_s2<2>, (const void *)k_wave_s2<4>, (const void *)k_wave_s2<8>,
                      (const void *)k_wave_s2<12>, (const void *)k_wave_s2<24>};
  hipError_t e = hipSuccess;
  for (int i = 0; i < 5 && e == hipSuccess; ++i)
    e = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, kS2LdsMax);
  if (e == hipSuccess && bit) done.fetch_or(bit);
  return e;
}

bool wave_stage2_combines(const Layer &Ly) { return Ly.P * Ly.Wk <= kS2MaxWords; }

hipError_t launch_wave_stage2(const Layer &Ly, const float *w, uint16_t *y, int64_t M,
                              const DeviceInfo &dev, hipStream_t st, const uint16_t *const *cin,
                              int ncin, float c, uint16_t *cout) {
  const int nw = (int)(Ly.P * Ly.Wk);
  if (nw <= kS2MaxWords) {
    hipError_t ea = s2_lds_attr(dev.device);
    if (ea != hipSuccess) return ea;
    const int64_t nblk = (Ly.b + kS2Rows - 1) / kS2Rows;
    int MB = 1, wall = 0;
    size_t lds = 0;
    s2_shape(nw, Ly.L, M, nblk, dev.cu_count > 0 ? dev.cu_count : 256, &MB, &wall, &lds);
    if (lds > (size_t)kS2LdsMax) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk);
    const int wpl = (nw + kW2Lanes - 1) / kW2Lanes;
    WaveCombine cb{};
    if (cout) {
      if (ncin < 0 || ncin > 7) return hipErrorInvalidValue;
      for (int u = 0; u < ncin; ++u) cb.in[u] = cin[u];
      cb.n = ncin;
      cb.c = c;
      cb.out = cout;
    }
#define LB_S2(WPLV)                                                                       \
  hipLaunchKernelGGL(k_wave_s2<WPLV>, grid, dim3(kW2Threads), lds, st, Ly.su2t, Ly.h, w, Ly.b, \
                     Ly.b16, Ly.s, Ly.L, Ly.P, Ly.Wk, (int)M, MB, wall, y, cb)
    if (wpl <= 2) LB_S2(2);
    else if (wpl <= 4) LB_S2(4);
    else if (wpl <= 8) LB_S2(8);
    else if (wpl <= 12) LB_S2(12);
    else LB_S2(24);
#undef LB_S2
    return hipGetLastError();
  }
  if (cout) return hipErrorInvalidValue;  // see wave_stage2_combines
  const size_t lds = ((size_t)Ly.L + 2 + 16) * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_wave_s2_bits, dim3((unsigned)((Ly.b + kS2Threads - 1) / kS2Threads)),
                     dim3(kS2Threads), lds, st, Ly.su2t, Ly.h, w, Ly.b, Ly.b16, Ly.s, Ly.L, Ly.P,
                     Ly.Wk, (int)M, y);
  return hipGetLastError();
}

// --------------------------------------------------------- one launch, M = 1
// The three steps above in one launch for a single row of a small layer
// (at most 16 input chunks and 256 latent columns; the 4096^2 projections).
// Workgroups take roles by ticket (an atomic counter taken as each
// workgroup starts):
//   [0, N1)        first product of input chunk c (as k_wave_s1), the chunk
//                  partial of every latent column stored tagged;
//   [N1, N1 + N2)  64 output rows (as k_wave_s2): each sums the N1 <= 16
//                  partials of every column itself, a thread per column, in
//                  the reduction's order (16 chunk ranges, then a fixed
//                  pairwise tree), applies l and goes on as k_wave_s2.
// Larger layers take the three launches: with hundreds of workgroups in
// one launch the waiting output blocks hold CU slots that the roles they
// wait for need (some start tens of us late), and the separate launches
// are faster (17 against 27 us for 8192 -> 28672, s = 302).
// A role waits only for lower tickets, held by workgroups that have already
// started, so the launch completes however many workgroups are resident (no
// co-residency needed; another stream's kernels can share the device).
// Words carry (fp32 bits | generation << 32); the generation is the one the
// previous launch finished with, plus 1, and the last workgroup to finish
// resets the ticket for the next launch.  Every wait is bounded and sets a
// host-mapped error word when it gives up.
struct Forward1Args {
  const uint16_t *sv16;
  const uint32_t *su2t;
  const uint16_t *g, *h, *l, *x;
  uint16_t *y;
  int64_t a, a16, b, b16, s, s8, L, Lp, R1, Wk;
  int P, G, N1, N2;
  unsigned *ctrl;  // one 64-bit word: the launch's generation (high half), the next ticket (low half)
  uint64_t *part;  // [N1][L] tagged chunk partials
  unsigned *herr;  // host-mapped: set when a wait gives up
};

constexpr int kF1Threads = 512;  // eight waves: two per SIMD
constexpr int kF1MaxL = 256;      // latent columns (one thread pair each in the first product)
constexpr int kF1Lanes = 8;       // lanes per output row
constexpr long kF1Spin = 1L << 24;
constexpr int kF1MaxChunks = 16;  // first-product chunks (one partial each per column)

// Up to N words at p(k), k < n, polled together (every pending word read in
// each round), values into v[k].
template <int N, class Ptr>
__device__ __forceinline__ void f1_wait_n(Ptr p, int n, unsigned gen, float (&v)[N], unsigned *herr) {
  unsigned pend = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    v[k] = 0.f;
    if (k < n) pend |= 1u << k;
  }
  for (long it = 0; pend && it < kF1Spin; ++it) {
    uint64_t wd[N];
#pragma unroll
    for (int k = 0; k < N; ++k)
      wd[k] = ((pend >> k) & 1u) ? __hip_atomic_load(p(k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (((pend >> k) & 1u) && (unsigned)(wd[k] >> 32) == gen) {
        v[k] = __uint_as_float((unsigned)wd[k]);
        pend &= ~(1u << k);
      }
  }
  if (pend) __hip_atomic_store(herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void f1_put(uint64_t *p, float v, unsigned gen) {
  __hip_atomic_store(p, (uint64_t)__float_as_uint(v) | ((uint64_t)gen << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

template <int WPL>
__global__ void __launch_bounds__(kF1Threads) k_forward1(Forward1Args A) {
  extern __shared__ float smem[];
  __shared__ unsigned s_tk, s_gen;
  const int t = threadIdx.x;
  // the workgroup that draws the last ticket moves the word to the next
  // generation with the count at 0: every workgroup of this launch has
  // drawn by then, and the next launch (stream-ordered) starts from there,
  // so no workgroup has to count finishers at the end
  if (t == 0) {
    unsigned long long *tw = reinterpret_cast<unsigned long long *>(A.ctrl);
    const unsigned long long old = __hip_atomic_fetch_add(tw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned tk = (unsigned)old, g = (unsigned)(old >> 32);
    if (tk == (unsigned)(A.N1 + A.N2) - 1u)
      __hip_atomic_store(tw, (unsigned long long)(g + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_tk = tk;
    s_gen = g + 1u;
  }
  __syncthreads();
  const int tk = (int)s_tk;
  const unsigned gen = s_gen;
  const int64_t L = A.L;
  if (tk < A.N1) {
    // first product over row groups [c G, c G + G) of the input
    const int c = tk;
    const int64_t r0 = (int64_t)c * A.G, r1 = min(r0 + A.G, A.R1);
    const int ng = (int)(r1 - r0) * 8;
    float *tab = smem;                                  // [P][G*8][16]
    float *sz = smem + (size_t)A.P * A.G * 8 * 16;      // [P]
    float *half1 = sz + 16;                             // [kF1MaxL]
    const int nr = (int)(r1 - r0);
    // four threads per table, four entries each (one 16-byte store)
    for (int gq = t; gq < A.P * ng * 4; gq += kF1Threads) {
      const int idx = gq >> 2, hq = gq & 3;
      const int p = idx / ng, gr = idx - p * ng;
      const int64_t i0 = r0 * 32 + 4 * gr;
      const uint16_t *gp = A.g + p * A.a16;
      float v[4];  // loads issued together, as in k_wave_s1
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e < A.a ? i0 + e : A.a - 1;
        v[e] = h2f(gp[i]) * h2f(A.x[i]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e >= A.a) v[e] = 0.f;
      *reinterpret_cast<float4 *>(tab + ((size_t)p * A.G * 8 + gr) * 16 + 4 * hq) =
          table_quarter(v[0], v[1], v[2], v[3], hq);
    }
    __syncthreads();
    if (t < A.P) {
      sz[t] = sum_totals(tab + (size_t)t * A.G * 8 * 16, ng);
    }
    __syncthreads();
    // two threads per column (L <= kF1MaxL), each on half of the chunk's row
    // groups; the second half's sum is added to the first's
    const int col = t & (kF1MaxL - 1), hf = t / kF1MaxL, rh = (nr + 1) / 2;
    const int ra = hf * rh, rb = min(nr, ra + rh);
    float acc = 0.f;
    int p = 0;
    if (col < L) {
      p = (int)((uint32_t)col / (uint32_t)A.s);
      const float *tb = tab + (size_t)p * A.G * 8 * 16;
      for (int r = ra; r < rb; ++r) acc += lut_word(tb + r * 8 * 16, sv_word(A.sv16, A.Lp, r0 + r, col));
      if (hf) half1[col] = acc;
    }
    __syncthreads();
    if (hf == 0 && col < L) f1_put(&A.part[(size_t)c * L + col], 2.f * (acc + half1[col]) - sz[p], gen);
  } else {
    // output rows [64 j, 64 j + 64): eight lanes per row split its words
    const int part = t & (kF1Lanes - 1), nw = A.P * (int)A.Wk;
    float *tab = smem;                         // [nw][8][16]
    float *wsum = smem + (size_t)nw * 128;     // [2]
    float *wl = wsum + 2;                      // [L]
    const int64_t j = (int64_t)(tk - A.N1) * kS2Rows + (t >> 3);
    const int64_t jc = j < A.b ? j : A.b - 1;
    uint32_t wd[WPL];
#pragma unroll
    for (int v = 0; v < WPL; ++v) {
      const int idx = part + kF1Lanes * v;
      wd[v] = idx < nw ? A.su2t[su_index(jc, nw, idx)] : 0u;
    }
    float hv[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) hv[p] = p < A.P ? h2f(A.h[p * A.b16 + jc]) : 0.f;
    // thread t sums column t over the N1 <= 16 chunks as ranges of one
    // chunk and the pairwise tree, then applies l
    if (t < L) {
      float v[kF1MaxChunks];
      f1_wait_n([&](int k) { return &A.part[(size_t)k * L + t]; }, A.N1, gen, v, A.herr);
#pragma unroll
      for (int o = kF1MaxChunks / 2; o >= 1; o >>= 1)
#pragma unroll
        for (int g = 0; g < o; ++g) v[g] += v[g + o];
      const int p = (int)((uint32_t)t / (uint32_t)A.s);
      wl[t] = h2f(A.l[p * A.s8 + (t - p * A.s)]) * v[0];
    }
    __syncthreads();
    for (int gq = t; gq < nw * 8 * 4; gq += kF1Threads) {
      const int gi = gq >> 2, hq = gq & 3;
      const int idx = gi >> 3, gg = gi & 7;
      const int p = idx / (int)A.Wk, qq = idx - p * (int)A.Wk;
      const int64_t k0 = (int64_t)qq * 32 + 4 * gg;
      const float *wm = wl + p * A.s;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k0 + e < A.s) ? wm[k0 + e] : 0.f;
      *reinterpret_cast<float4 *>(tab + (size_t)gi * 16 + 4 * hq) = table_quarter(v[0], v[1], v[2], v[3], hq);
    }
    __syncthreads();
    if (t < A.P) {
      wsum[t] = sum_totals(tab + (size_t)t * A.Wk * 128, (int)A.Wk * 8);
    }
    __syncthreads();
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int v = 0; v < WPL; ++v) {
      const int idx = part + kF1Lanes * v;
      if (idx < nw) {
        const float sum = lut_word(tab + (size_t)idx * 128, wd[v]);
        if (idx < (int)A.Wk) acc[0] += sum; else acc[1] += sum;
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      acc[p] += __shfl_xor(acc[p], 1, 64);
      acc[p] += __shfl_xor(acc[p], 2, 64);
      acc[p] += __shfl_xor(acc[p], 4, 64);
    }
    if (part == 0 && j < A.b) {
      float out = 0.f;
      for (int p = 0; p < A.P; ++p) out += hv[p] * (2.f * acc[p] - wsum[p]);
      A.y[j] = f2h(out);
    }
  }
}

// Sizes of the one-launch forward, or false when the layer is outside it
// (more than 16 chunks or 256 latent columns, or tables beyond its LDS).
bool forward1_plan(const Layer &Ly, Forward1Plan *pl) {
  const int nw = Ly.P * (int)Ly.Wk;
  // small layers only: at most 16 chunks of at most 8 row groups, L <= 256
  if (nw > kS2MaxWords || Ly.L > kF1MaxL || (Ly.R1 + kF1MaxChunks - 1) / kF1MaxChunks > 8) return false;
  const int nch = (int)std::min<int64_t>(kF1MaxChunks, Ly.R1);
  const int G = (int)((Ly.R1 + nch - 1) / nch);
  pl->G = G;
  pl->N1 = (int)((Ly.R1 + G - 1) / G);
  pl->N2 = (int)((Ly.b + kS2Rows - 1) / kS2Rows);
  pl->wpl = (nw + kF1Lanes - 1) / kF1Lanes;
  const size_t l1 = ((size_t)Ly.P * G * 8 * 16 + 16 + kF1MaxL + 16) * sizeof(float);
  const size_t l2 = ((size_t)nw * 128 + 2 + Ly.L + 16) * sizeof(float);
  pl->lds = std::max(l1, l2);
  pl->state_bytes = 256 + (size_t)pl->N1 * Ly.L * 8;
  return pl->lds <= 64 * 1024;
}

hipError_t launch_forward1(const Layer &Ly, const Forward1Plan &pl, void *state, unsigned *herr,
                           const uint16_t *x, uint16_t *y, hipStream_t st) {
  Forward1Args A;
  A.sv16 = Ly.sv16; A.su2t = Ly.su2t; A.g = Ly.g; A.h = Ly.h; A.l = Ly.l; A.x = x; A.y = y;
  A.a = Ly.a; A.a16 = Ly.a16; A.b = Ly.b; A.b16 = Ly.b16; A.s = Ly.s; A.s8 = Ly.s8; A.L = Ly.L; A.Lp = Ly.Lp;
  A.R1 = Ly.R1; A.Wk = Ly.Wk; A.P = Ly.P;
  A.G = pl.G; A.N1 = pl.N1; A.N2 = pl.N2;
  unsigned char *base = static_cast<unsigned char *>(state);
  A.ctrl = reinterpret_cast<unsigned *>(base);
  A.part = reinterpret_cast<uint64_t *>(base + 256);
  A.herr = herr;
  const dim3 grid((unsigned)(pl.N1 + pl.N2));
#define LB_F1(WPLV) hipLaunchKernelGGL(k_forward1<WPLV>, grid, dim3(kF1Threads), pl.lds, st, A)
  if (pl.wpl <= 2) LB_F1(2);
  else if (pl.wpl <= 4) LB_F1(4);
  else if (pl.wpl <= 8) LB_F1(8);
  else LB_F1(12);  // nw <= kS2MaxWords = 96
#undef LB_F1
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
