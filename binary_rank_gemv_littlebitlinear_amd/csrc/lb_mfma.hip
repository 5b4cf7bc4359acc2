// MFMA path (used for M >= 64 rows of x), one "unit" per pair of launches.
//
// With many rows of x the two binary products of [LB news] Sec. 2 are
// real dense contractions, so they run on the fp16 matrix cores.  A unit
// is a group of layers that read the same input (one layer for a plain
// forward; q/k/v or gate/up in a stack).  Per unit:
//
//   stage 1: T[M x Lt] = x[M x a] . B1[a x Lt],  B1[i][col(m,p,k)] = S_V,mp[i,k] * g_mp[i]
//   stage 2: y_m[M x b] = fp16( sum_p h_mp * ( T_mp[M x s] . B2_mp[s x b] ) ),
//            B2_mp[k][j] = S_U,mp[j,k] * l_mp[k]
//            and, in a stack, x_next = fp16(c_out * sum_m y_m) in the same
//            epilogue.
//
// +-g and +-l are exact in fp16 (a sign flip of the stored scale), so the
// only rounding of an operand is T -> fp16, once.  Accumulation is fp32.
// The sign bits are expanded in registers right before the MFMA that uses
// them: a lane's 8 operand values are 8 stored scales with the fp16 sign
// bit flipped where the sign is -1.
//
// Latent columns: every (layer m, path p) owns a segment of T of s
// columns rounded up to 32; padding columns are exactly zero.  T is kept
// in a tiled layout so that one wave's operand load is 1 KB contiguous:
//   T[((tok / 32) * (Lt / 8) + col / 8) * 256 + (tok % 32) * 8 + col % 8].
//
// Instruction: v_mfma_f32_32x32x16_f16.  Operand lanes: A[i][k] in lane
// i + 32 * (k / 8), element k % 8; B[k][j] in lane j + 32 * (k / 8),
// element k % 8; D[i][j] in lane j + 32 * ((i / 4) % 2), register
// 4 * (i / 8) + i % 4.
//
// Stage 1 computes 32 x 128 tiles (each of 4 waves owns 32 columns, so no
// cross-wave sum); stage 2 computes 32 x 64 tiles with the 4 waves
// interleaved over the (path, 32-column) chunks of K and their partials
// summed in wave order through LDS.  Each workgroup copies its operands
// into LDS with LDS-DMA in rounds (x or T rows, sign words and the
// per-k scales g or l), the next round in flight while the current one
// is multiplied.  Stage 1 also splits K across workgroups when the tiles
// alone cannot fill the chip; the last workgroup of a tile to finish (an
// atomic counter per tile) sums the partials in split order, so the
// result does not depend on timing.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <vector>

#include "lb_internal.h"

namespace lbi {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kMaxSplit = 8;
// stage 1: a workgroup computes 32 rows x 128 latent columns (32 per wave);
// a round stages kRC1 32-row chunks of the input dimension in LDS
constexpr int kRC1 = 14;
constexpr int kS1X = kRC1 * 4 * 512;   // x rows: [c8][32 rows][8 fp16]
constexpr int kS1W = 4 * kRC1 * 128;   // sign words: [wave][chunk][32 columns]
constexpr int kS1G = 4 * 1024;         // column scales g: [wave][16 chunks][32 rows]
constexpr int kS1Buf = kS1X + kS1W + kS1G;
// stage 2: a workgroup computes 32 rows x 64 outputs; a round stages kRC2
// (path, 32-column) chunks of one layer's latent rows and sign words
constexpr int kRC2 = 28;
constexpr int kS2T = kRC2 * 4 * 512;   // T rows: [c8][32 rows][8 fp16]
constexpr int kS2W = kRC2 * 256;       // sign words: [chunk][64 outputs]
constexpr int kS2L = 32 * 64;          // latent scales l: [chunk][32] (2 instructions of 16 chunks)
constexpr int kS2Buf = kS2T + kS2W + kS2L;
constexpr int kRP2 = 64 + 4;           // LDS pitch (floats) of a wave's 32 x 64 partial
static_assert(4 * 32 * kRP2 * 4 <= kS2Buf, "the reduction buffer fits one round buffer");
static_assert(kRC1 % 2 == 0 && kRC1 <= 16, "stage-1 round: two chunks of words, 16 of g per instruction");
static_assert(kRC2 <= 32, "stage-2 round: l of 16 chunks per instruction, two instructions");

struct S1Seg {
  const uint32_t *bits;  // sv1m + p*s: word (row group r, column k) at bits[r * pitch + k]
  const uint16_t *g;     // g + p*a16
  int pitch;             // latent columns L of the layer
  int s;                 // valid columns of the segment
  int seg0;              // first column of the segment in T (multiple of 32)
  int pad_;
};
static_assert(sizeof(S1Seg) == 32, "S1Seg layout");

struct S1Args {
  const uint16_t *x;
  uint16_t *T;
  float *part;
  unsigned *cnt;
  const void *zero;  // >= 16 zero bytes (DMA source for padding)
  int64_t M;         // rows of this chunk
  int a, a16, Lt, ntile32, kcps, nsplit, nseg, xvec;
  S1Seg seg[kMaxUnitSegs];
};

struct S2Layer {
  const uint32_t *su2;  // su2m (matrix-core bit order)
  const uint16_t *l;
  const uint16_t *h;
  uint16_t *y;  // per-layer output (may be null)
  int b16, s8, Wk, P, seg0[2], pad_[2];
};
static_assert(sizeof(S2Layer) == 64, "S2Layer layout");

struct S2Args {
  const uint16_t *T;
  uint16_t *xout;  // combined output (stack) or null
  const void *zero;
  int64_t M;
  int b, Lt, nl, direct;
  float c_out;
  int nrounds;
  S2Layer ly[kMaxUnitLayersM];
};

struct MfmaPlan {
  int nl = 0;
  int64_t a = 0, b = 0;
  int a16 = 0, Lt = 0, ntile32 = 0, nseg = 0, nrounds2 = 0;
  S1Seg seg[kMaxUnitSegs];
  S2Layer ly[kMaxUnitLayersM];
};

// ----------------------------------------------------------- primitives
__device__ __forceinline__ float mh2f(uint16_t v) { return __half2float(__ushort_as_half(v)); }
__device__ __forceinline__ uint16_t mf2h(float v) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ void st_rel(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_rel(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte stores / loads with the cache policy of relaxed agent-scope
// atomics (sc1: coherent across the device's L2s), through a buffer
// resource over [base, base + bytes)
constexpr int kCoherent = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// LDS-DMA: lane i's 16 (4) source bytes land at dst + 16 i (dst + 4 i).
__device__ __forceinline__ void dma16(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

__device__ __forceinline__ half8_t as_h8(u32x4 v) { return __builtin_bit_cast(half8_t, v); }

// Flip the fp16 signs of a lane's 8 operand values: wl is its sign word
// in the matrix-core bit order, already shifted left by 4 g for the lane's
// group g of 8 elements, so (wl << j) & 0x80008000 flips elements 2 j, 2 j + 1.
__device__ __forceinline__ u32x4 flip_signs(u32x4 v, uint32_t wl) {
  v.x ^= wl & 0x80008000u;
  v.y ^= (wl << 1) & 0x80008000u;
  v.z ^= (wl << 2) & 0x80008000u;
  v.w ^= (wl << 3) & 0x80008000u;
  return v;
}

__device__ __forceinline__ uint4 pack8(const float *v) {
  uint4 o;
  o.x = mf2h(v[0]) | ((uint32_t)mf2h(v[1]) << 16);
  o.y = mf2h(v[2]) | ((uint32_t)mf2h(v[3]) << 16);
  o.z = mf2h(v[4]) | ((uint32_t)mf2h(v[5]) << 16);
  o.w = mf2h(v[6]) | ((uint32_t)mf2h(v[7]) << 16);
  return o;
}

// 8 fp16 to row-major [rows x n] at (row, col..col+7), columns >= n dropped.
__device__ __forceinline__ void store8(uint16_t *base, int n, int64_t row, int col, const float *v) {
  uint16_t *dst = base + row * n + col;
  if ((n & 7) == 0 && col + 8 <= n) {
    *reinterpret_cast<uint4 *>(dst) = pack8(v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (col + e < n) dst[e] = mf2h(v[e]);
  }
}

// ------------------------------------------------------------- stage 1
// grid = (Lt / 128, ceil(M / 32), nsplit).  Block (cx, ty, z) computes
// columns [128 cx, 128 cx + 128) of rows [32 ty, 32 ty + 32) over the
// 32-row chunks [z * kcps, (z + 1) * kcps) of the input dimension; wave w
// owns columns 32 w .. 32 w + 31 of the block.  Rows past M and columns
// past the last segment come out as zeros, so every element of T that
// the second stage reads is written.
__global__ void __launch_bounds__(kThreads)
k_unit_s1(S1Args A) {
  extern __shared__ __align__(16) unsigned char smem[];  // 2 round buffers
  __shared__ int s_last;
  const int w = wave_id(), lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const int t32 = blockIdx.x * 4 + w;
  const int64_t tok0 = (int64_t)blockIdx.y * 32;

  // the wave's 32 columns lie in one segment
  const bool active = t32 < A.ntile32;
  bool cval = false, full_cols = false;
  const uint32_t *bb = nullptr;
  const uint16_t *gb = nullptr;
  int pitch = 0;
  if (active) {
    int e = 0;
    for (int q = 1; q < A.nseg; ++q)
      if (t32 * 32 >= A.seg[q].seg0) e = q;
    const int k = t32 * 32 - A.seg[e].seg0 + lr;
    cval = k < A.seg[e].s;
    full_cols = t32 * 32 - A.seg[e].seg0 + 32 <= A.seg[e].s;  // uniform
    bb = A.seg[e].bits + k;
    gb = A.seg[e].g;
    pitch = A.seg[e].pitch;
  }
  const int nkc = (A.a + 31) >> 5;
  const int kc0 = blockIdx.z * A.kcps;
  const int kc1 = min(nkc, kc0 + A.kcps);
  const int nr = (kc1 - kc0 + kRC1 - 1) / kRC1;

  // round r: chunks [kc0 + r kRC1, +nch) of x rows (all waves) and of the
  // wave's sign words, into buffer r & 1
  auto issue = [&](int r) {
    unsigned char *buf = smem + (r & 1) * kS1Buf;
    const int kcr = kc0 + r * kRC1, nch = min(kRC1, kc1 - kcr);
    if (A.xvec) {
      for (int u = w; u < nch * 2; u += 4) {
        const int c8 = 2 * u + lh;
        const int64_t tok = tok0 + lr;
        const int i = kcr * 32 + c8 * 8;
        const void *src = (tok < A.M && i < A.a) ? (const void *)(A.x + tok * A.a + i) : A.zero;
        dma16(src, buf + u * 1024);
      }
    } else {
      for (int idx = threadIdx.x; idx < nch * 4 * 32; idx += kThreads) {
        const int c8 = idx >> 5, row = idx & 31;
        const int64_t tok = tok0 + row;
        const int i = kcr * 32 + c8 * 8;
        uint32_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (tok < A.M && i + e < A.a) ? A.x[tok * A.a + i + e] : 0u;
        uint4 o;
        o.x = hv[0] | (hv[1] << 16); o.y = hv[2] | (hv[3] << 16);
        o.z = hv[4] | (hv[5] << 16); o.w = hv[6] | (hv[7] << 16);
        *reinterpret_cast<uint4 *>(buf + idx * 16) = o;
      }
    }
    if (active) {
      for (int v = 0; v < (nch + 1) / 2; ++v) {
        const int kk = 2 * v + lh;
        const void *src = (cval && kk < nch) ? (const void *)(bb + (size_t)(kcr + kk) * pitch) : A.zero;
        dma4(src, buf + kS1X + (w * kRC1 + 2 * v) * 128);
      }
      // g of the chunks: lane = 4 chunk + piece, 8 rows per piece
      const int kk = lane >> 2, i = (kcr + kk) * 32 + 8 * (lane & 3);
      const void *src = (kk < nch && i + 8 <= A.a16) ? (const void *)(gb + i) : A.zero;
      dma16(src, buf + kS1X + kS1W + w * 1024);
    }
  };

  // two accumulators (even / odd chunks) keep two independent MFMA chains
  float16_t acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  issue(0);
  for (int r = 0; r < nr; ++r) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of round r landed
    __syncthreads();                // ... and every other wave's
    if (r + 1 < nr) issue(r + 1);   // overlaps the products below
    if (!active) continue;
    const unsigned char *buf = smem + (r & 1) * kS1Buf;
    const int kcr = kc0 + r * kRC1, nch = min(kRC1, kc1 - kcr);
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(buf);
    const uint32_t *wsd = reinterpret_cast<const uint32_t *>(buf + kS1X) + w * kRC1 * 32;
    const u32x4 *gsd = reinterpret_cast<const u32x4 *>(buf + kS1X + kS1W + w * 1024);
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    // operands of one chunk: x rows (A), g (B values before the signs), words
    struct Ops { u32x4 a[2], g[2]; uint32_t wd; };
    auto fetch = [&](int kk, Ops &o) {
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        o.a[step] = xs[(kk * 4 + 2 * step + lh) * 32 + lr];
        o.g[step] = gsd[kk * 4 + 2 * step + lh];  // g of rows 32 kk + 16 step + 8 lh ..
      }
      o.wd = wsd[kk * 32 + lr];
    };
    auto mma = [&](const Ops &o, float16_t &acc, auto masked) {
      const uint32_t wl = o.wd << (4 * lh);  // group g = 2 step + lh
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        u32x4 bv = flip_signs(o.g[step], wl << (8 * step));
        if (decltype(masked)::value && !cval) bv = z4;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(o.a[step]), as_h8(bv), acc, 0, 0, 0);
      }
    };
    // the prefetches are unconditional (index clamped) so the wait before a
    // chunk's products covers only that chunk's reads
    auto sweep = [&](auto masked) {
      Ops c0, c1;
      fetch(0, c0);
      fetch(min(1, nch - 1), c1);
      for (int kk = 0; kk < nch; kk += 2) {
        Ops n0, n1;
        fetch(min(kk + 2, nch - 1), n0);
        fetch(min(kk + 3, nch - 1), n1);
        mma(c0, acc0, masked);
        if (kk + 1 < nch) mma(c1, acc1, masked);
        c0 = n0;
        c1 = n1;
      }
    };
    if (full_cols)
      sweep(std::false_type());
    else
      sweep(std::true_type());
  }
  __syncthreads();  // the round buffers are free

  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = acc0[r] + acc1[r];
  if (A.nsplit > 1) {
    // split z's partial: registers 4q..4q+3 of lane l of wave w as one
    // 16-byte word at [(tile*nsplit + z)*1024 + (4 w + q)*64 + l] (float4 units)
    const __amdgpu_buffer_rsrc_t rs =
        coherent_rsrc(A.part + (size_t)tile * A.nsplit * 4096, (uint32_t)A.nsplit * 16384u);
    const int o0 = blockIdx.z * 16384 + ((w * 4) * 64 + lane) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 o;
      o.x = __float_as_uint(v[4 * q]); o.y = __float_as_uint(v[4 * q + 1]);
      o.z = __float_as_uint(v[4 * q + 2]); o.w = __float_as_uint(v[4 * q + 3]);
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, o0 + q * 1024, 0, kCoherent);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned old =
          __hip_atomic_fetch_add(&A.cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (unsigned)(A.nsplit - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // the last block of the tile sums the splits in split order; every load
    // is unconditional (splits past nsplit re-read the last one) so all of
    // them are in flight at once
    u32x4 q[kMaxSplit][4];
    const int l0 = ((w * 4) * 64 + lane) * 16;
#pragma unroll
    for (int z = 0; z < kMaxSplit; ++z)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        q[z][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, min(z, A.nsplit - 1) * 16384 + l0 + j * 1024, 0,
                                                        kCoherent);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sum = __uint_as_float(q[0][j][e]);
#pragma unroll
        for (int z = 1; z < kMaxSplit; ++z)
          if (z < A.nsplit) sum += __uint_as_float(q[z][j][e]);
        v[4 * j + e] = sum;
      }
    if (threadIdx.x == 0) __hip_atomic_store(&A.cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // fp16 tile [16 c8][32 rows][8] in LDS, then one contiguous 8 KB copy into T
  uint16_t *tl = reinterpret_cast<uint16_t *>(smem);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * lh + (r & 3), col = w * 32 + lr;
    tl[((col >> 3) * 32 + row) * 8 + (col & 7)] = mf2h(v[r]);
  }
  __syncthreads();
  uint4 *dst = reinterpret_cast<uint4 *>(A.T + ((size_t)blockIdx.y * (A.Lt >> 3) + blockIdx.x * 16) * 256);
  const uint4 *srcl = reinterpret_cast<const uint4 *>(smem);
  dst[threadIdx.x] = srcl[threadIdx.x];
  dst[threadIdx.x + kThreads] = srcl[threadIdx.x + kThreads];
}

// ------------------------------------------------------------- stage 2
// grid = (ceil(b / 64), ceil(M / 32)).  Block (jx, ty) computes outputs
// [64 jx, 64 jx + 64) of rows [32 ty, 32 ty + 32) for every layer of the
// unit, then their combine.  The waves interleave over a layer's
// (path, 32-column) chunks, each wave accumulating 32 x 64 per path; the
// four partials are summed in wave order through LDS.
__global__ void __launch_bounds__(kThreads)
k_unit_s2(S2Args A) {
  extern __shared__ __align__(16) unsigned char smem[];  // 2 round buffers
  const int w = wave_id(), lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const int t = threadIdx.x;
  const int tb = blockIdx.y;
  const int64_t tok0 = (int64_t)tb * 32;
  const int j0 = blockIdx.x * 64;
  const int Lt8 = A.Lt >> 3;

  // round r -> (layer m, first chunk ch0, chunk count nch); chunk ch of a
  // layer is path ch / Wk, 32-column block ch % Wk
  auto round_of = [&](int r, int &m, int &ch0, int &nch) {
    m = 0;
    int rr = r;
    while (true) {
      const int nc = A.ly[m].P * A.ly[m].Wk;
      const int nrm = (nc + kRC2 - 1) / kRC2;
      if (rr < nrm) {
        ch0 = rr * kRC2;
        nch = min(kRC2, nc - ch0);
        return;
      }
      rr -= nrm;
      ++m;
    }
  };
  auto issue = [&](int r) {
    int m, ch0, nch;
    round_of(r, m, ch0, nch);
    const S2Layer &Ly = A.ly[m];
    unsigned char *buf = smem + (r & 1) * kS2Buf;
    const uint16_t *tsrc = A.T + ((size_t)tb * Lt8 + (Ly.seg0[0] >> 3) + ch0 * 4) * 256;
    for (int u = w; u < nch * 2; u += 4) dma16(tsrc + u * 512 + lane * 8, buf + u * 1024);
    for (int v = w; v < (nch + 3) / 4; v += 4) {
      const int chl = 4 * v + (lane >> 4);
      const int j = j0 + 4 * (lane & 15);
      const void *src = (chl < nch && j + 4 <= Ly.b16)
                            ? (const void *)(Ly.su2 + (size_t)(ch0 + chl) * Ly.b16 + j)
                            : A.zero;
      dma16(src, buf + kS2T + v * 1024);
    }
    // l of the chunks: lane = 4 chunk + piece, 8 latent columns per piece
    for (int v = w; v < (nch + 15) / 16; v += 4) {
      const int chl = 16 * v + (lane >> 2);
      const int ch = ch0 + chl;
      const int p = ch >= Ly.Wk ? 1 : 0;
      const int k = (ch - p * Ly.Wk) * 32 + 8 * (lane & 3);
      const void *src = (chl < nch && k + 8 <= Ly.s8) ? (const void *)(Ly.l + (size_t)p * Ly.s8 + k) : A.zero;
      dma16(src, buf + kS2T + kS2W + v * 1024);
    }
  };

  float ys[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ys[e] = 0.f;
  const int row_o = t >> 3, c_o = 8 * (t & 7);  // this thread's 8 outputs per layer
  issue(0);
  int r = 0;
  for (int m = 0; m < A.nl; ++m) {
    const S2Layer &Ly = A.ly[m];
    const int nc = Ly.P * Ly.Wk, nrm = (nc + kRC2 - 1) / kRC2;
    float hv[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int j = j0 + ni * 32 + lr;
        hv[p][ni] = (p < Ly.P && j < A.b) ? mh2f(Ly.h[(size_t)p * Ly.b16 + j]) : 0.f;
      }
    float16_t acc0[2], acc1[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc0[ni][e] = acc1[ni][e] = 0.f;
    for (int rm = 0; rm < nrm; ++rm, ++r) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (r + 1 < A.nrounds) issue(r + 1);
      const unsigned char *buf = smem + (r & 1) * kS2Buf;
      const int ch0 = rm * kRC2, nch = min(kRC2, nc - ch0);
      const u32x4 *ts = reinterpret_cast<const u32x4 *>(buf);
      const uint32_t *wsd = reinterpret_cast<const uint32_t *>(buf + kS2T);
      const u32x4 *lsd = reinterpret_cast<const u32x4 *>(buf + kS2T + kS2W);
      struct Ops { u32x4 a[2], l[2]; uint32_t wd[2]; };
      auto fetch = [&](int chl, Ops &o) {
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          o.a[step] = ts[(chl * 4 + 2 * step + lh) * 32 + lr];
          o.l[step] = lsd[chl * 4 + 2 * step + lh];  // l of columns 32 q + 16 step + 8 lh ..
        }
        o.wd[0] = wsd[chl * 64 + lr];
        o.wd[1] = wsd[chl * 64 + 32 + lr];
      };
      auto mma = [&](const Ops &o, float16_t (&acc)[2]) {
        const uint32_t wl0 = o.wd[0] << (4 * lh), wl1 = o.wd[1] << (4 * lh);  // group g = 2 step + lh
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          const half8_t av = as_h8(o.a[step]);
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              av, as_h8(flip_signs(o.l[step], wl0 << (8 * step))), acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              av, as_h8(flip_signs(o.l[step], wl1 << (8 * step))), acc[1], 0, 0, 0);
        }
      };
      // chunks are path-major: [0, nch0) are path 0, [nch0, nch) path 1;
      // wave w takes the chunks chl = w (mod 4), path by path
      const int nch0 = max(0, min(nch, Ly.Wk - ch0));
      auto run = [&](int lo, int hi, float16_t (&acc)[2]) {
        int chl = lo + ((w - lo) % 4 + 4) % 4;
        if (chl >= hi) return;
        Ops c;
        fetch(chl, c);
        for (; chl < hi; chl += 4) {
          Ops n;
          fetch(min(chl + 4, hi - 1), n);  // unconditional: see stage 1
          mma(c, acc);
          c = n;
        }
      };
      run(0, nch0, acc0);
      run(nch0, nch, acc1);
    }
    // layer epilogue: the layer's last round buffer becomes the reduction area
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem + ((r - 1) & 1) * kS2Buf);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * lh + (e & 3), col = ni * 32 + lr;
        red[(w * 32 + row) * kRP2 + col] = hv[0][ni] * acc0[ni][e] + hv[1][ni] * acc1[ni][e];
      }
    __syncthreads();
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int o = row_o * kRP2 + c_o + e;
      v[e] = ((red[o] + red[32 * kRP2 + o]) + red[2 * 32 * kRP2 + o]) + red[3 * 32 * kRP2 + o];
      v[e] = mh2f(mf2h(v[e]));  // the layer's fp16 output
      ys[e] += v[e];
    }
    if (Ly.y && tok0 + row_o < A.M) store8(Ly.y, A.b, tok0 + row_o, j0 + c_o, v);
  }
  if (A.direct || !A.xout || tok0 + row_o >= A.M) return;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = A.c_out * ys[e];
  store8(A.xout, A.b, tok0 + row_o, j0 + c_o, o);
}

// ------------------------------------------------------------------ host
static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
static constexpr size_t kS1Lds = (size_t)2 * kS1Buf;
static constexpr size_t kS2Lds = (size_t)2 * kS2Buf;

MfmaPlan *mfma_plan_build(const Layer *const *layers, int n) {
  if (n < 1 || n > kMaxUnitLayersM) return nullptr;
  MfmaPlan *P = new MfmaPlan();
  P->nl = n;
  P->a = layers[0]->a;
  P->b = layers[0]->b;
  P->a16 = (int)layers[0]->a16;
  int col = 0, nseg = 0, nr2 = 0;
  for (int m = 0; m < n; ++m) {
    const Layer &Ly = *layers[m];
    if (Ly.a != P->a || Ly.b != P->b) {
      delete P;
      return nullptr;
    }
    S2Layer &D = P->ly[m];
    D.su2 = Ly.su2m; D.l = Ly.l; D.h = Ly.h; D.y = nullptr;
    D.b16 = (int)Ly.b16; D.s8 = (int)Ly.s8; D.Wk = (int)Ly.Wk; D.P = Ly.P;
    D.seg0[0] = D.seg0[1] = 0;
    D.pad_[0] = D.pad_[1] = 0;
    for (int p = 0; p < Ly.P; ++p) {
      S1Seg &S = P->seg[nseg++];
      S.bits = Ly.sv1m + (size_t)p * Ly.s;
      S.g = Ly.g + (size_t)p * Ly.a16;
      S.pitch = (int)Ly.L;
      S.s = (int)Ly.s;
      S.seg0 = col;
      S.pad_ = 0;
      D.seg0[p] = col;
      col += (int)round_up(Ly.s, 32);
    }
    nr2 += (int)((Ly.P * Ly.Wk + kRC2 - 1) / kRC2);
  }
  P->nseg = nseg;
  P->ntile32 = col / 32;
  P->Lt = (int)round_up(col, 128);
  P->nrounds2 = nr2;
  return P;
}

void mfma_plan_free(MfmaPlan *p) { delete p; }

static int64_t s1_tiles(const MfmaPlan &P, int64_t Mc) { return (int64_t)(P.Lt / 128) * ((Mc + 31) / 32); }

static int s1_nsplit(const MfmaPlan &P, int64_t Mc, const DeviceInfo &dev, int *kcps) {
  const int64_t tiles = s1_tiles(P, Mc);
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int nkc = (int)((P.a + 31) / 32);
  int ns = (int)std::min<int64_t>(kMaxSplit, std::max<int64_t>(1, (cus + tiles - 1) / tiles));
  ns = std::min(ns, nkc);
  const int k = (nkc + ns - 1) / ns;
  *kcps = k;
  return (nkc + k - 1) / k;
}

size_t mfma_unit_ws_bytes(const MfmaPlan *p) {
  const size_t T = (size_t)round_up((int64_t)kMfmaRows * p->Lt * 2, 256);
  const size_t part = (size_t)kMaxSplit * s1_tiles(*p, kMfmaRows) * 4096 * sizeof(float);
  return T + part;
}

size_t mfma_cnt_entries(const MfmaPlan *p) { return (size_t)s1_tiles(*p, kMfmaRows); }

static hipError_t set_lds_attr(int device) {
  static std::atomic<uint64_t> done{0};
  const uint64_t bit = device >= 0 && device < 64 ? (1ull << device) : 0;
  if (bit && (done.load() & bit)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void *)k_unit_s1,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kS1Lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void *)k_unit_s2, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kS2Lds);
  if (e == hipSuccess && bit) done.fetch_or(bit);
  return e;
}

hipError_t launch_mfma_unit(const MfmaPlan *p, const uint16_t *x, int64_t M,
                            uint16_t *const *y_layers, uint16_t *xout, float c_out, bool direct,
                            void *ws, unsigned *cnt, const void *zero, const DeviceInfo &dev,
                            hipStream_t st) {
  hipError_t e = set_lds_attr(dev.device);
  if (e != hipSuccess) return e;
  uint16_t *T = reinterpret_cast<uint16_t *>(ws);
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) +
                                          round_up((int64_t)kMfmaRows * p->Lt * 2, 256));
  for (int64_t mb = 0; mb < M; mb += kMfmaRows) {
    const int64_t Mc = std::min<int64_t>(kMfmaRows, M - mb);
    S1Args A1;
    A1.x = x + mb * p->a;
    A1.T = T;
    A1.part = part;
    A1.cnt = cnt;
    A1.zero = zero;
    A1.M = Mc;
    A1.a = (int)p->a;
    A1.a16 = p->a16;
    A1.Lt = p->Lt;
    A1.ntile32 = p->ntile32;
    A1.nsplit = s1_nsplit(*p, Mc, dev, &A1.kcps);
    A1.nseg = p->nseg;
    A1.xvec = (p->a % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    for (int i = 0; i < kMaxUnitSegs; ++i) A1.seg[i] = p->seg[i];
    dim3 g1((unsigned)(p->Lt / 128), (unsigned)((Mc + 31) / 32), (unsigned)A1.nsplit);
    hipLaunchKernelGGL(k_unit_s1, g1, dim3(kThreads), kS1Lds, st, A1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    S2Args A2;
    A2.T = T;
    A2.xout = xout ? xout + mb * p->b : nullptr;
    A2.zero = zero;
    A2.M = Mc;
    A2.b = (int)p->b;
    A2.Lt = p->Lt;
    A2.nl = p->nl;
    A2.direct = direct ? 1 : 0;
    A2.c_out = c_out;
    A2.nrounds = p->nrounds2;
    for (int m = 0; m < kMaxUnitLayersM; ++m) {
      A2.ly[m] = p->ly[m];
      A2.ly[m].y = (m < p->nl && y_layers && y_layers[m]) ? y_layers[m] + mb * p->b : nullptr;
    }
    dim3 g2((unsigned)((p->b + 63) / 64), (unsigned)((Mc + 31) / 32));
    hipLaunchKernelGGL(k_unit_s2, g2, dim3(kThreads), kS2Lds, st, A2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lbi
