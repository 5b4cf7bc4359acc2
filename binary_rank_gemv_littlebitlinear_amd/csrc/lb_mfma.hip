// MFMA path (used for M >= 64 rows of x), one "unit" per pair of launches.
//
// With many rows of x the two binary products of [LB news] Sec. 2 are
// real dense contractions, so they run on the fp16 matrix cores.  A unit
// is a group of layers that read the same input (one layer for a plain
// forward; q/k/v or gate/up in a stack).  Per unit:
//
//   stage 1: T[M x Lt] = fp16( (x[M x a] . B1[a x Lt]) * l ),
//            B1[i][col(m,p,k)] = S_V,mp[i,k] * g_mp[i], l = l_mp[k] of the column
//   stage 2: y_m[M x b] = fp16( sum_p h_mp * ( T_mp[M x s] . B2_mp[s x b] ) ),
//            B2_mp[k][j] = S_U,mp[j,k]  (+-1)
//            and, in a stack, x_next = fp16(c_out * sum_m y_m) in the same
//            epilogue.
//
// +-g and +-1 are exact in fp16 (a sign flip of the stored scale, or of
// 1.0), so the only rounding of an operand is l * t -> fp16, once.
// Accumulation is fp32.  The sign bits are expanded in registers right
// before the MFMA that uses them: a lane's 8 operand values are 8 stored
// scales (or 1.0) with the fp16 sign bit set where the sign is -1.
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
// Stage 1 computes 32 x 128 tiles with 8 waves (two per 32 columns, on
// the even and the odd input chunks) and requests a split's whole operand
// range at once when it fits in LDS.  Stage 2 computes 32 x 64 nb tiles
// (nb = 1, 2 or 4), the waves interleaved over the (path, 32-column) chunks
// of K and their partials summed in a fixed order through LDS.  Each
// workgroup copies its operands into LDS with LDS-DMA (x or T rows, sign
// words, and g in stage 1).  Stage 1 also splits K across workgroups (one
// per CU); the last workgroup of a tile to finish (an atomic counter per
// tile) sums the partials in split order, so the result does not depend
// on timing.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <map>
#include <new>
#include <string>
#include <type_traits>
#include <vector>

#include "lb_internal.h"

namespace lbi {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads1 = 512;  // 8 waves (first stage)
constexpr int kMaxSplit = 8;
// stage 1: a workgroup computes 32 rows x 128 latent columns (32 per wave)
// over a range of 32-row chunks of the input dimension.  A round stages up
// to C chunks at once (C even, at most kS1MaxC): x rows, and per wave its
// columns' sign words and the chunks' scales g.
constexpr int kS1MaxC = 56;
constexpr int kS1RoundC = 14;  // chunks per round when a split takes several (two buffers)
__host__ __device__ constexpr int s1_c16(int C) { return (C + 15) & ~15; }
__host__ __device__ constexpr int s1_words_off(int C) { return C * 2048; }
__host__ __device__ constexpr int s1_g_off(int C) { return C * 2048 + 4 * C * 128; }
__host__ __device__ constexpr int s1_lds_bytes(int C) { return s1_g_off(C) + 4 * s1_c16(C) * 64; }
static_assert(s1_lds_bytes(kS1MaxC) <= 160 * 1024, "a stage-1 round fits the LDS");
static_assert(2 * s1_lds_bytes(kS1RoundC) <= 80 * 1024, "two buffered rounds leave room for two blocks per CU");
// stage 2: a workgroup computes 32 rows x 64 nb outputs; a round stages
// up to kRC2 (path, 32-column) chunks of one layer's latent rows and sign
// words (two round buffers)
constexpr int kRC2 = 32;  // a multiple of 4
constexpr int kS2MinC = 18;            // the wave partials fit one round buffer from here
constexpr int kS2Lds = 158 * 1024;  // leaves room for the static LDS of the one-launch stack
constexpr int kRP2 = 64 + 4;           // LDS pitch (floats) of a wave's 32 x 64 partial
static_assert(4 * 32 * kRP2 * 4 <= kS2MinC * 2048, "the reduction buffer fits one round buffer");
// with 8 waves (nb = 2 or 4) the partials need 8 * 32 rows: they fit the
// round buffer of the chunk counts s2_shape picks for those widths

struct S1Seg {
  const uint32_t *bits;  // sv1m + p*s: word (row group r, column k) at bits[r * pitch + k]
  const uint16_t *g;     // g + p*a16
  int pitch;             // latent columns L of the layer
  int s;                 // valid columns of the segment
  int seg0;              // first column of the segment in T (multiple of 32)
  int pad_;
  const uint16_t *l;     // l + p*s8: the latent scale folded into T
};
static_assert(sizeof(S1Seg) == 40, "S1Seg layout");

struct alignas(16) S1Args {
  const uint16_t *x;
  uint16_t *T;
  float *part;
  unsigned *cnt;
  const void *zero;  // >= 16 zero bytes (DMA source for padding)
  int64_t M;         // rows of this chunk
  int a, a16, Lt, ntile32, kcps, cround, nsplit, nseg, xvec;
  // addressing: x row pitch (elements), T row-block pitch (8-column
  // blocks), tiles per row block and split slots per tile of part / cnt
  int xpitch, tp8, tstride, psplit;
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

struct alignas(16) S2Args {
  const uint16_t *T;
  uint16_t *xout;  // combined output (stack) or null
  const void *zero;
  int64_t M;
  int b, Lt, nl, direct;
  float c_out;
  int nrounds;
  int nb;  // 64-output column pairs per block (1, 2 or 4)
  int c2;  // chunks per round
  int tp8, opitch;  // T row-block pitch (8-column blocks), xout row pitch
  S2Layer ly[kMaxUnitLayersM];
};

struct MfmaPlan {
  int nl = 0;
  int64_t a = 0, b = 0;
  int a16 = 0, Lt = 0, ntile32 = 0, nseg = 0;
  S1Seg seg[kMaxUnitSegs];  // sign pointers filled at launch (seg_layer, seg_path)
  S2Layer ly[kMaxUnitLayersM];
  const Layer *src[kMaxUnitLayersM] = {};
  int seg_layer[kMaxUnitSegs] = {}, seg_path[kMaxUnitSegs] = {};
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
// The same for data another workgroup of the running launch wrote: the
// device-scope cache policy, so no stale L2 line of this XCD is returned.
template <bool kCoh>
__device__ __forceinline__ void dma16c(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kCoh ? kCoherent : 0);
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

// The lane's 8 operand values +-1 (fp16) from its sign word, same bit
// convention as flip_signs: bit set = -1.
__device__ __forceinline__ u32x4 sign_ones(uint32_t wl) {
  u32x4 v;
  v.x = (wl & 0x80008000u) | 0x3C003C00u;
  v.y = ((wl << 1) & 0x80008000u) | 0x3C003C00u;
  v.z = ((wl << 2) & 0x80008000u) | 0x3C003C00u;
  v.w = ((wl << 3) & 0x80008000u) | 0x3C003C00u;
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

// 8 fp16 to [rows x n] (row pitch `pitch`) at (row, col..col+7), columns
// >= n dropped, with device-scope stores (read by other workgroups of the
// running launch).  rs covers the whole output.
__device__ __forceinline__ void store8c(__amdgpu_buffer_rsrc_t rs, int n, int pitch, int64_t row, int col,
                                        const float *v) {
  const int off = (int)((row * pitch + col) * 2);
  if ((n & 7) == 0 && (pitch & 7) == 0 && col + 8 <= n) {
    const uint4 o = pack8(v);
    u32x4 q;
    q.x = o.x; q.y = o.y; q.z = o.z; q.w = o.w;
    __builtin_amdgcn_raw_buffer_store_b128(q, rs, off, 0, kCoherent);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (col + e < n) __builtin_amdgcn_raw_buffer_store_b16(mf2h(v[e]), rs, off + 2 * e, 0, kCoherent);
  }
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
// 32-row chunks [z * kcps, (z + 1) * kcps) of the input dimension.  Waves
// w and w + 4 own columns 32 w .. 32 w + 31 of the block, the even and the
// odd chunks respectively; their sums are added in that order, then each
// finishes half of the tile's values.  Rows past M and columns
// past the last segment come out as zeros, so every element of T that
// the second stage reads is written.
//
// All of a round's operands are requested at once; a round is the block's
// whole chunk range when it fits (up to kS1MaxC chunks), so the copies run
// at the full depth the memory system allows.  Longer ranges go in rounds
// of kS1RoundC chunks through two buffers, the next round's copies
// overlapping this round's products.  LDS layout of a round of C chunks:
//   x      [chunk][row 32][4 pieces of 8 fp16], piece c8 of row r stored in
//          slot c8 ^ swz(r): one copy instruction reads 16 rows x 64 bytes,
//          and the operand reads (32 rows, one piece) hit distinct banks
//   words  [wave][chunk C][32 columns]
//   g      [wave][chunk c16(C)][4 pieces of 8 fp16]
__device__ __forceinline__ int s1_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// The argument structs may be read through a constant-address-space view
// (AT), so that uniform fields load into scalar registers.
typedef __attribute__((address_space(4))) const S1Args CS1Args;
typedef __attribute__((address_space(4))) const S2Args CS2Args;

// Tile (bx, by, bz) of a grid with gx tiles across; kCoh: x comes from
// and T goes to other workgroups of the running launch (device-scope
// loads and stores).  dep() is a workgroup-wide call, true once x may be
// read; with kCoh the first round's sign words and g are requested before
// it (M = 128 stack 2.79 -> 2.72 ms), its x rows after it.  Returns 1 when this block completed the tile (the only
// split, or the last of its splits: then its T values are stored), 0 when
// another split completes it, -1 when dep() returned false.
template <bool kCoh, class AT, class Dep>
__device__ __forceinline__ int s1_tile(AT &A, const uint16_t *xp, int bx, int by, int bz,
                                       unsigned char *smem, int *s_last, Dep &&dep) {
  const int w = wave_id(), lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const int tw = w & 3, par = w >> 2;  // column tile, chunk parity
  const int t32 = bx * 4 + tw;
  const int64_t tok0 = (int64_t)by * 32;

  // the tile's 32 columns lie in one segment
  const bool active = t32 < A.ntile32;
  bool cval = false, full_cols = false;
  float lcol = 0.f;  // l of the lane's column (0 past the segment)
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
    if (cval) lcol = mh2f(A.seg[e].l[k]);
  }
  const int nkc = (A.a + 31) >> 5;
  const int kc0 = bz * A.kcps;
  const int kc1 = min(nkc, kc0 + A.kcps);
  const int C = A.cround;
  const int nr = (kc1 - kc0 + C - 1) / C;
  const int wofs = s1_words_off(C), gofs = s1_g_off(C), c16 = s1_c16(C);

  // round r: chunks [kc0 + r C, +nch) of x rows (all waves), and of the
  // tile's sign words and g (waves 0-3, one tile each)
  auto issue_x = [&](unsigned char *buf, int kcr, int nch) {
    if (A.xvec) {
      // instruction u: chunk u / 2, rows 16 (u & 1) + lane / 4
      const int rw = lane >> 2;
      for (int u = w; u < nch * 2; u += kThreads1 / 64) {
        const int row = 16 * (u & 1) + rw;
        const int c8 = (lane & 3) ^ s1_swz(row);
        const int64_t tok = tok0 + row;
        const int i = (kcr + (u >> 1)) * 32 + c8 * 8;
        const void *src = (tok < A.M && i < A.a) ? (const void *)(xp + tok * A.xpitch + i) : A.zero;
        dma16c<kCoh>(src, buf + u * 1024);
      }
    } else {
      for (int idx = threadIdx.x; idx < nch * 128; idx += kThreads1) {
        const int kk = idx >> 7, row = (idx >> 2) & 31;
        const int c8 = (idx & 3) ^ s1_swz(row);
        const int64_t tok = tok0 + row;
        const int i = (kcr + kk) * 32 + c8 * 8;
        uint32_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = (tok < A.M && i + e < A.a) ? xp[tok * A.xpitch + i + e] : 0u;
        uint4 o;
        o.x = hv[0] | (hv[1] << 16); o.y = hv[2] | (hv[3] << 16);
        o.z = hv[4] | (hv[5] << 16); o.w = hv[6] | (hv[7] << 16);
        *reinterpret_cast<uint4 *>(buf + idx * 16) = o;
      }
    }
  };
  auto issue_w = [&](unsigned char *buf, int kcr, int nch) {
    if (active && par == 0) {
      // words: lanes 0-31 chunk 2 v, lanes 32-63 chunk 2 v + 1 (C is even)
      for (int v = 0; v < (nch + 1) / 2; ++v) {
        const int kk = 2 * v + lh;
        const void *src = (cval && kk < nch) ? (const void *)(bb + (size_t)(kcr + kk) * pitch) : A.zero;
        dma4(src, buf + wofs + (tw * C + 2 * v) * 128);
      }
      // g: lane = 4 chunk + piece, 16 chunks per instruction
      for (int v = 0; v < (nch + 15) / 16; ++v) {
        const int kk = 16 * v + (lane >> 2), i = (kcr + kk) * 32 + 8 * (lane & 3);
        const void *src = (kk < nch && i + 8 <= A.a16) ? (const void *)(gb + i) : A.zero;
        dma16(src, buf + gofs + (tw * c16 + 16 * v) * 64);
      }
    }
  };
  auto issue = [&](int r) {
    unsigned char *buf = smem + (r & 1) * s1_lds_bytes(C);
    const int kcr = kc0 + r * C, nch = min(C, kc1 - kcr);
    issue_x(buf, kcr, nch);
    issue_w(buf, kcr, nch);
  };

  // chunks of the wave's parity alternate between two accumulators, so two
  // independent MFMA chains interleave
  float16_t acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  const int xo0 = lr * 4 + (lh ^ s1_swz(lr)), xo1 = lr * 4 + ((2 + lh) ^ s1_swz(lr));
  const int bstride = s1_lds_bytes(C);  // rounds alternate between two buffers when there are several
  if constexpr (kCoh) {
    const int nch0 = min(C, kc1 - kc0);
    issue_w(smem, kc0, nch0);
    if (!dep()) {
      __builtin_amdgcn_s_waitcnt(0);  // the copies land before the LDS is left
      return -1;
    }
    issue_x(smem, kc0, nch0);
  } else {
    // a launch of its own: x first (measured faster there)
    if (!dep()) return -1;
    issue(0);
  }
  for (int r = 0; r < nr; ++r) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of round r landed
    __syncthreads();                // ... and every other wave's
    if (r + 1 < nr) issue(r + 1);   // overlaps the products below
    if (!active) continue;
    const unsigned char *buf = smem + (r & 1) * bstride;
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(buf);
    const uint32_t *wsd = reinterpret_cast<const uint32_t *>(buf + wofs) + tw * C * 32;
    const u32x4 *gsd = reinterpret_cast<const u32x4 *>(buf + gofs) + tw * c16 * 4;
    const int nch = min(C, kc1 - kc0 - r * C);
    if (par >= nch) continue;
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    // operands of one chunk: x rows (A), g (B values before the signs), words
    struct Ops { u32x4 a[2], g[2]; uint32_t wd; };
    auto fetch = [&](int kk, Ops &o) {
      o.a[0] = xs[kk * 128 + xo0];
      o.a[1] = xs[kk * 128 + xo1];
#pragma unroll
      for (int step = 0; step < 2; ++step) o.g[step] = gsd[kk * 4 + 2 * step + lh];  // rows 32 kk + 16 step + 8 lh ..
      o.wd = wsd[kk * 32 + lr];
    };
    auto bvals = [&](const Ops &o, u32x4 (&bv)[2], auto masked) {
      const uint32_t wl = o.wd << (4 * lh);  // group g = 2 step + lh
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        bv[step] = flip_signs(o.g[step], wl << (8 * step));
        if (decltype(masked)::value && !cval) bv[step] = z4;
      }
    };
    // the prefetches are unconditional (index clamped) so the wait before a
    // chunk's products covers only that chunk's reads
    auto sweep = [&](auto masked) {
      Ops c0, c1;
      fetch(par, c0);
      fetch(min(par + 2, nch - 1), c1);
      for (int kk = par; kk < nch; kk += 4) {
        Ops n0, n1;
        fetch(min(kk + 4, nch - 1), n0);
        fetch(min(kk + 6, nch - 1), n1);
        u32x4 b0[2], b1[2];
        bvals(c0, b0, masked);
        if (kk + 2 < nch) {
          bvals(c1, b1, masked);
#pragma unroll
          for (int step = 0; step < 2; ++step) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(c0.a[step]), as_h8(b0[step]), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(c1.a[step]), as_h8(b1[step]), acc1, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int step = 0; step < 2; ++step)
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(c0.a[step]), as_h8(b0[step]), acc0, 0, 0, 0);
        }
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
  // the pair (w, w + 4) splits the tile's 16 registers: wave w finishes
  // 0-7, wave w + 4 finishes 8-15, each adding parity 0's sum to parity 1's
  const int r0 = 8 * par;
  float v[8];
  {
    float *red = reinterpret_cast<float *>(smem);
    float lo[8], hi[8];  // sums of registers 0-7 and 8-15 (constant indices: no scratch)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      lo[r] = acc0[r] + acc1[r];
      hi[r] = acc0[8 + r] + acc1[8 + r];
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)  // the partner's half
      red[((par * 4 + tw) * 8 + r) * 64 + lane] = par == 0 ? hi[r] : lo[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float other = red[(((1 - par) * 4 + tw) * 8 + r) * 64 + lane];
      v[r] = par == 0 ? lo[r] + other : other + hi[r];
    }
    __syncthreads();  // red is free again
  }

  const int tile = by * A.tstride + bx;
  if (A.nsplit > 1) {
    // split z's partial: registers 4q..4q+3 of lane l of tile tw as one
    // 16-byte word at [(tile*nsplit + z)*1024 + (4 tw + q)*64 + l] (float4
    // units); wave (tw, par) holds q = 2 par, 2 par + 1
    const __amdgpu_buffer_rsrc_t rs =
        coherent_rsrc(A.part + (size_t)tile * A.psplit * 4096, (uint32_t)A.nsplit * 16384u);
    const int l0 = ((tw * 4 + 2 * par) * 64 + lane) * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 o;
      o.x = __float_as_uint(v[4 * q]); o.y = __float_as_uint(v[4 * q + 1]);
      o.z = __float_as_uint(v[4 * q + 2]); o.w = __float_as_uint(v[4 * q + 3]);
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, bz * 16384 + l0 + q * 1024, 0, kCoherent);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned old =
          __hip_atomic_fetch_add(&A.cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = old == (unsigned)(A.nsplit - 1);
    }
    __syncthreads();
    if (!*s_last) return 0;
    // the last block of the tile sums the splits in split order; every load
    // is unconditional (splits past nsplit re-read the last one) so all of
    // them are in flight at once
    u32x4 q[kMaxSplit][2];
#pragma unroll
    for (int z = 0; z < kMaxSplit; ++z)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        q[z][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, min(z, A.nsplit - 1) * 16384 + l0 + j * 1024, 0,
                                                        kCoherent);
#pragma unroll
    for (int j = 0; j < 2; ++j)
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
  for (int r = 0; r < 8; ++r) {
    const int rr = r0 + r;
    const int row = 8 * (rr >> 2) + 4 * lh + (rr & 3), col = tw * 32 + lr;
    tl[((col >> 3) * 32 + row) * 8 + (col & 7)] = mf2h(v[r] * lcol);
  }
  __syncthreads();
  uint4 *dst = reinterpret_cast<uint4 *>(A.T + ((size_t)by * A.tp8 + bx * 16) * 256);
  const uint4 *srcl = reinterpret_cast<const uint4 *>(smem);
  if (kCoh) {
    const uint4 o = srcl[threadIdx.x];
    u32x4 q;
    q.x = o.x; q.y = o.y; q.z = o.z; q.w = o.w;
    __builtin_amdgcn_raw_buffer_store_b128(q, coherent_rsrc(dst, 8192u), threadIdx.x * 16, 0, kCoherent);
  } else {
    dst[threadIdx.x] = srcl[threadIdx.x];
  }
  return 1;
}

__global__ void __launch_bounds__(kThreads1)
k_unit_s1(S1Args A) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_last;
  (void)s1_tile<false>(A, A.x, blockIdx.x, blockIdx.y, blockIdx.z, smem, &s_last, [] { return true; });
}

// ------------------------------------------------------------- stage 2
// grid = (ceil(b / (64 nb)), ceil(M / 32)).  Block (jx, ty) computes
// outputs [64 nb jx, 64 nb (jx + 1)) of rows [32 ty, 32 ty + 32) for every
// layer of the unit, then their combine.  T already carries l (the first
// stage folds it in), so the B operand is the +-1 signs of S_U alone.
// NW waves (4 or 8): wave w works on column pair cp = w % nb (64 outputs,
// two 32-column tiles) and takes the layer's (path, 32-column) chunks of
// phase w / nb (mod NW / nb), accumulating 32 x 64 per path; the phase
// partials of a pair are summed in phase order through LDS.  With 8 waves
// two share each SIMD, so one's sign expansion overlaps the other's MFMAs.
// LDS round buffer of C chunks (C a multiple of 4): T rows
// [chunk][c8 4][32 rows][8 fp16], then the sign words [pair][chunk][64 outputs].
__host__ __device__ constexpr int s2_buf_bytes(int C, int nb) { return C * 2048 + nb * C * 256; }

// Tile (bx, by); kCoh: T comes from and xout goes to other workgroups of
// the running launch (device-scope loads and stores).  dep() is a
// workgroup-wide call, true once T may be read; with kCoh the first round's
// sign words are requested before it, its T rows after it.  False when
// dep() returned false.
template <int NB, int NW, bool kCoh, class AT, class Dep>
__device__ __forceinline__ bool s2_tile(AT &A, uint16_t *xout, int bx, int by, unsigned char *smem,
                                        Dep &&dep) {
  const int w = wave_id(), lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const int t = threadIdx.x;
  constexpr int nb = NB, nph = NW / NB;
  const int C = A.c2;
  const int cp = w % nb, phase = w / nb;
  const int tb = by;
  const int64_t tok0 = (int64_t)tb * 32;
  const int j0 = bx * 64 * nb;
  const int Lt8 = A.tp8;
  const int bufb = s2_buf_bytes(C, nb), wofs = C * 2048;

  // round r -> (layer m, first chunk ch0, chunk count nch); chunk ch of a
  // layer is path ch / Wk, 32-column block ch % Wk
  auto round_of = [&](int r, int &m, int &ch0, int &nch) {
    m = 0;
    int rr = r;
    while (true) {
      const int nc = A.ly[m].P * A.ly[m].Wk;
      const int nrm = (nc + C - 1) / C;
      if (rr < nrm) {
        ch0 = rr * C;
        nch = min(C, nc - ch0);
        return;
      }
      rr -= nrm;
      ++m;
    }
  };
  auto issue_t = [&](int r, int m, int ch0, int nch) {
    auto &Ly = A.ly[m];
    unsigned char *buf = smem + (r & 1) * bufb;
    const uint16_t *tsrc = A.T + ((size_t)tb * Lt8 + (Ly.seg0[0] >> 3) + ch0 * 4) * 256;
    // the blocks of a row tile all read the same T rows: each starts at its
    // own place in the list so they do not queue on the same lines
    const int nu = nch * 2, u0 = (bx * 4) % nu;
    for (int i = w; i < nu; i += NW) {
      const int u = u0 + i < nu ? u0 + i : u0 + i - nu;
      dma16c<kCoh>(tsrc + u * 512 + lane * 8, buf + u * 1024);
    }
  };
  auto issue_w = [&](int r, int m, int ch0, int nch) {
    auto &Ly = A.ly[m];
    unsigned char *buf = smem + (r & 1) * bufb;
    // words: instruction (pair q, v) covers chunks 4 v .. 4 v + 3 of pair q
    const int nv = (nch + 3) / 4;
    for (int iv = w; iv < nb * nv; iv += NW) {
      const int q = iv / nv, v = iv - q * nv;
      const int chl = 4 * v + (lane >> 4);
      const int j = j0 + q * 64 + 4 * (lane & 15);
      const void *src = (chl < nch && j + 4 <= Ly.b16)
                            ? (const void *)(Ly.su2 + (size_t)(ch0 + chl) * Ly.b16 + j)
                            : A.zero;
      dma16(src, buf + wofs + (q * C + 4 * v) * 256);
    }
  };
  auto issue = [&](int r) {
    int m, ch0, nch;
    round_of(r, m, ch0, nch);
    issue_t(r, m, ch0, nch);
    issue_w(r, m, ch0, nch);
  };

  // outputs of thread t: row t / 8, columns q * 64 + 8 (t % 8) .. + 7 of each pair q
  float ys[NB][8];
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) ys[q][e] = 0.f;
  const int row_o = t >> 3, c_o = 8 * (t & 7);
  if constexpr (kCoh) {
    int m0, ch00, nch0;
    round_of(0, m0, ch00, nch0);
    issue_w(0, m0, ch00, nch0);
    if (!dep()) {
      __builtin_amdgcn_s_waitcnt(0);  // the copies land before the LDS is left
      return false;
    }
    issue_t(0, m0, ch00, nch0);
  } else {
    // a launch of its own: T first (measured faster there)
    if (!dep()) return false;
    issue(0);
  }
  int r = 0;
  for (int m = 0; m < A.nl; ++m) {
    auto &Ly = A.ly[m];
    const int nc = Ly.P * Ly.Wk, nrm = (nc + C - 1) / C;
    // h of the wave's columns; the loads are unconditional (clamped index)
    // so no wait for them lands before the round's copies are needed
    float hv[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int j = j0 + cp * 64 + ni * 32 + lr;
        const uint16_t hraw = Ly.h[(size_t)min(p, Ly.P - 1) * Ly.b16 + min(j, Ly.b16 - 1)];
        hv[p][ni] = (p < Ly.P && j < A.b) ? mh2f(hraw) : 0.f;
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
      const unsigned char *buf = smem + (r & 1) * bufb;
      const int ch0 = rm * C, nch = min(C, nc - ch0);
      const u32x4 *ts = reinterpret_cast<const u32x4 *>(buf);
      const uint32_t *wsd = reinterpret_cast<const uint32_t *>(buf + wofs) + cp * C * 64;
      struct Ops { u32x4 a[2]; uint32_t wd[2]; };
      auto fetch = [&](int chl, Ops &o) {
#pragma unroll
        for (int step = 0; step < 2; ++step) o.a[step] = ts[(chl * 4 + 2 * step + lh) * 32 + lr];
        o.wd[0] = wsd[chl * 64 + lr];
        o.wd[1] = wsd[chl * 64 + 32 + lr];
      };
      auto mma = [&](const Ops &o, float16_t (&acc)[2]) {
        const uint32_t wl0 = o.wd[0] << (4 * lh), wl1 = o.wd[1] << (4 * lh);  // group g = 2 step + lh
#pragma unroll
        for (int step = 0; step < 2; ++step) {
          const half8_t av = as_h8(o.a[step]);
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, as_h8(sign_ones(wl0 << (8 * step))), acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, as_h8(sign_ones(wl1 << (8 * step))), acc[1], 0, 0, 0);
        }
      };
      // chunks are path-major: [0, nch0) are path 0, [nch0, nch) path 1;
      // the wave takes the chunks chl = phase (mod nph), path by path
      const int nch0 = max(0, min(nch, Ly.Wk - ch0));
      auto run = [&](int lo, int hi, float16_t (&acc)[2]) {
        int chl = lo + ((phase - lo) % nph + nph) % nph;
        if (chl >= hi) return;
        Ops c;
        fetch(chl, c);
        for (; chl < hi; chl += nph) {
          Ops n;
          fetch(min(chl + nph, hi - 1), n);  // unconditional: see stage 1
          mma(c, acc);
          c = n;
        }
      };
      run(0, nch0, acc0);
      run(nch0, nch, acc1);
    }
    // layer epilogue: the layer's last round buffer becomes the reduction area
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem + ((r - 1) & 1) * bufb);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 8 * (e >> 2) + 4 * lh + (e & 3), col = ni * 32 + lr;
        red[(w * 32 + row) * kRP2 + col] = hv[0][ni] * acc0[ni][e] + hv[1][ni] * acc1[ni][e];
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      if (t >= 256) break;  // threads 0-255 own the outputs
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // phases of pair q are waves q, q + nb, ...: summed in phase order
        const int o = (q * 32 + row_o) * kRP2 + c_o + e;
        float sum = red[o];
#pragma unroll
        for (int ph = 1; ph < nph; ++ph) sum += red[o + ph * nb * 32 * kRP2];
        v[e] = mh2f(mf2h(sum));  // the layer's fp16 output
        ys[q][e] += v[e];
      }
      if (Ly.y && tok0 + row_o < A.M) store8(Ly.y, A.b, tok0 + row_o, j0 + q * 64 + c_o, v);
    }
  }
  if (t >= 256 || A.direct || !xout || tok0 + row_o >= A.M) return true;
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = A.c_out * ys[q][e];
    if (kCoh)
      store8c(coherent_rsrc(xout, (uint32_t)(A.M * A.opitch * 2)), A.b, A.opitch, tok0 + row_o,
              j0 + q * 64 + c_o, o);
    else
      store8(xout, A.b, tok0 + row_o, j0 + q * 64 + c_o, o);
  }
  return true;
}

template <int NB, int NW>
__global__ void __launch_bounds__(NW * 64)
k_unit_s2(S2Args A) {
  extern __shared__ __align__(16) unsigned char smem[];  // 2 round buffers
  (void)s2_tile<NB, NW, false>(A, A.xout, blockIdx.x, blockIdx.y, smem, [] { return true; });
}

// ------------------------------------------------------------------ host
static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
static constexpr size_t kS1Lds = (size_t)s1_lds_bytes(kS1MaxC);

MfmaPlan *mfma_plan_build(const Layer *const *layers, int n) {
  if (n < 1 || n > kMaxUnitLayersM) return nullptr;
  MfmaPlan *P = new MfmaPlan();
  P->nl = n;
  P->a = layers[0]->a;
  P->b = layers[0]->b;
  P->a16 = (int)layers[0]->a16;
  int col = 0, nseg = 0;
  for (int m = 0; m < n; ++m) {
    const Layer &Ly = *layers[m];
    if (Ly.a != P->a || Ly.b != P->b) {
      delete P;
      return nullptr;
    }
    P->src[m] = &Ly;
    S2Layer &D = P->ly[m];
    D.su2 = nullptr; D.l = Ly.l; D.h = Ly.h; D.y = nullptr;
    D.b16 = (int)Ly.b16; D.s8 = (int)Ly.s8; D.Wk = (int)Ly.Wk; D.P = Ly.P;
    D.seg0[0] = D.seg0[1] = 0;
    D.pad_[0] = D.pad_[1] = 0;
    for (int p = 0; p < Ly.P; ++p) {
      P->seg_layer[nseg] = m;
      P->seg_path[nseg] = p;
      S1Seg &S = P->seg[nseg++];
      S.bits = nullptr;
      S.g = Ly.g + (size_t)p * Ly.a16;
      S.pitch = (int)Ly.L;
      S.s = (int)Ly.s;
      S.seg0 = col;
      S.pad_ = 0;
      S.l = Ly.l + (size_t)p * Ly.s8;
      D.seg0[p] = col;
      col += (int)round_up(Ly.s, 32);
    }
  }
  P->nseg = nseg;
  P->ntile32 = col / 32;
  P->Lt = (int)round_up(col, 128);
  return P;
}

void mfma_plan_free(MfmaPlan *p) { delete p; }

static int64_t s1_tiles(const MfmaPlan &P, int64_t Mc) { return (int64_t)(P.Lt / 128) * ((Mc + 31) / 32); }

// Splits of the input dimension: at most one block per CU (at most
// kMaxSplit splits), kcps chunks per split.  A split of at most kS1MaxC chunks is
// one round (cround = kcps rounded up to even); a longer one runs in
// double-buffered rounds of kS1RoundC chunks.
static int s1_nsplit(const MfmaPlan &P, int64_t Mc, const DeviceInfo &dev, int *kcps, int *cround) {
  const int64_t tiles = s1_tiles(P, Mc);
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int nkc = (int)((P.a + 31) / 32);
  // one 8-wave block per CU: as many splits as fill the CUs in one wave of blocks
  int ns = (int)std::min<int64_t>(kMaxSplit, std::max<int64_t>(1, cus / tiles));
  ns = std::min(ns, nkc);
  const int k = (nkc + ns - 1) / ns;
  *kcps = k;
  *cround = k <= kS1MaxC ? (k + 1) & ~1 : kS1RoundC;
  return (nkc + k - 1) / k;
}

// Stage-2 block width: the widest (nb column pairs) that still gives about
// 0.6 blocks per CU (one per CU from four 32-row blocks on), so wide
// outputs do not re-read T from many blocks; c2 = chunks per round, as
// many as two buffers allow.  The unit launches and the one-launch stack
// share the rule, so they run the same tiles in the same order.
static void s2_shape(const MfmaPlan &P, int64_t Mc, const DeviceInfo &dev, int *nb, int *c2) {
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int64_t rt = (Mc + 31) / 32;
  int n = 4;
  // with four or more row blocks the one-launch stack pipelines them and
  // is faster with the narrower blocks (M = 128: 2.80 against 2.90 ms; the
  // unit launches then take 3.03 against 2.91 ms, and are no longer the
  // automatic choice there)
  const int64_t fill10 = rt >= 4 ? 10 : 6;
  while (n > 1 && (P.b + 64 * n - 1) / (64 * n) * rt < cus * fill10 / 10) n /= 2;
  *nb = n;
  // a multiple of 4: one word instruction covers 4 chunks of a pair, and
  // must not spill into the next pair's words
  *c2 = std::min(kRC2, kS2Lds / 2 / s2_buf_bytes(1, n)) & ~3;
  static_assert(kS2Lds / 2 / s2_buf_bytes(1, 4) >= kS2MinC, "rounds hold the wave partials");
  static_assert(8 * 32 * kRP2 * 4 <= s2_buf_bytes((kS2Lds / 2 / s2_buf_bytes(1, 4)) & ~3, 4) &&
                    8 * 32 * kRP2 * 4 <= s2_buf_bytes(std::min(kRC2, kS2Lds / 2 / s2_buf_bytes(1, 2)) & ~3, 2) &&
                    8 * 32 * kRP2 * 4 <= s2_buf_bytes(std::min(kRC2, kS2Lds / 2 / s2_buf_bytes(1, 1)) & ~3, 1),
                "8-wave partials fit the round buffer");
}

static size_t s1_lds_launch(int kcps, int cround) {
  const size_t one = (size_t)s1_lds_bytes(cround);
  return std::max<size_t>(kcps > cround ? 2 * one : one, 16384);  // >= the epilogue's wave sums
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
  const void *s2k[3] = {(const void *)k_unit_s2<1, 8>, (const void *)k_unit_s2<2, 8>,
                        (const void *)k_unit_s2<4, 8>};
  for (int i = 0; i < 3 && e == hipSuccess; ++i)
    e = hipFuncSetAttribute(s2k[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)kS2Lds);
  if (e == hipSuccess && bit) done.fetch_or(bit);
  return e;
}

hipError_t launch_mfma_unit(const MfmaPlan *p, const uint16_t *x, int64_t M,
                            uint16_t *const *y_layers, uint16_t *xout, float c_out, bool direct,
                            void *ws, unsigned *cnt, const void *zero, const DeviceInfo &dev,
                            hipStream_t st) {
  hipError_t e = set_lds_attr(dev.device);
  if (e != hipSuccess) return e;
  // the matrix-core sign copies are built on first use, so their addresses
  // are taken here
  S1Seg segs[kMaxUnitSegs];
  S2Layer lys[kMaxUnitLayersM];
  for (int i = 0; i < kMaxUnitSegs; ++i) segs[i] = p->seg[i];
  for (int m = 0; m < kMaxUnitLayersM; ++m) lys[m] = p->ly[m];
  for (int m = 0; m < p->nl; ++m) {
    if (!p->src[m]->sv1m || !p->src[m]->su2m) return hipErrorInvalidValue;
    lys[m].su2 = p->src[m]->su2m;
  }
  for (int i = 0; i < p->nseg; ++i) {
    const Layer &Ly = *p->src[p->seg_layer[i]];
    segs[i].bits = Ly.sv1m + (size_t)p->seg_path[i] * Ly.s;
  }
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
    A1.nsplit = s1_nsplit(*p, Mc, dev, &A1.kcps, &A1.cround);
    A1.nseg = p->nseg;
    A1.xvec = (p->a % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    A1.xpitch = (int)p->a;
    A1.tp8 = p->Lt >> 3;
    A1.tstride = p->Lt / 128;
    A1.psplit = A1.nsplit;
    for (int i = 0; i < kMaxUnitSegs; ++i) A1.seg[i] = segs[i];
    dim3 g1((unsigned)(p->Lt / 128), (unsigned)((Mc + 31) / 32), (unsigned)A1.nsplit);
    const size_t lds1 = s1_lds_launch(A1.kcps, A1.cround);
    hipLaunchKernelGGL(k_unit_s1, g1, dim3(kThreads1), lds1, st, A1);
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
    s2_shape(*p, Mc, dev, &A2.nb, &A2.c2);
    A2.tp8 = p->Lt >> 3;
    A2.opitch = (int)p->b;
    A2.nrounds = 0;
    for (int m = 0; m < p->nl; ++m) A2.nrounds += (p->ly[m].P * p->ly[m].Wk + A2.c2 - 1) / A2.c2;
    for (int m = 0; m < kMaxUnitLayersM; ++m) {
      A2.ly[m] = lys[m];
      A2.ly[m].y = (m < p->nl && y_layers && y_layers[m]) ? y_layers[m] + mb * p->b : nullptr;
    }
    dim3 g2((unsigned)((p->b + 64 * A2.nb - 1) / (64 * A2.nb)), (unsigned)((Mc + 31) / 32));
    const size_t lds2 = (size_t)2 * s2_buf_bytes(A2.c2, A2.nb);
    if (A2.nb == 4)
      hipLaunchKernelGGL((k_unit_s2<4, 8>), g2, dim3(512), lds2, st, A2);
    else if (A2.nb == 2)
      hipLaunchKernelGGL((k_unit_s2<2, 8>), g2, dim3(512), lds2, st, A2);
    else
      hipLaunchKernelGGL((k_unit_s2<1, 8>), g2, dim3(512), lds2, st, A2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------ persistent stack, M >= 64
// The whole stack in one launch: the stage-1 and stage-2 tiles of every
// unit above are its work items, in a fixed order, item i on workgroup
// i % G.
// Items are ordered by chain step c (2 u for unit u's first stage, 2 u + 1
// for its second), then by 32-row block rb, then by tile (split-major in
// stage 1).  Rows are independent through the whole stack, so an item of
// step c and row block rb waits only for step c - 1 of the same row block
// (a counter of completed tiles per step and row block): the row blocks
// pipeline, a block's next unit starting while other blocks are still in
// the previous one, and no launch boundary separates the units.
// A workgroup runs its items in increasing order, and an item waits only
// for items of the previous step, which their workgroups reach after
// items of lower steps alone: the launch completes once every workgroup
// has become resident (G is the device's resident capacity, so kernels on
// other streams only delay it).  A ticket counter instead (the next item
// to whichever workgroup finishes first, which needs no co-residency) made
// the M = 128 stack 3.57 ms against 2.96: every item's workgroup waited for
// its ticket from one contended word.  Intermediate x and T rows are written and read
// with device-scope stores and loads, each row block in its own region
// (fixed pitches), so concurrent steps of different row blocks never
// share memory.  The last workgroup to finish clears the counters for
// the next launch.  Every wait is bounded: one that gives up sets the
// error word (and its host-mapped copy) and its workgroup stops.
struct MStackArgs {
  const S1Args *__restrict__ s1;       // [U]; unit 0's x is x0
  const S2Args *__restrict__ s2;       // [U]; the last unit's xout is y
  const int *__restrict__ step_off;    // [2 U + 1] first item of each step
  const int *__restrict__ step_tiles;  // [2 U] tiles of one row block that complete a step
  int nsteps, nrb;
  const uint16_t *x0;
  uint16_t *y;
  unsigned *ctrl;  // [1] finished workgroups (zero between launches), [3] the last launch's generation
  unsigned *done;  // [2 U][nrb][fstride] per-tile flags: the generation of the launch that completed it
  int fstride;     // flag slots per (step, row block): at least every step's tiles per row block
  unsigned *err;   // device error word
  unsigned *herr;  // host-mapped error word
};

constexpr long kMSpin = 1L << 22;  // polls (each after a short sleep) before a wait gives up


__global__ void __launch_bounds__(kThreads1) k_mstack(MStackArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_last, s_ok, s_final;
  const int t = threadIdx.x;
  const int total = A.step_off[A.nsteps];
  const int U = A.nsteps >> 1;
  // items in round robin: item i on workgroup i % G, each workgroup's in
  // increasing order.  An item waits only for items of the previous step,
  // whose workgroups reach them after items of lower steps alone, so the
  // waits resolve once every workgroup has run (G is at most the device's
  // resident capacity)
  if (t == 0) s_ok = 1;
  // this launch's generation: the last one's plus 1 (kept on the device, so
  // graph replays stay distinct); a tile's flag holds it once it is done
  const unsigned gen = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&A.ctrl[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u);
  __syncthreads();
  unsigned tk = blockIdx.x;
  int c = 0;  // items only grow, so each step search starts at the last one
  while (tk < (unsigned)total) {
    while ((unsigned)A.step_off[c + 1] <= tk) ++c;
    c = __builtin_amdgcn_readfirstlane(c);
    const int u = c >> 1;
    const int per_rb = (A.step_off[c + 1] - A.step_off[c]) / A.nrb;
    const int local = (int)tk - A.step_off[c];
    const int rb = __builtin_amdgcn_readfirstlane(local / per_rb);
    const int k = __builtin_amdgcn_readfirstlane(local - rb * per_rb);
    // the dependency, waited for inside the tile once its weights are
    // requested: wave 0, lane i polls flags i, i + 64, ... of step c - 1 and
    // this row block until every one carries this launch's generation
    // flags [f0, f1) of step c - 1: every tile of it, except that a stage-1
    // split needs only the stage-2 column blocks that hold its x columns
    int f0 = 0, f1 = c > 0 ? A.step_tiles[c - 1] : 0;
    if (c > 0 && (c & 1) == 0) {
      CS1Args &P = *(CS1Args *)(A.s1 + u);
      const int nkc = (P.a + 31) >> 5, kc0 = (k / (P.Lt / 128)) * P.kcps, kc1 = min(nkc, kc0 + P.kcps);
      const int wcb = 64 * ((CS2Args *)(A.s2 + u - 1))->nb;  // columns per stage-2 tile of unit u - 1
      f0 = (32 * kc0) / wcb;
      f1 = min(f1, (min(32 * kc1, P.a) - 1) / wcb + 1);
    }
    f0 = __builtin_amdgcn_readfirstlane(f0);
    f1 = __builtin_amdgcn_readfirstlane(f1);
    auto dep = [&]() -> bool {
      if (c > 0 && t < 64) {
        const unsigned *f = A.done + ((size_t)(c - 1) * A.nrb + rb) * A.fstride;
        long sp = 0;
        bool ok = true;
        for (int b0 = f0; b0 < f1 && ok; b0 += 64) {
          const int i = b0 + t;
          const int need = f1;
          while (true) {
            const unsigned v = i < need ? __hip_atomic_load(const_cast<unsigned *>(f + i), __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : gen;
            if (__all(v == gen)) break;
            const unsigned ev = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(A.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (++sp > kMSpin || ev != 0u) {
              if (t == 0) {
                __hip_atomic_store(A.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(A.herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                s_ok = 0;
              }
              ok = false;
              break;
            }
            __builtin_amdgcn_s_sleep(4);
          }
        }
      }
      __syncthreads();  // the dependency is met (or s_ok is 0)
      return s_ok != 0;
    };
    int res;
    int slot = k;  // the tile's place among its step's tiles of this row block
    if ((c & 1) == 0) {
      CS1Args &P = *(CS1Args *)(A.s1 + u);  // uniform: scalar loads
      const int gx = P.Lt / 128;
      slot = k % gx;
      res = s1_tile<true>(P, u == 0 ? A.x0 : P.x, k % gx, rb, k / gx, smem, &s_last, dep);
    } else {
      CS2Args &P = *(CS2Args *)(A.s2 + u);
      uint16_t *xo = u == U - 1 ? A.y : P.xout;
      bool ok2;
      if (P.nb == 4)
        ok2 = s2_tile<4, 8, true>(P, xo, k, rb, smem, dep);
      else if (P.nb == 2)
        ok2 = s2_tile<2, 8, true>(P, xo, k, rb, smem, dep);
      else
        ok2 = s2_tile<1, 8, true>(P, xo, k, rb, smem, dep);
      res = ok2 ? 1 : -1;
    }
    if (res < 0) break;
    const bool completed = res == 1;
    // every wave's device-scope stores have completed before the tile is
    // counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0 && completed) {
      __hip_atomic_store(&A.done[((size_t)c * A.nrb + rb) * A.fstride + slot], gen, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // LDS free for the next item
    tk += gridDim.x;
  }
  if (t == 0) {
    const unsigned f = __hip_atomic_fetch_add(&A.ctrl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_final = f == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_final) return;
  // every other workgroup has finished: the next launch counts from zero
  // and takes the next generation
  if (t == 0) {
    __hip_atomic_store(&A.ctrl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&A.ctrl[3], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct MStackArgSet {
  S1Args *s1 = nullptr;
  S2Args *s2 = nullptr;
  int *steps = nullptr;  // step_off [2U + 1] then step_tiles [2U]
  size_t lds = 0;
};

struct MStackPlan {
  std::vector<const MfmaPlan *> units;
  int device = 0;
  int64_t a0 = 0, b_last = 0, max_width = 0;
  float kappa = 1.f;
  int G = 0;
  int Ltmax = 0, gxmax = 0;
  int fstride = 0;           // flag slots per (step, row block)
  unsigned *ctrl = nullptr;  // finish count at ctrl[1], err at ctrl[2], generation at ctrl[3]
  unsigned *done = nullptr;
  unsigned *herr = nullptr, *herr_dev = nullptr;
  bool broken = false;
  // argument sets by (rows, scratch addresses); kept until the plan is freed
  std::map<std::vector<uintptr_t>, MStackArgSet> sets;
};

static void mstack_free_sets(MStackPlan *p) {
  for (auto &kv : p->sets) {
    if (kv.second.s1) (void)hipFree(kv.second.s1);
    if (kv.second.s2) (void)hipFree(kv.second.s2);
    if (kv.second.steps) (void)hipFree(kv.second.steps);
  }
  p->sets.clear();
}

void mstack_free(MStackPlan *p) {
  if (!p) return;
  mstack_free_sets(p);
  if (p->ctrl) (void)hipFree(p->ctrl);
  if (p->done) (void)hipFree(p->done);
  if (p->herr) (void)hipHostFree(p->herr);
  delete p;
}

MStackPlan *mstack_build(const std::vector<const MfmaPlan *> &units, float kappa, const DeviceInfo &dev) {
  if (units.empty()) return nullptr;
  MStackPlan *P = new (std::nothrow) MStackPlan();
  if (!P) return nullptr;
  P->units = units;
  P->device = dev.device;
  P->kappa = kappa;
  P->a0 = units.front()->a;
  P->b_last = units.back()->b;
  for (const MfmaPlan *u : units) {
    // 16-byte rows throughout (the x copies are LDS-DMA of 8 fp16)
    if (u->a % 8 != 0 || u->b % 8 != 0) {
      delete P;
      return nullptr;
    }
    P->max_width = std::max<int64_t>(P->max_width, std::max(u->a, u->b));
    P->Ltmax = std::max(P->Ltmax, u->Lt);
    // a step's tiles per row block: Lt / 128 in stage 1, at most b / 64 in stage 2
    P->fstride = std::max(P->fstride, (int)std::max<int64_t>(u->Lt / 128, (u->b + 63) / 64));
  }
  P->fstride = (P->fstride + 15) / 16 * 16;
  P->gxmax = P->Ltmax / 128;
  const int U = (int)units.size();
  const int nrb = kMfmaRows / 32;
  bool ok = hipMalloc(&P->ctrl, 64) == hipSuccess && hipMemset(P->ctrl, 0, 64) == hipSuccess;
  const size_t done_bytes = sizeof(unsigned) * 2 * U * nrb * P->fstride;
  ok = ok && hipMalloc(&P->done, done_bytes) == hipSuccess && hipMemset(P->done, 0, done_bytes) == hipSuccess;
  ok = ok && hipHostMalloc(&P->herr, 64, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
       hipHostGetDevicePointer((void **)&P->herr_dev, P->herr, 0) == hipSuccess;
  if (ok) *(volatile unsigned *)P->herr = 0u;
  const size_t lds_max = std::max(kS1Lds, (size_t)kS2Lds);
  ok = ok && hipFuncSetAttribute((const void *)k_mstack, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds_max) == hipSuccess;
  int occ = 0;
  ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_mstack, kThreads1, lds_max) == hipSuccess;
  if (!ok || occ < 1) {
    (void)hipGetLastError();  // not an error of the caller's next call
    mstack_free(P);
    return nullptr;
  }
  P->G = (dev.cu_count > 0 ? dev.cu_count : 256) * occ;
  return P;
}

size_t mstack_ws_bytes(const MStackPlan *p) {
  return 2 * (size_t)round_up((int64_t)kMfmaRows * p->Ltmax * 2, 256) +
         (size_t)(kMfmaRows / 32) * p->gxmax * kMaxSplit * 4096 * sizeof(float);
}
size_t mstack_cnt_entries(const MStackPlan *p) { return (size_t)(kMfmaRows / 32) * p->gxmax; }

// The device argument set for Mc rows and these scratch buffers, built on
// first use (allocates and copies synchronously).
static lb_status mstack_args(MStackPlan *p, int64_t Mc, void *ws, unsigned *cnt, uint16_t *xb0,
                             uint16_t *xb1, const void *zero, const DeviceInfo &dev, hipStream_t st,
                             MStackArgSet **out, std::string *msg) {
  const std::vector<uintptr_t> key = {(uintptr_t)Mc, (uintptr_t)ws, (uintptr_t)cnt, (uintptr_t)xb0,
                                      (uintptr_t)xb1};
  auto it = p->sets.find(key);
  if (it != p->sets.end()) {
    *out = &it->second;
    return LB_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    if (msg) *msg = "the persistent M >= 64 launch for this row count is not set up yet (run this M once "
                    "outside capture first)";
    return LB_ENOTREADY;
  }
  const int U = (int)p->units.size();
  const int nrb = (int)((Mc + 31) / 32);
  std::vector<S1Args> h1(U);
  std::vector<S2Args> h2(U);
  std::vector<int> steps(4 * U + 1, 0);
  // T alternates between two regions by unit parity: a stage-1 split of
  // unit u + 1 waits only for the stage-2 tiles of unit u that produce its
  // x columns, so it may run while other stage-2 tiles of unit u still read
  // unit u's T
  const size_t tbytes = (size_t)round_up((int64_t)kMfmaRows * p->Ltmax * 2, 256);
  uint16_t *Tr[2] = {reinterpret_cast<uint16_t *>(ws),
                     reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(ws) + tbytes)};
  float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + 2 * tbytes);
  size_t lds = 16384;
  int off = 0;
  for (int u = 0; u < U; ++u) {
    const MfmaPlan &P = *p->units[u];
    for (int m = 0; m < P.nl; ++m)
      if (!P.src[m]->sv1m || !P.src[m]->su2m) {
        if (msg) *msg = "matrix-core sign copies missing";
        return LB_ENOTREADY;
      }
    S1Args &A1 = h1[u];
    A1.x = u == 0 ? nullptr : (((u - 1) & 1) ? xb1 : xb0);
    A1.T = Tr[u & 1];
    A1.part = part;
    A1.cnt = cnt;
    A1.zero = zero;
    A1.M = Mc;
    A1.a = (int)P.a;
    A1.a16 = P.a16;
    A1.Lt = P.Lt;
    A1.ntile32 = P.ntile32;
    A1.nsplit = s1_nsplit(P, Mc, dev, &A1.kcps, &A1.cround);
    A1.nseg = P.nseg;
    A1.xvec = 1;
    A1.xpitch = u == 0 ? (int)p->a0 : (int)p->max_width;
    A1.tp8 = p->Ltmax >> 3;
    A1.tstride = p->gxmax;
    A1.psplit = kMaxSplit;
    for (int i = 0; i < kMaxUnitSegs; ++i) A1.seg[i] = P.seg[i];
    for (int i = 0; i < P.nseg; ++i) {
      const Layer &Ly = *P.src[P.seg_layer[i]];
      A1.seg[i].bits = Ly.sv1m + (size_t)P.seg_path[i] * Ly.s;
    }
    lds = std::max(lds, s1_lds_launch(A1.kcps, A1.cround));
    S2Args &A2 = h2[u];
    A2.T = Tr[u & 1];
    A2.xout = u == U - 1 ? nullptr : ((u & 1) ? xb1 : xb0);
    A2.zero = zero;
    A2.M = Mc;
    A2.b = (int)P.b;
    A2.Lt = P.Lt;
    A2.nl = P.nl;
    A2.direct = 0;
    A2.c_out = p->kappa / std::sqrt((float)P.nl);
    s2_shape(P, Mc, dev, &A2.nb, &A2.c2);
    A2.tp8 = p->Ltmax >> 3;
    A2.opitch = u == U - 1 ? (int)p->b_last : (int)p->max_width;
    A2.nrounds = 0;
    for (int m = 0; m < P.nl; ++m) A2.nrounds += (P.ly[m].P * P.ly[m].Wk + A2.c2 - 1) / A2.c2;
    for (int m = 0; m < kMaxUnitLayersM; ++m) {
      A2.ly[m] = P.ly[m];
      A2.ly[m].su2 = m < P.nl ? P.src[m]->su2m : nullptr;
      A2.ly[m].y = nullptr;
    }
    lds = std::max(lds, (size_t)2 * s2_buf_bytes(A2.c2, A2.nb));
    const int gx = P.Lt / 128;
    const int njx = (int)((P.b + 64 * A2.nb - 1) / (64 * A2.nb));
    steps[2 * u] = off;
    off += nrb * gx * A1.nsplit;
    steps[2 * u + 1] = off;
    off += nrb * njx;
    steps[2 * U + 1 + 2 * u] = gx;
    steps[2 * U + 1 + 2 * u + 1] = njx;
  }
  steps[2 * U] = off;
  MStackArgSet set;
  set.lds = lds;
  hipError_t e = hipMalloc(&set.s1, sizeof(S1Args) * U);
  if (e == hipSuccess) e = hipMalloc(&set.s2, sizeof(S2Args) * U);
  if (e == hipSuccess) e = hipMalloc(&set.steps, sizeof(int) * steps.size());
  if (e == hipSuccess) e = hipMemcpy(set.s1, h1.data(), sizeof(S1Args) * U, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(set.s2, h2.data(), sizeof(S2Args) * U, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(set.steps, steps.data(), sizeof(int) * steps.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    if (set.s1) (void)hipFree(set.s1);
    if (set.s2) (void)hipFree(set.s2);
    if (set.steps) (void)hipFree(set.steps);
    if (msg) *msg = std::string("persistent M >= 64 setup: ") + hipGetErrorString(e);
    return LB_EHIP;
  }
  *out = &(p->sets[key] = set);
  return LB_OK;
}

bool mstack_ready(const MStackPlan *p, int64_t M, void *ws, unsigned *cnt, uint16_t *xb0, uint16_t *xb1) {
  for (int64_t mb = 0; mb < M; mb += kMfmaRows) {
    const int64_t Mc = std::min<int64_t>(kMfmaRows, M - mb);
    const std::vector<uintptr_t> key = {(uintptr_t)Mc, (uintptr_t)ws, (uintptr_t)cnt, (uintptr_t)xb0,
                                        (uintptr_t)xb1};
    if (p->sets.find(key) == p->sets.end()) return false;
  }
  return true;
}

lb_status mstack_run(MStackPlan *p, const uint16_t *x0, uint16_t *y, int64_t M, void *ws, unsigned *cnt,
                     uint16_t *xb0, uint16_t *xb1, const void *zero, const DeviceInfo &dev,
                     hipStream_t st, std::string *msg) {
  if (!p->broken && *(volatile unsigned *)p->herr != 0u) {
    p->broken = true;
    if (msg) *msg = "persistent M >= 64 stack: an earlier launch gave up a device-side wait (its output "
                    "is undefined); this call did not run, the next one resets";
    return LB_ETIMEOUT;
  }
  if (p->broken) {
    if (hipDeviceSynchronize() != hipSuccess || hipMemset(p->ctrl, 0, 64) != hipSuccess ||
        hipMemset(p->done, 0, sizeof(unsigned) * 2 * p->units.size() * (kMfmaRows / 32) * p->fstride) !=
            hipSuccess ||
        hipMemset(cnt, 0, sizeof(unsigned) * mstack_cnt_entries(p)) != hipSuccess)
      return LB_EHIP;
    *(volatile unsigned *)p->herr = 0u;
    p->broken = false;
  }
  if (((uintptr_t)x0 & 15) || ((uintptr_t)y & 15)) {
    if (msg) *msg = "x0 and y must be 16-byte aligned";
    return LB_EINVAL;
  }
  const int U = (int)p->units.size();
  for (int64_t mb = 0; mb < M; mb += kMfmaRows) {
    const int64_t Mc = std::min<int64_t>(kMfmaRows, M - mb);
    MStackArgSet *set = nullptr;
    lb_status s = mstack_args(p, Mc, ws, cnt, xb0, xb1, zero, dev, st, &set, msg);
    if (s != LB_OK) return s;
    MStackArgs A;
    A.s1 = set->s1;
    A.s2 = set->s2;
    A.step_off = set->steps;
    A.step_tiles = set->steps + 2 * U + 1;
    A.nsteps = 2 * U;
    A.nrb = (int)((Mc + 31) / 32);
    A.x0 = x0 + mb * p->a0;
    A.y = y + mb * p->b_last;
    A.ctrl = p->ctrl;
    A.done = p->done;
    A.fstride = p->fstride;
    A.err = p->ctrl + 2;
    A.herr = p->herr_dev;
    hipLaunchKernelGGL(k_mstack, dim3(p->G), dim3(kThreads1), set->lds, st, A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      if (msg) *msg = std::string("persistent M >= 64 launch: ") + hipGetErrorString(e);
      return LB_EHIP;
    }
  }
  return LB_OK;
}

}  // namespace lbi
