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
// Both stages compute 64 x 64 output tiles with 4 waves per workgroup.
// The waves split K (interleaved 32-row chunks); their partial tiles are
// summed in a fixed order through LDS.  Stage 1 also splits K across
// workgroups when the tile count alone cannot fill the chip; the last
// workgroup of a tile to finish (an atomic counter per tile) sums the
// partials in split order, so the result does not depend on timing.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "lb_internal.h"

namespace lbi {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // 4 waves
constexpr int kRP = 64 + 4;    // LDS pitch (floats) of a 64 x 64 partial tile
constexpr int kMaxSplit = 8;

struct S1Seg {
  const uint32_t *bits;  // sv1 + p*s: word (row group r, column k) at bits[r * pitch + k]
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
  int64_t M;  // rows of this chunk
  int a, a16, Lt, ntile32, kcps, nsplit, nseg, xvec;
  S1Seg seg[kMaxUnitSegs];
};

struct S2Layer {
  const uint32_t *su2;
  const uint16_t *l;
  const uint16_t *h;
  uint16_t *y;  // per-layer output (may be null)
  int b16, s8, Wk, P, seg0[2], pad_[2];
};
static_assert(sizeof(S2Layer) == 64, "S2Layer layout");

struct S2Args {
  const uint16_t *T;
  uint16_t *xout;  // combined output (stack) or null
  int64_t M;
  int b, Lt, nl, direct;
  float c_out;
  int pad_;
  S2Layer ly[kMaxUnitLayersM];
};

struct MfmaPlan {
  int nl = 0;
  int64_t a = 0, b = 0;
  int a16 = 0, Lt = 0, ntile32 = 0, nseg = 0;
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

__device__ __forceinline__ half8_t as_h8(uint4 v) { return __builtin_bit_cast(half8_t, v); }

// Flip the fp16 sign bit of element e of v where bit e of `bits` is 0
// (sign -1); bit 1 (sign +1) keeps the value.
__device__ __forceinline__ uint4 apply_signs(uint4 v, uint32_t bits) {
  const uint32_t nb = ~bits;
  v.x ^= ((nb << 15) & 0x8000u) | ((nb << 30) & 0x80000000u);
  v.y ^= ((nb << 13) & 0x8000u) | ((nb << 28) & 0x80000000u);
  v.z ^= ((nb << 11) & 0x8000u) | ((nb << 26) & 0x80000000u);
  v.w ^= ((nb << 9) & 0x8000u) | ((nb << 24) & 0x80000000u);
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

// 8 fp16 of row `tok` of x from column i0 (zero outside the matrix).
__device__ __forceinline__ uint4 load_x8(const uint16_t *__restrict__ x, int64_t M, int a,
                                         int xvec, int64_t tok, int i0) {
  uint4 v = {0u, 0u, 0u, 0u};
  if (tok >= M || i0 >= a) return v;
  const uint16_t *p = x + tok * a + i0;
  if (xvec && i0 + 8 <= a) return *reinterpret_cast<const uint4 *>(p);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = i0 + e < a ? p[e] : 0u;
  v.x = h[0] | (h[1] << 16); v.y = h[2] | (h[3] << 16);
  v.z = h[4] | (h[5] << 16); v.w = h[6] | (h[7] << 16);
  return v;
}

// This wave's 2 x 2 tiles of 32 x 32 into red[wave] (64 rows, pitch kRP),
// column tile ni scaled by sc[ni].
__device__ __forceinline__ void spill_acc(float *red, const float16_t (&acc)[2][2], float sc0,
                                          float sc1) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  float *rw = red + wave * 64 * kRP;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mi * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
        rw[row * kRP + ni * 32 + lr] = acc[mi][ni][r] * (ni ? sc1 : sc0);
      }
}

// Sum of the 4 waves' tiles, in wave order, at (row, 8 columns from c0).
__device__ __forceinline__ void sum_waves(const float *red, int row, int c0, float *v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int o = row * kRP + c0 + e;
    v[e] = ((red[o] + red[64 * kRP + o]) + red[2 * 64 * kRP + o]) + red[3 * 64 * kRP + o];
  }
}

// ------------------------------------------------------------- stage 1
// grid = (Lt / 64, ceil(M / 64), nsplit).  Block (cx, ty, z) computes
// columns [64 cx, 64 cx + 64) of rows [64 ty, 64 ty + 64) over the 32-row
// chunks [z * kcps, (z + 1) * kcps) of the input dimension.  Rows past M
// come out as zeros, so every row of T the second stage reads is written.
__global__ void __launch_bounds__(kThreads)
k_unit_s1(S1Args A) {
  extern __shared__ __align__(16) float red[];  // 4 x 64 x kRP
  __shared__ int s_last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const int t = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.y * 64;

  // per 32-column tile ni: the lane's column, its bits and scales
  const uint32_t *bp[2];
  const uint16_t *gp[2];
  int pitch[2];
  bool cval[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    const int t32 = blockIdx.x * 2 + ni;
    bp[ni] = nullptr; gp[ni] = nullptr; pitch[ni] = 0; cval[ni] = false;
    if (t32 < A.ntile32) {
      int e = 0;
      for (int q = 1; q < A.nseg; ++q)
        if (t32 * 32 >= A.seg[q].seg0) e = q;
      const int k = t32 * 32 - A.seg[e].seg0 + lr;
      cval[ni] = k < A.seg[e].s;
      bp[ni] = A.seg[e].bits + k;
      gp[ni] = A.seg[e].g;
      pitch[ni] = A.seg[e].pitch;
    }
  }

  const int nkc = (A.a + 31) >> 5;
  const int kc0 = blockIdx.z * A.kcps;
  const int kc1 = min(nkc, kc0 + A.kcps);

  float16_t acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // raw operands of one 32-row chunk: x[step][mi], g[step][ni], words[ni];
  // the next chunk's are loaded while the current one is multiplied
  uint4 cx[2][2], cg[2][2], nx[2][2], ng[2][2];
  uint32_t cw[2], nw[2];
  auto load = [&](int kc, uint4 (&xo)[2][2], uint4 (&go)[2][2], uint32_t (&wo)[2]) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) wo[ni] = cval[ni] ? bp[ni][(size_t)kc * pitch[ni]] : 0u;
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const int i0 = kc * 32 + step * 16 + lh * 8;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        xo[step][mi] = load_x8(A.x, A.M, A.a, A.xvec, tok0 + mi * 32 + lr, i0);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        go[step][ni] = (gp[ni] && i0 + 8 <= A.a16) ? *reinterpret_cast<const uint4 *>(gp[ni] + i0)
                                                   : uint4{0u, 0u, 0u, 0u};
    }
  };
  int kc = kc0 + wave;
  if (kc < kc1) load(kc, cx, cg, cw);
  for (; kc < kc1; kc += 4) {
    if (kc + 4 < kc1) load(kc + 4, nx, ng, nw);
#pragma unroll
    for (int step = 0; step < 2; ++step) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        uint4 bv = apply_signs(cg[step][ni], (cw[ni] >> (8 * (2 * step + lh))) & 255u);
        if (!cval[ni]) bv = uint4{0u, 0u, 0u, 0u};
        const half8_t bh = as_h8(bv);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(cx[step][mi]), bh, acc[mi][ni], 0, 0, 0);
      }
    }
#pragma unroll
    for (int step = 0; step < 2; ++step)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        cx[step][i] = nx[step][i];
        cg[step][i] = ng[step][i];
      }
    cw[0] = nw[0];
    cw[1] = nw[1];
  }

  spill_acc(red, acc, 1.f, 1.f);
  __syncthreads();

  // thread t owns (row = P & 63, 8 columns from 8 * (P >> 6)) for P = t, t + 256
  float v[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int P = t + 256 * hh;
    sum_waves(red, P & 63, 8 * (P >> 6), v[hh]);
  }
  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  if (A.nsplit > 1) {
    // split z's partial: value (hh, e) of thread t at [((tile*nsplit + z)*16 + hh*8 + e)*256 + t]
    float *pp = A.part + ((size_t)tile * A.nsplit + blockIdx.z) * 4096;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) st_rel(&pp[(hh * 8 + e) * 256 + t], v[hh][e]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {
      const unsigned old =
          __hip_atomic_fetch_add(&A.cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (unsigned)(A.nsplit - 1);
    }
    __syncthreads();
    if (!s_last) return;
    const float *pt = A.part + (size_t)tile * A.nsplit * 4096;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float q[kMaxSplit][8];
#pragma unroll
      for (int z = 0; z < kMaxSplit; ++z)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          q[z][e] = z < A.nsplit ? ld_rel(&pt[((size_t)z * 16 + hh * 8 + e) * 256 + t]) : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float s = q[0][e];
#pragma unroll
        for (int z = 1; z < kMaxSplit; ++z)
          if (z < A.nsplit) s += q[z][e];
        v[hh][e] = s;
      }
    }
    if (t == 0) __hip_atomic_store(&A.cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int Lt8 = A.Lt >> 3;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int P = t + 256 * hh;
    const int row = P & 63, c8 = blockIdx.x * 8 + (P >> 6);
    const int64_t tb = (tok0 >> 5) + (row >> 5);
    *reinterpret_cast<uint4 *>(A.T + ((tb * Lt8 + c8) * 32 + (row & 31)) * 8) = pack8(v[hh]);
  }
}

// ------------------------------------------------------------- stage 2
// grid = (ceil(b / 64), ceil(M / 64)).  Block (jx, ty) computes outputs
// [64 jx, 64 jx + 64) of rows [64 ty, 64 ty + 64) for every layer of the
// unit, then their combine.
__global__ void __launch_bounds__(kThreads)
k_unit_s2(S2Args A) {
  extern __shared__ __align__(16) float red[];  // 4 x 64 x kRP
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
  const int t = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.y * 64;
  const int j0 = blockIdx.x * 64;
  const int Lt8 = A.Lt >> 3;
  const int64_t tb0 = tok0 >> 5;
  // thread t owns (row = P >> 3, 8 columns from 8 * (P & 7)) for P = t, t + 256
  float ys[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) ys[hh][e] = 0.f;

  for (int m = 0; m < A.nl; ++m) {
    const S2Layer &Ly = A.ly[m];
    // waves 0-1 take path 0 and 2-3 path 1 (or all four path 0), and
    // interleave over the path's 32-column chunks
    int p, q0, qs;
    if (Ly.P == 2) {
      p = wave >> 1; q0 = wave & 1; qs = 2;
    } else {
      p = 0; q0 = wave; qs = 4;
    }
    const uint32_t *wb[2];
    bool jv[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int j = j0 + ni * 32 + lr;
      jv[ni] = j < A.b;
      wb[ni] = Ly.su2 + (size_t)p * Ly.Wk * Ly.b16 + j;
    }
    const uint16_t *lb = Ly.l + (size_t)p * Ly.s8;
    const int c8b = Ly.seg0[p] >> 3;
    const int Wk = Ly.Wk, b16 = Ly.b16, s8 = Ly.s8;

    float16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    uint4 ca[2][2], cl[2], na[2][2], nl[2];
    uint32_t cw[2], nw[2];
    auto load = [&](int q, uint4 (&ao)[2][2], uint4 (&lo)[2], uint32_t (&wo)[2]) {
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) wo[ni] = jv[ni] ? wb[ni][(size_t)q * b16] : 0u;
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const int k = q * 32 + step * 16 + lh * 8;
        lo[step] = k + 8 <= s8 ? *reinterpret_cast<const uint4 *>(lb + k) : uint4{0u, 0u, 0u, 0u};
        const int c8 = c8b + q * 4 + step * 2 + lh;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          ao[step][mi] = *reinterpret_cast<const uint4 *>(A.T + (((tb0 + mi) * Lt8 + c8) * 32 + lr) * 8);
      }
    };
    int q = q0;
    if (q < Wk) load(q, ca, cl, cw);
    for (; q < Wk; q += qs) {
      if (q + qs < Wk) load(q + qs, na, nl, nw);
#pragma unroll
      for (int step = 0; step < 2; ++step) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const half8_t bh = as_h8(apply_signs(cl[step], (cw[ni] >> (8 * (2 * step + lh))) & 255u));
#pragma unroll
          for (int mi = 0; mi < 2; ++mi)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(ca[step][mi]), bh, acc[mi][ni], 0, 0, 0);
        }
      }
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        cl[step] = nl[step];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) ca[step][mi] = na[step][mi];
      }
      cw[0] = nw[0];
      cw[1] = nw[1];
    }
    float hv[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
      hv[ni] = jv[ni] ? mh2f(Ly.h[(size_t)p * b16 + j0 + ni * 32 + lr]) : 0.f;
    spill_acc(red, acc, hv[0], hv[1]);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int P = t + 256 * hh;
      const int row = P >> 3, c0 = 8 * (P & 7);
      float v[8];
      sum_waves(red, row, c0, v);
      const int64_t tok = tok0 + row;
      const int jj = j0 + c0;
      uint16_t y16[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y16[e] = mf2h(v[e]);
        ys[hh][e] += mh2f(y16[e]);
      }
      if (Ly.y && tok < A.M) {
        uint16_t *dst = Ly.y + tok * A.b + jj;
        if ((A.b & 7) == 0 && jj + 8 <= A.b) {
          uint4 o;
          o.x = y16[0] | ((uint32_t)y16[1] << 16); o.y = y16[2] | ((uint32_t)y16[3] << 16);
          o.z = y16[4] | ((uint32_t)y16[5] << 16); o.w = y16[6] | ((uint32_t)y16[7] << 16);
          *reinterpret_cast<uint4 *>(dst) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (jj + e < A.b) dst[e] = y16[e];
        }
      }
    }
    __syncthreads();
  }
  if (A.direct || !A.xout) return;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int P = t + 256 * hh;
    const int row = P >> 3, c0 = 8 * (P & 7);
    const int64_t tok = tok0 + row;
    const int jj = j0 + c0;
    if (tok >= A.M) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = A.c_out * ys[hh][e];
    uint16_t *dst = A.xout + tok * A.b + jj;
    if ((A.b & 7) == 0 && jj + 8 <= A.b) {
      *reinterpret_cast<uint4 *>(dst) = pack8(o);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (jj + e < A.b) dst[e] = mf2h(o[e]);
    }
  }
}

// ------------------------------------------------------------------ host
static inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
static constexpr size_t kRedBytes = (size_t)4 * 64 * kRP * sizeof(float);

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
    S2Layer &D = P->ly[m];
    D.su2 = Ly.su2; D.l = Ly.l; D.h = Ly.h; D.y = nullptr;
    D.b16 = (int)Ly.b16; D.s8 = (int)Ly.s8; D.Wk = (int)Ly.Wk; D.P = Ly.P;
    D.seg0[0] = D.seg0[1] = 0;
    D.pad_[0] = D.pad_[1] = 0;
    for (int p = 0; p < Ly.P; ++p) {
      S1Seg &S = P->seg[nseg++];
      S.bits = Ly.sv1 + (size_t)p * Ly.s;
      S.g = Ly.g + (size_t)p * Ly.a16;
      S.pitch = (int)Ly.L;
      S.s = (int)Ly.s;
      S.seg0 = col;
      S.pad_ = 0;
      D.seg0[p] = col;
      col += (int)round_up(Ly.s, 32);
    }
  }
  P->nseg = nseg;
  P->ntile32 = col / 32;
  P->Lt = (int)round_up(col, 64);
  return P;
}

void mfma_plan_free(MfmaPlan *p) { delete p; }

static int s1_nsplit(const MfmaPlan &P, int64_t Mc, const DeviceInfo &dev, int *kcps) {
  const int64_t tiles = (int64_t)(P.Lt / 64) * ((Mc + 63) / 64);
  const int64_t cus = dev.cu_count > 0 ? dev.cu_count : 256;
  const int nkc = (int)((P.a + 31) / 32);
  int ns = (int)std::min<int64_t>(kMaxSplit, std::max<int64_t>(1, (cus + tiles - 1) / tiles));
  ns = std::min(ns, std::max(1, nkc / 8));  // at least two chunks per wave
  const int k = (nkc + ns - 1) / ns;
  *kcps = k;
  return (nkc + k - 1) / k;
}

size_t mfma_unit_ws_bytes(const MfmaPlan *p) {
  const size_t T = (size_t)round_up((int64_t)kMfmaRows * p->Lt * 2, 256);
  const size_t part = (size_t)kMaxSplit * (p->Lt / 64) * (kMfmaRows / 64) * 4096 * sizeof(float);
  return T + part;
}

size_t mfma_cnt_entries(const MfmaPlan *p) { return (size_t)(p->Lt / 64) * (kMfmaRows / 64); }

static hipError_t set_lds_attr(int device) {
  static std::atomic<uint64_t> done{0};
  const uint64_t bit = device >= 0 && device < 64 ? (1ull << device) : 0;
  if (bit && (done.load() & bit)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void *)k_unit_s1,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRedBytes);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void *)k_unit_s2, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kRedBytes);
  if (e == hipSuccess && bit) done.fetch_or(bit);
  return e;
}

hipError_t launch_mfma_unit(const MfmaPlan *p, const uint16_t *x, int64_t M,
                            uint16_t *const *y_layers, uint16_t *xout, float c_out, bool direct,
                            void *ws, unsigned *cnt, const DeviceInfo &dev, hipStream_t st) {
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
    A1.M = Mc;
    A1.a = (int)p->a;
    A1.a16 = p->a16;
    A1.Lt = p->Lt;
    A1.ntile32 = p->ntile32;
    A1.nsplit = s1_nsplit(*p, Mc, dev, &A1.kcps);
    A1.nseg = p->nseg;
    A1.xvec = (p->a % 8 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    for (int i = 0; i < kMaxUnitSegs; ++i) A1.seg[i] = p->seg[i];
    dim3 g1((unsigned)(p->Lt / 64), (unsigned)((Mc + 63) / 64), (unsigned)A1.nsplit);
    hipLaunchKernelGGL(k_unit_s1, g1, dim3(kThreads), kRedBytes, st, A1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    S2Args A2;
    A2.T = T;
    A2.xout = xout ? xout + mb * p->b : nullptr;
    A2.M = Mc;
    A2.b = (int)p->b;
    A2.Lt = p->Lt;
    A2.nl = p->nl;
    A2.direct = direct ? 1 : 0;
    A2.c_out = c_out;
    A2.pad_ = 0;
    for (int m = 0; m < kMaxUnitLayersM; ++m) {
      A2.ly[m] = p->ly[m];
      A2.ly[m].y = (m < p->nl && y_layers && y_layers[m]) ? y_layers[m] + mb * p->b : nullptr;
    }
    dim3 g2((unsigned)((p->b + 63) / 64), (unsigned)((Mc + 63) / 64));
    hipLaunchKernelGGL(k_unit_s2, g2, dim3(kThreads), kRedBytes, st, A2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lbi
