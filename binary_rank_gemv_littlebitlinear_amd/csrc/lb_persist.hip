// Persistent whole-stack sweep for one decode row (M = 1).
//
// [LB news] Sec. 2: each layer is two small binary products with
// elementwise scales; the residual path is a second factorisation whose
// output is added.  A stack chains layers (units of layers that share an
// input; unit outputs are combined in fp32 and rounded to fp16).
//
// One launch of G = #CU workgroups (one per CU) runs the whole sweep as
// U + 1 phases.  Workgroup w owns fixed 16-row tiles of every width, so
// the second product of unit u-1 (rows j), the combine and the first
// product of unit u (rows i = j) stay inside the workgroup:
//
//   phase 0 : X_0 rows -> partial t of unit 0 over own rows
//   phase u : t_{u-1} -> y rows of unit u-1 -> combine -> X_u rows
//             -> partial t of unit u over own rows
//   phase U : t_{U-1} -> y rows -> final combine -> output rows
//
// Products.  With S in {+-1}, sum_i s_i v_i is evaluated four signs at a
// time: for every group of four values a 16-entry table holds all sixteen
// signed sums, and each 4-bit nibble of a sign word selects one entry.  A
// wave reads at most 16 distinct entries of one table per lookup, which
// the LDS serves without bank conflicts.  The first product's tables are
// built from z = g * x over the workgroup's own rows (a thread looks up 1,
// 2 or 4 adjacent latent columns per bit read, the width chosen per unit
// on the host); the second product's tables from w = l * t.
//
// Issue.  Both products are bound by instruction issue on the busiest
// SIMD, not by data: scalar setup on the critical wave (a 64-bit division,
// say) shows up directly in the phase time.
//
// Memory.  The sign bits and scales a workgroup needs in a phase form a
// few contiguous blocks (layouts in lb_internal.h).  Waves 4-7 copy them
// into LDS with LDS-DMA loads while waves 0-3 run the previous phase's
// exchange (the partials are issued first, the copies right after), so
// HBM latency overlaps the device-wide synchronisation.
//
// Exchange.  Partial latent vectors (one per workgroup) are all-reduced
// between phases in three levels that follow the chip: 8 XCDs of 32 CUs,
// each XCD with its own L2, workgroup w on XCD w % 8 (checked when the plan
// is built).  Workgroup (x, i) = w with x = w % 8, i = w / 8 owns the
// slice i of ceil(Lu / 32) latent columns.
//   A  every workgroup stores its partials into its XCD's area; owner
//      (x, i) sums slice i over the 32 workgroups of XCD x;
//   B  owner (x, i) publishes that XCD sum device-wide and sums slice i
//      over the 8 XCDs, in XCD order (every XCD gets the same total);
//   C  owner (x, i) stores the total into XCD x's area, from which every
//      workgroup of XCD x builds the next phase's tables.
// Levels A and C never leave the XCD: their words are written with
// workgroup-scope stores, which stay in the XCD's L2, and read with
// device-scope loads, which skip the CU's L1 and find the line in that L2;
// only level B's 8-way slices cross XCDs (device-scope stores and loads).
// Every exchanged word is a 64-bit value | generation pair, so a reader
// knows a word is current from the word itself and no flag (or
// store-completion wait) is needed.  A launch takes its generation base
// from the tags the previous launch left, so a launch captured into a
// graph and replayed stays correct.  Every wait is bounded: on timeout a
// device error word (and a host-mapped copy) is set, all workgroups leave,
// and the next lb_stack_forward or lb_stack_check returns LB_ETIMEOUT.
#include <hip/hip_fp16.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "lb_persist.h"

namespace lbi {

constexpr int kThreads = 512;  // 8 waves: 0-3 exchange, 4-7 prefetch
constexpr int kWaves = kThreads / 64;
constexpr int kXThreads = 256;  // threads that touch exchange memory
constexpr int kTMax = 8;        // 16-row tiles per workgroup and width
constexpr int kMaxUnitLayers = 8;
constexpr int kLuMax = 2048;    // latent columns per unit
constexpr int kStgBytes = 56 * 1024;
constexpr int kTab2Floats = 11264;
// Table layouts (floats).  Every table is 16 entries, 64-byte aligned, so an
// entry address is the table address OR-ed with nibble * 4.  Blocks are
// padded by one table so that reads of neighbouring blocks by one wave land
// on the other half of the LDS banks instead of the same banks:
//   second product: a word's 8 tables form a block of kWordF floats; the
//   blocks of one (layer, path) form a set of s2_set_floats(Wk) floats,
//   rounded so that consecutive sets start on alternating bank halves;
//   first product: a 16-row tile's 4 tables form a block of kTileF floats;
//   the tiles of one (layer, path) form a set of s1_set_floats(nt) floats.
constexpr int kWordF = 8 * 16 + 16;
constexpr int kTileF = 4 * 16 + 16;
__host__ __device__ constexpr int s2_set_floats(int Wk) { return (Wk * kWordF + 31) / 32 * 32 + 16; }
__host__ __device__ constexpr int s1_set_floats(int nt) { return (nt * kTileF + 31) / 32 * 32 + 16; }
constexpr int kTab1Floats = 4096;
constexpr long kSpin = 4000000;      // polls before a wait gives up
constexpr long kSpinFailTest = 2048;  // the same in the host-requested failure test
constexpr int kXcd = 8;          // XCDs; workgroup w runs on XCD w % 8
constexpr int kPerXcd = 32;      // workgroups per XCD (the grid is 256 = one per CU)
constexpr int kSliceMax = kLuMax / kPerXcd;  // latent columns one owner sums

struct alignas(16) PLayer {
  const uint32_t *su2t;
  const uint16_t *sv16, *ht, *gt, *l;
  int a, b, s, P, L, Lp, Wk, a16, b16, s8;
  int col0;         // first latent column within the unit
  int tb2;          // offset (floats) of the layer's path-0 second-product tables; path p at
                    // + p s2_set_floats(Wk)
  int64_t trace_y;  // element offset of this layer's output in the trace
};

// One group of the second product's tables: 4 latent columns of one
// layer and path, built by one exchange thread from the reduced latent
// words tcol .. tcol + nval - 1 and their l (lp).
struct alignas(16) PGroup {
  const uint16_t *lp;
  int tcol;
  int nd;  // nval (0..4) | table offset in floats << 4
};

struct alignas(16) PUnit {
  int first, n;
  int a, b;
  int Lu;
  float c_out;      // kappa / sqrt(n): combine of this unit's outputs
  int64_t trace_x;  // element offset of this unit's input in the trace
  const PGroup *grp;  // the unit's table groups, in table order
  int ngrp;
  // first product: adjacent columns per thread for workgroups with nt0 row
  // tiles (bits 0-7) and with nt0 + 1 (bits 8-15); nt0 in bits 16-31
  int cpt;
};

// One block a workgroup copies into LDS for a phase: src + t0 * stride,
// fixed + nt * per_tile bytes (t0, nt: the workgroup's first tile and tile
// count).  A phase's list starts with a header record (per_tile = the
// phase's row width, fixed = record count).  Lists are kMaxSeg records
// apart, so the next phase's list is found without reading this one.
enum : int { kSegHeader = 0, kSegUnits = 1, kSegLayers = 2, kSegS2 = 3, kSegH = 4, kSegL = 5,
             kSegS1 = 6, kSegG = 7 };
constexpr int kMaxSeg = 3 + 5 * kMaxUnitLayers;

struct alignas(16) PSeg {
  const void *src;
  long long stride;
  int per_tile;
  int fixed;
  int kind;  // kind | layer << 8
  int offp;  // LDS offset in the staging buffer: (offp & 0xffff) + nt * (offp >> 16)
};

static_assert(sizeof(PLayer) % 16 == 0 && sizeof(PUnit) % 16 == 0 && sizeof(PSeg) == 32 &&
                  sizeof(PGroup) == 16,
              "descriptors are copied to LDS in 16-byte units");

struct PArgs {
  const PUnit *units;
  const PLayer *layers;
  int nunits;
  const uint16_t *x0;
  uint16_t *y;
  uint16_t *trace;  // may be null
  // tagged words (fp32 value bits | generation << 32)
  uint64_t *PA;  // [kXcd][kPerXcd][kLuMax] partials, in their XCD's L2
  uint64_t *PB;  // [2][kXcd][kLuMax] XCD sums of the slices (generation parity), device-wide
  uint64_t *PC;  // [kXcd][kLuMax] totals, in their XCD's L2
  int xcd_local;  // 1: levels A and C stay in the XCD's L2; 0: device-scope stores throughout
  unsigned *err;
  unsigned *herr;      // host-mapped copy of the error word (read by the next run on the host)
  uint64_t *timeline;  // optional [G][U+1][4] device timestamps (100 MHz)
  const PSeg *segs;    // [(U+1) * kMaxSeg] per-phase copy lists
  const PGroup *grp0;  // the first table group (a valid address for idle loads)
  unsigned wait_skew;  // added to the generation a wait expects: 0, nonzero only in
                       // the host-requested failure test (no wait can succeed;
                       // each gives up after kSpinFailTest polls)
  unsigned delay_seed;  // stress test: per-wave random delays at the exchange's
  unsigned delay_max;   // steps, up to delay_max ticks of 10 ns (0 = off)
};

struct PersistPlan {
  int device = 0;
  int G = 0;
  int nunits = 0, nlayers = 0;
  size_t lds = 0;
  PUnit *d_units = nullptr;
  PLayer *d_layers = nullptr;
  PSeg *d_segs = nullptr;
  PGroup *d_groups = nullptr;
  std::vector<PUnit> h_units;
  std::vector<PLayer> h_layers;
  uint64_t *PA = nullptr, *PB = nullptr, *PC = nullptr;
  int xcd_local = 0;
  unsigned *err = nullptr;  // 64 words; word 0 is the error word
  unsigned *herr = nullptr;      // pinned host word, set by a wait that gives up
  unsigned *herr_dev = nullptr;  // its device address
  bool fail_test = false;  // next sweeps: unsatisfiable waits with a short bound
  unsigned delay_seed = 0, delay_max = 0;  // next sweeps: random per-wave delays
  bool broken = false;
  uint64_t *timeline = nullptr;
};

// ----------------------------------------------------------- primitives
__device__ __forceinline__ float h2f(uint16_t v) { return __half2float(__ushort_as_half(v)); }
__device__ __forceinline__ uint16_t f2h(float v) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ unsigned ld_u(unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f(float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A tagged word: fp32 value bits in the low half, the generation in the
// high half (a running phase count carried from launch to launch in the
// tags themselves, plus the phase plus 1); one aligned 64-bit atomic
// store, so a reader sees the old word or the new one.
__device__ __forceinline__ void st_tag(uint64_t *p, float v, unsigned gen) {
  __hip_atomic_store(p, (uint64_t)__float_as_uint(v) | ((uint64_t)gen << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same word for readers on this XCD only: a workgroup-scope store
// leaves the line in this XCD's L2 (no write-through to memory), where the
// readers' device-scope loads find it.  With local == 0 (XCD placement not
// confirmed) it is a device-scope store.
__device__ __forceinline__ void st_tag_xcd(uint64_t *p, float v, unsigned gen, int local) {
  const uint64_t w = (uint64_t)__float_as_uint(v) | ((uint64_t)gen << 32);
  if (local)
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// N adjacent tagged words (N = 1, 2 or 4, the first one 8 N bytes
// aligned) for readers on this XCD: with local, plain stores of 8 N bytes
// (as the workgroup-scope store above; an aligned 8-byte word within one
// vector store is never torn), else one device-scope store per word.
template <int N>
__device__ __forceinline__ void st_tags_xcd(uint64_t *p, const float (&v)[N], unsigned gen,
                                            int local) {
  uint64_t w[N];
#pragma unroll
  for (int k = 0; k < N; ++k) w[k] = (uint64_t)__float_as_uint(v[k]) | ((uint64_t)gen << 32);
  if (local && N == 4) {
    reinterpret_cast<ulonglong2 *>(p)[0] = make_ulonglong2(w[0], w[1]);
    reinterpret_cast<ulonglong2 *>(p)[1] = make_ulonglong2(w[2], w[3]);
  } else if (local && N == 2) {
    reinterpret_cast<ulonglong2 *>(p)[0] = make_ulonglong2(w[0], w[1]);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) st_tag_xcd(p + k, v[k], gen, local);
  }
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// 16-row tiles [t0, t1) owned by workgroup w out of `tiles`.
// tiles <= kTMax G (checked when the plan is built), so tiles (w + 1) fits
// in 32 bits and the division is a 32-bit one.
__device__ __forceinline__ void my_tiles(int tiles, int G, int w, int &t0, int &t1) {
  t0 = (int)((unsigned)(tiles * w) / (unsigned)G);
  t1 = (int)((unsigned)(tiles * (w + 1)) / (unsigned)G);
}

// Block-wide AND through LDS only (waits on LDS, never on global memory).
// ------------------------------------------------------ LDS arrangement
// Everything a phase reads besides its tables lives in LDS: the staged
// sign bits and scales, and a copy of the descriptors of the two units the
// phase touches (unit A = ph-1 for the second product, unit B = ph for the
// first), so the compute never waits on global memory.
struct PhaseCtx {
  PUnit ua, ub;                       // copied by LDS-DMA (adjacent units)
  PLayer la[2 * kMaxUnitLayers];      // layers of A, then of B (copied by LDS-DMA)
  int has_a;                          // the phase has a second product (ph > 0)
  int t0, t1;                         // row tiles of the phase
  int s2_off[kMaxUnitLayers], h_off[kMaxUnitLayers], l_off[kMaxUnitLayers];
  int s1_off[kMaxUnitLayers], g_off[kMaxUnitLayers];
};

// The LDS regions after the context start at multiples of 64 bytes, so a
// 16-entry table's address has its entry index in bits 2..5 (or-ed in).
constexpr size_t kCtxBytes = (sizeof(PhaseCtx) + 63) / 64 * 64;
static_assert((2 * kMaxSeg * sizeof(PSeg)) % 64 == 0 && kStgBytes % 64 == 0 && (kTab2Floats * 4) % 64 == 0,
              "table regions 64-byte aligned");

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}
__device__ __forceinline__ float lds_f32(uint32_t a) {
  return *(const __attribute__((address_space(3))) float *)(uintptr_t)a;
}
__device__ __forceinline__ uint32_t lds_u32(uint32_t a) {
  return *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)a;
}
__device__ __forceinline__ uint2 lds_u64(uint32_t a) {
  typedef unsigned int u2v __attribute__((ext_vector_type(2)));
  const u2v v = *(const __attribute__((address_space(3))) u2v *)(uintptr_t)a;
  return make_uint2(v.x, v.y);
}
// Byte offset of entry (w >> sh) & 15 of a 16-float table.
template <int sh>
__device__ __forceinline__ uint32_t nib_off(uint32_t w) {
  if constexpr (sh >= 2) return (w >> (sh - 2)) & 0x3cu;
  else return (w << (2 - sh)) & 0x3cu;
}

struct Lds {
  unsigned char *stg;  // kStgBytes staged bits and scales of the phase
  float *tab2;         // kTab2Floats second-product tables
  float *tab1;         // kTab1Floats first-product tables
  float *acc2;         // kMaxUnitLayers * 2 * 16 * kTMax
  float *xs;           // 16 * kTMax input rows (fp16 values as fp32)
  float *red;          // kXThreads exchange scratch
  int *flags8;         // kWaves
  int *xcnt;           // level-A arrivals of the exchange waves (grows by 4 a phase)
  PhaseCtx *ctx;
  PSeg *segbuf;        // [2][kMaxSeg] copy lists of this and the next phase
  uint64_t *tl;        // diagnostics: this workgroup's timestamps, or null
};

// Diagnostics: timestamp k of phase ph (100 MHz counter), thread 0 only.
constexpr int kStamps = 8;
__device__ __forceinline__ void stamp(const Lds &L, int ph, int k) {
  if (L.tl && threadIdx.x == 0) L.tl[ph * kStamps + k] = __builtin_amdgcn_s_memrealtime();
}

// Stage phase ph: copy the blocks of its list (descriptors of units ph-1
// and ph, sign bits, scales) into LDS with LDS-DMA loads (16 bytes per
// lane, 1 KB per wave instruction), and the next phase's list into the
// other list buffer.  Waves 4-7 only: wave 4 + i takes records 1 + i,
// 5 + i, ...  It reads all of its records with one vector LDS load and
// takes their fields with readlane, so the issue loop has no LDS reads
// (they would queue behind the incoming copies), and the host-computed
// block offsets need no running sum.
__device__ void stage_phase(const PArgs &A, int ph, Lds &L) {
  const int G = gridDim.x;
  const PSeg *lst = L.segbuf + (ph & 1) * kMaxSeg;
  const uint32_t *lw = reinterpret_cast<const uint32_t *>(lst);
  const int pw = wave_id() - 4;  // 0..3
  const int lane = threadIdx.x & 63;
  const int width = lst[0].per_tile, nseg = lst[0].fixed;
  // record 1 + pw + 4 j, dword f, for j = 8 b + (lane >> 3), f = lane & 7
  uint32_t rv0, rv1;
  {
    const int k0 = 1 + pw + 4 * (lane >> 3), k1 = k0 + 32;
    rv0 = k0 < kMaxSeg ? lw[k0 * 8 + (lane & 7)] : 0u;
    rv1 = k1 < kMaxSeg ? lw[k1 * 8 + (lane & 7)] : 0u;
  }
  int t0, t1;
  my_tiles((width + 15) / 16, G, blockIdx.x, t0, t1);
  const int nt = t1 - t0;
  PhaseCtx &C = *L.ctx;
  if (pw == 0 && lane == 0) {
    C.has_a = ph > 0;
    C.t0 = t0;
    C.t1 = t1;
  }
  auto copy = [&](const char *src, unsigned char *dst, int nbytes) {
    const int units = nbytes / 16;
    const int nch = (units + 63) / 64;
    for (int c = 0; c < nch; ++c) {
      const int u = c * 64 + lane;
      if (u < units) __builtin_amdgcn_global_load_lds(src + (size_t)u * 16, dst + c * 1024, 16, 0, 0);
    }
  };
  for (int j = 0; 1 + pw + 4 * j < nseg; ++j) {
    const uint32_t v = j < 8 ? rv0 : rv1;
    const int base = 8 * (j & 7);
    // readlane returns int: every field goes through uint32_t before it is
    // widened, so a low word with bit 31 set is not sign-extended
    uint32_t f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (uint32_t)__builtin_amdgcn_readlane((int)v, base + i);
    const uint64_t srcv = (uint64_t)f[0] | ((uint64_t)f[1] << 32);
    const int64_t stride = (int64_t)((uint64_t)f[2] | ((uint64_t)f[3] << 32));
    const int per_tile = (int)f[4], fixed = (int)f[5], kindm = (int)f[6];
    const uint32_t offp = f[7];
    const int bytes = fixed + nt * per_tile;
    const char *src = reinterpret_cast<const char *>(srcv) + (int64_t)t0 * stride;
    const int kind = kindm & 255, m = kindm >> 8;
    unsigned char *dst;
    if (kind == kSegUnits) {
      dst = reinterpret_cast<unsigned char *>(ph > 0 ? &C.ua : &C.ub);
    } else if (kind == kSegLayers) {
      dst = reinterpret_cast<unsigned char *>(C.la);
    } else {
      const int off = (int)(offp & 0xffffu) + nt * (int)(offp >> 16);
      dst = L.stg + off;
      if (lane == 0) {
        if (kind == kSegS2) C.s2_off[m] = off;
        else if (kind == kSegH) C.h_off[m] = off;
        else if (kind == kSegL) C.l_off[m] = off;
        else if (kind == kSegS1) C.s1_off[m] = off;
        else if (kind == kSegG) C.g_off[m] = off;
      }
    }
    copy(src, dst, bytes);
  }
  if (ph < A.nunits && pw == 3)
    copy(reinterpret_cast<const char *>(A.segs + (size_t)(ph + 1) * kMaxSeg),
         reinterpret_cast<unsigned char *>(L.segbuf + ((ph + 1) & 1) * kMaxSeg), kMaxSeg * 32);
}

// Entries lo + 4*hi (lo = 0..3) of the table over (v0, v1, v2, v3), entry
// e = sum_j (bit j of e ? v_j : -v_j), summed as ((+-v0 +- v1) + (+-v2 +- v3)).
__device__ __forceinline__ void table_quad(float *tab, float v0, float v1, float v2, float v3,
                                           int hi) {
  const float hs = ((hi & 1) ? v2 : -v2) + ((hi & 2) ? v3 : -v3);
  float4 e;
  e.x = (-v0 - v1) + hs;
  e.y = (v0 - v1) + hs;
  e.z = (-v0 + v1) + hs;
  e.w = (v0 + v1) + hs;
  *reinterpret_cast<float4 *>(tab + 4 * hi) = e;
}

// The value of lane i of this lane's quad (lanes 4k .. 4k + 3), by a DPP
// lane move; every lane of the quad must be active.
template <int i>
__device__ __forceinline__ float quad_lane(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), i * 0x55, 0xf, 0xf, false));
}

// ceil(2^32 / n) for 1 <= n <= kTMax (the division for larger n).
__device__ __forceinline__ uint64_t ceil_recip32(int n) {
  static_assert(kTMax == 8, "constants for n <= 8");
  switch (n) {
    case 1: return 0x100000000ull;
    case 2: return 0x80000000ull;
    case 3: return 0x55555556ull;
    case 4: return 0x40000000ull;
    case 5: return 0x33333334ull;
    case 6: return 0x2aaaaaabull;
    case 7: return 0x24924925ull;
    case 8: return 0x20000000ull;
    default: return (0x100000000ull + (unsigned)n - 1) / (unsigned)n;
  }
}

// ----------------------------------------------------------- products
// The phase context lives in LDS.  Every function below first loads the
// context fields it needs for all layers at once (unconditional loads, so
// they are in flight together) and only then branches on them; a chain
// of dependent LDS reads costs ~0.1 us per link.

// The second product's lookups of one task: its words q = sub, sub + lpt,
// ... below Wk, R words per step.  Every read is unconditional (index
// clamped, result masked), and all 8 R table reads of a step are gathered
// before any is summed (a tree per word), so they are in flight at once
// instead of each waiting for the previous one's sum; the words are added
// to the total in order.
template <int R>
__device__ __forceinline__ float s2_words(const uint32_t *wb, uint32_t tba, int sub, int lpt,
                                          int Wk) {
  float acc = 0.f;
  for (int q = sub; q < Wk; q += R * lpt) {
    uint32_t wd[R];
#pragma unroll
    for (int i = 0; i < R; ++i) wd[i] = wb[min(q + i * lpt, Wk - 1) * 16];
    float v[R][8];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      // the word's 8 tables are one block: entry address =
      // block | nibble * 4, table n at immediate offset 64 n
      const uint32_t tq = tba + 4u * kWordF * (uint32_t)min(q + i * lpt, Wk - 1);
      const uint32_t w = wd[i];
      v[i][0] = lds_f32(tq | nib_off<0>(w));
      v[i][1] = lds_f32((tq | nib_off<4>(w)) + 64);
      v[i][2] = lds_f32((tq | nib_off<8>(w)) + 128);
      v[i][3] = lds_f32((tq | nib_off<12>(w)) + 192);
      v[i][4] = lds_f32((tq | nib_off<16>(w)) + 256);
      v[i][5] = lds_f32((tq | nib_off<20>(w)) + 320);
      v[i][6] = lds_f32((tq | nib_off<24>(w)) + 384);
      v[i][7] = lds_f32((tq | nib_off<28>(w)) + 448);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float e = ((v[i][0] + v[i][1]) + (v[i][2] + v[i][3])) +
                      ((v[i][4] + v[i][5]) + (v[i][6] + v[i][7]));
      acc += q + i * lpt < Wk ? e : 0.f;
    }
  }
  return acc;
}

// Second product of unit A over the workgroup's rows: every layer's fp16
// outputs (trace), their combine, and the output rows on the last phase or
// else the first-product tables of unit B over the combined rows.
__device__ void second_product(const PArgs &A, int ph, Lds &L) {
  const PhaseCtx &C = *L.ctx;
  const PUnit &U = C.ua;
  const int na = U.n, ub = U.b;
  const int t0 = C.t0, nt = C.t1 - C.t0, rows = 16 * nt;
  int Pm[kMaxUnitLayers];
#pragma unroll
  for (int m = 0; m < kMaxUnitLayers; ++m) Pm[m] = C.la[m].P;
  // lookups: task = (layer, path, row) over every layer and both path
  // slots; lpt lanes of a task split its words.  The task's pair index is
  // (task / 16) / nt, by a 64-bit multiply with a per-phase constant.  The
  // layer's fields come from indexed LDS reads; its tables (a group is 4
  // latent columns with a 16-entry table) were built by the previous exchange.
  if (rows > 0) {
    const int ntk = na * 2 * rows;
    int lpt = 1, lg = 0;
    while (lpt < 64 && ntk * lpt * 2 <= kThreads) {
      lpt *= 2;
      ++lg;
    }
    // ceil(2^32 / nt) (33 bits for nt = 1: the product is taken in 64 bits),
    // from a constant for nt <= kTMax rather than a 64-bit division
    const uint64_t magic = ceil_recip32(nt);
    const int sub = threadIdx.x & (lpt - 1);
    for (int tk0 = 0; tk0 < ntk; tk0 += kThreads >> lg) {
      const int tk = tk0 + ((int)threadIdx.x >> lg);
      const int mp = (int)(((uint64_t)((unsigned)tk >> 4) * magic) >> 32), r = tk - mp * rows;
      const int m = tk < ntk ? mp >> 1 : 0, p = mp & 1;
      const PLayer &Ly = C.la[m];
      const int P = Ly.P, Wk = Ly.Wk, s2o = C.s2_off[m];
      const uint32_t tba = lds_addr(L.tab2) + 4u * (uint32_t)(Ly.tb2 + p * s2_set_floats(Wk));
      float acc = 0.f;
      if (tk < ntk && p < P) {
        const uint32_t *wb = reinterpret_cast<const uint32_t *>(L.stg + s2o) +
                             ((size_t)((r >> 4) * P + p) * Wk) * 16 + (r & 15);
        // R words per step: 4, or 5 where that takes fewer steps for the
        // task's first lane (the same choice for every lane of a task; the
        // sum order does not depend on it)
        const int wpt = (Wk + lpt - 1) >> lg;
        if ((wpt + 4) / 5 < (wpt + 3) / 4)
          acc = s2_words<5>(wb, tba, sub, lpt, Wk);
        else
          acc = s2_words<4>(wb, tba, sub, lpt, Wk);
      }
      for (int o = 1; o < lpt; o <<= 1) acc += __shfl_xor(acc, o, 64);
      if (sub == 0 && tk < ntk) L.acc2[mp * (16 * kTMax) + r] = acc;
    }
  }
  stamp(L, ph, 1);
  // per-layer offsets for the epilogue, loaded before the barrier
  int hoff[kMaxUnitLayers];
  int64_t trace_y[kMaxUnitLayers];
#pragma unroll
  for (int m = 0; m < kMaxUnitLayers; ++m) {
    hoff[m] = C.h_off[m];
    trace_y[m] = C.la[m].trace_y;
  }
  const float c_out = U.c_out;
  const int64_t trace_x = C.ub.trace_x;
  __syncthreads();
  // epilogue, a thread per row r in each of four groups of 128 threads: y
  // per layer, the combine and (group 0) the output row.  The combined rows
  // are the next unit's input, so the same threads build its first
  // product's tables from them, group jg taking pairs jg, jg + 4, ...: the
  // four lanes of rows 4 qd .. 4 qd + 3 (one quad of a wave) share their
  // z = g * x values by lane moves, and lane k writes entries 4 k .. 4 k + 3
  // of the pair's table of that quad.
  {
    const bool next = ph < A.nunits;
    const PLayer *LB = C.la + na;
    const int Pu = next ? LB[0].P : 1;
    const int npairs = next ? C.ub.n * Pu : 0;
    int goff[kMaxUnitLayers];
#pragma unroll
    for (int m = 0; m < kMaxUnitLayers; ++m) goff[m] = C.g_off[m];
    static_assert(16 * kTMax <= kThreads / 4, "a group of threads per 128 rows");
    const int r = threadIdx.x & (kThreads / 4 - 1), jg = threadIdx.x / (kThreads / 4);
    if (r < rows && (jg == 0 || jg < npairs)) {
      const int j = 16 * t0 + r;
      float ys = 0.f;
#pragma unroll
      for (int m = 0; m < kMaxUnitLayers; ++m) {
        if (m >= na) break;
        const uint16_t *hv = reinterpret_cast<const uint16_t *>(L.stg + hoff[m]);
        const int P = Pm[m];
        float yv = h2f(hv[((r >> 4) * P) * 16 + (r & 15)]) * L.acc2[(m * 2) * (16 * kTMax) + r];
        if (P > 1) yv += h2f(hv[((r >> 4) * P + 1) * 16 + (r & 15)]) * L.acc2[(m * 2 + 1) * (16 * kTMax) + r];
        const uint16_t y16 = f2h(yv);
        if (jg == 0 && j < ub && A.trace) A.trace[trace_y[m] + j] = y16;
        ys += h2f(y16);
      }
      const uint16_t xv = f2h(c_out * ys);
      const float xr = j < ub ? h2f(xv) : 0.f;
      if (jg == 0 && j < ub) {
        if (!next)
          A.y[j] = xv;
        else if (A.trace)
          A.trace[trace_x + j] = xv;
      }
      // rows is a multiple of 16, so every quad of lanes is whole here
      const int qd = r >> 2, hi = r & 3;
      for (int jt = jg; jt < npairs; jt += kThreads / (kThreads / 4)) {
        const int m = Pu == 2 ? jt >> 1 : jt, p = jt - m * Pu;
        const uint16_t *gv = reinterpret_cast<const uint16_t *>(L.stg + goff[m]);
        const float v = h2f(gv[((r >> 4) * Pu + p) * 16 + (r & 15)]) * xr;
        const float v0 = quad_lane<0>(v), v1 = quad_lane<1>(v), v2 = quad_lane<2>(v),
                    v3 = quad_lane<3>(v);
        table_quad(L.tab1 + jt * s1_set_floats(nt) + (qd >> 2) * kTileF + (qd & 3) * 16, v0, v1,
                   v2, v3, hi);
      }
    }
  }
  __syncthreads();
}

// The first product's lookups: a thread takes CPT adjacent columns of one
// layer (CPT divides every layer's column count, so a group never spans
// two layers), and lpt lanes split the group's nt 16-row words; one LDS
// read gives a tile's bits of all CPT columns.  Per column and tile the four
// entries are summed as ((q0 + q1) + (q2 + q3)) and added in tile order.
// The column's partial goes straight from the register to the workgroup's
// slot of its XCD's exchange area (level A of the exchange), tagged.
template <int CPT>
__device__ __forceinline__ void s1_lookups(Lds &L, const PhaseCtx &C, const PLayer *LB, int nb,
                                           int Lu, int nt, int Pu,
                                           const int (&col0m)[kMaxUnitLayers], uint64_t *pa,
                                           unsigned gen, int xcd_local) {
  const int ngr = Lu / CPT;
  int lpt = 1, lg = 0;
  while (lpt < 64 && lpt < nt && ngr * lpt * 2 <= kThreads) {
    lpt *= 2;
    ++lg;
  }
  const int sub = threadIdx.x & (lpt - 1);
  const uint32_t taba = lds_addr(L.tab1), stga = lds_addr(L.stg);
  constexpr uint32_t kTileBytes = 4u * kTileF;  // the block of one pair and tile
  const uint32_t kPairBytes = 4u * (uint32_t)s1_set_floats(nt);
  for (int q0 = 0; q0 < ngr; q0 += kThreads >> lg) {
    const int q = q0 + ((int)threadIdx.x >> lg);
    float acc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = 0.f;
    if (q < ngr) {
      const int c = q * CPT;
      int m = 0;
#pragma unroll
      for (int i = 1; i < kMaxUnitLayers; ++i)
        if (i < nb && col0m[i] <= c) m = i;
      const PLayer &Ly = LB[m];
      const int cl = c - Ly.col0, s = Ly.s, Lp = Ly.Lp, s1o = C.s1_off[m];
      const uint32_t wa = stga + (uint32_t)(s1o + 2 * cl), wstride = 2u * (uint32_t)Lp;
      uint32_t tq[CPT];  // the column's tile-0 tables (its path's)
#pragma unroll
      for (int j = 0; j < CPT; ++j)
        tq[j] = taba + kPairBytes * (uint32_t)(m * Pu + (cl + j < s ? 0 : 1));
      for (int g0 = sub; g0 < nt; g0 += 2 * lpt) {
        uint32_t wd[2][(CPT + 1) / 2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t a = wa + (uint32_t)min(g0 + i * lpt, nt - 1) * wstride;
          if constexpr (CPT == 4) {
            const uint2 v = lds_u64(a);
            wd[i][0] = v.x;
            wd[i][1] = v.y;
          } else if constexpr (CPT == 2) {
            wd[i][0] = lds_u32(a);
          } else {
            wd[i][0] = *(const __attribute__((address_space(3))) uint16_t *)(uintptr_t)a;
          }
        }
        // every table read of the step first, then the sums: the reads are
        // all in flight together rather than pairwise behind each sum
        float v[2][CPT][4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t toff = kTileBytes * (uint32_t)min(g0 + i * lpt, nt - 1);
#pragma unroll
          for (int j = 0; j < CPT; ++j) {
            const uint32_t w = wd[i][j >> 1], tb = tq[j] + toff;
            if ((j & 1) == 0) {
              v[i][j][0] = lds_f32(tb | nib_off<0>(w));
              v[i][j][1] = lds_f32((tb | nib_off<4>(w)) + 64);
              v[i][j][2] = lds_f32((tb | nib_off<8>(w)) + 128);
              v[i][j][3] = lds_f32((tb | nib_off<12>(w)) + 192);
            } else {
              v[i][j][0] = lds_f32(tb | nib_off<16>(w));
              v[i][j][1] = lds_f32((tb | nib_off<20>(w)) + 64);
              v[i][j][2] = lds_f32((tb | nib_off<24>(w)) + 128);
              v[i][j][3] = lds_f32((tb | nib_off<28>(w)) + 192);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int gi = g0 + i * lpt;
#pragma unroll
          for (int j = 0; j < CPT; ++j) {
            const float e = (v[i][j][0] + v[i][j][1]) + (v[i][j][2] + v[i][j][3]);
            acc[j] += gi < nt ? e : 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      for (int o = 1; o < lpt; o <<= 1) acc[j] += __shfl_xor(acc[j], o, 64);
    }
    if (sub == 0 && q < ngr) st_tags_xcd<CPT>(&pa[q * CPT], acc, gen, xcd_local);
  }
}

// First product of unit B over the workgroup's rows: the partial of every
// latent column of every layer of the unit, published tagged into this
// workgroup's slot of its XCD's exchange area.  In phase 0 the tables are
// built here from the input rows (xs); later phases find them built by the
// second product's epilogue.
__device__ void first_product(const PArgs &A, Lds &L, int ph, unsigned gen) {
  const PhaseCtx &C = *L.ctx;
  const PUnit &U = C.ub;
  const int nb = U.n, Lu = U.Lu;
  const PLayer *LB = C.la + (C.has_a ? C.ua.n : 0);
  const int nt = C.t1 - C.t0, quads = 4 * nt;
  const int w = blockIdx.x;
  uint64_t *pa = A.PA + ((size_t)(w % kXcd) * kPerXcd + w / kXcd) * kLuMax;
  if (nt == 0) {
    for (int c = threadIdx.x; c < Lu; c += kThreads) st_tag_xcd(&pa[c], 0.f, gen, A.xcd_local);
    return;
  }
  // every layer of a unit has the same path count Pu; pair j = m Pu + p
  // (layer m, path p) has its tile blocks at tab1 + j * s1_set_floats(nt)
  const int Pu = LB[0].P;
  if (ph == 0) {
    // tables from z = g * x: thread t builds the table of quad t % 32 of pair t / 32
    const int j = (int)threadIdx.x >> 5, qd = (int)threadIdx.x & 31;
    const int m = Pu == 2 ? j >> 1 : j, p = j - m * Pu;
    if (m < nb && qd < quads) {
      const uint16_t *gv = reinterpret_cast<const uint16_t *>(L.stg + C.g_off[m]);
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 4 * qd + k;
        v[k] = h2f(gv[((r >> 4) * Pu + p) * 16 + (r & 15)]) * L.xs[r];
      }
      float *tab = L.tab1 + j * s1_set_floats(nt) + (qd >> 2) * kTileF + (qd & 3) * 16;
#pragma unroll
      for (int hi = 0; hi < 4; ++hi) table_quad(tab, v[0], v[1], v[2], v[3], hi);
    }
    __syncthreads();
  }
  int col0m[kMaxUnitLayers];
#pragma unroll
  for (int m = 0; m < kMaxUnitLayers; ++m) col0m[m] = LB[m].col0;
  const int cpt = nt == (U.cpt >> 16) ? (U.cpt & 255) : ((U.cpt >> 8) & 255);
  stamp(L, ph, 3);
  if (cpt == 4) s1_lookups<4>(L, C, LB, nb, Lu, nt, Pu, col0m, pa, gen, A.xcd_local);
  else if (cpt == 2) s1_lookups<2>(L, C, LB, nb, Lu, nt, Pu, col0m, pa, gen, A.xcd_local);
  else s1_lookups<1>(L, C, LB, nb, Lu, nt, Pu, col0m, pa, gen, A.xcd_local);
}

// -------------------------------------------------------- the exchange
// The partials every workgroup published (first_product) -> the next
// phase's second-product tables over their sum, in the three levels
// described at the top of this file.  Each level costs one store and one
// read (plus re-reads while words are missing).  Levels A and B run on
// the first kXThreads threads, level C on all of them; every spin is
// bounded and checks the error word every 64 rounds.

// Wait (per thread) until the words at p(k), k < N with valid(k),
// carry gen; their values go to vals.  False on give-up or error.
template <class Ptr, class Valid, int N>
__device__ __forceinline__ bool spin_tagged(Ptr p, Valid valid, unsigned gen, unsigned *err,
                                            unsigned *herr, bool fail_test, float (&vals)[N]) {
  static_assert(N <= 32, "one pending bit per word");
  unsigned pend = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    vals[k] = 0.f;
    if (valid(k)) pend |= 1u << k;
  }
  long spins = 0;
  while (pend) {
    uint64_t wds[N];
#pragma unroll
    for (int k = 0; k < N; ++k) wds[k] = ((pend >> k) & 1u) ? ld_tag(p(k)) : 0ull;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (((pend >> k) & 1u) && (unsigned)(wds[k] >> 32) == gen) {
        vals[k] = __uint_as_float((unsigned)wds[k]);
        pend &= ~(1u << k);
      }
    if (pend && (++spins & 63) == 0) {
      if (ld_u(err) != 0) return false;
      if (spins > kSpin || (fail_test && spins > kSpinFailTest)) {
        atomicOr(err, 1u);
        __hip_atomic_store(herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return false;
      }
    }
  }
  return true;
}

// The second product's tables of the next phase (unit B of this phase):
// group g (4 latent columns of one layer and path) is built by thread
// g % 512 from the reduced latent words and l (every wave takes part in
// level C, so a thread has at most one group up to 512 groups).  The groups are
// listed on the host; a thread loads its own at the start of the phase, so
// the loads are long done when the exchange needs them.
constexpr int kGroupsPerThread = (kTab2Floats / 16 + kThreads - 1) / kThreads;
struct TabPlan {
  int n;                                 // groups of this thread
  int tcol[kGroupsPerThread];            // latent column of the group's first word
  int nval[kGroupsPerThread];            // valid columns (< s) of the group, 0..4
  int dst[kGroupsPerThread];             // table offset in tab2 (floats)
  const uint16_t *lp[kGroupsPerThread];  // l of the group (global)
};

__device__ TabPlan load_tables(const PArgs &A, const Lds &L, bool live) {
  const PUnit &UB = L.ctx->ub;
  // every load is unconditional (index clamped into a valid list), so the
  // three are in flight together and nothing waits for them before the
  // exchange uses them
  const PGroup *gp = live ? UB.grp : A.grp0;
  const int ng = live ? UB.ngrp : 0;
  const int gmax = (live ? ng : 1) - 1;
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(1))) u4v *global_u4;
  const global_u4 gg = (global_u4)(uintptr_t)gp;  // a device-memory list: global, not flat, loads
  TabPlan T;
  T.n = 0;
#pragma unroll
  for (int i = 0; i < kGroupsPerThread; ++i) {
    const int g = (int)threadIdx.x + i * kThreads;
    const bool v = g < ng;
    const u4v rv = gg[min(g, gmax)];
    const uint4 raw = v ? make_uint4(rv.x, rv.y, rv.z, rv.w) : make_uint4(0u, 0u, 0u, 0u);
    T.lp[i] = reinterpret_cast<const uint16_t *>((uint64_t)raw.x | ((uint64_t)raw.y << 32));
    T.tcol[i] = (int)raw.z;
    T.nval[i] = (int)(raw.w & 15u);
    T.dst[i] = (int)(raw.w >> 4);
    if (v) T.n = i + 1;
  }
  return T;
}

// Stress test of the exchange ordering: when the host asks for it, each
// wave waits a pseudo-random time (a hash of the seed, the generation, the
// workgroup, the wave and the site; zero for about half of the draws, else
// up to delay_max ticks of the 100 MHz clock) before a step, so that
// publishes, the LDS meeting after level A, the cross-XCD store and the
// polls happen in orders the undisturbed sweep never shows.  The results
// must not change: every sum has a fixed order.
// The sweep is compiled twice: with kDelay false (every normal launch) these
// calls are empty, so the stress hooks cost the timed kernel nothing.
template <bool kDelay>
__device__ __forceinline__ void test_delay(const PArgs &A, unsigned gen, int site) {
  if (!kDelay || A.delay_max == 0u) return;
  unsigned h = A.delay_seed ^ (gen * 0x9E3779B1u) ^ ((unsigned)blockIdx.x * 0x85EBCA77u) ^
               ((unsigned)wave_id() * 0xC2B2AE3Du) ^ ((unsigned)site * 0x27D4EB2Fu);
  h ^= h >> 16; h *= 0x7FEB352Du; h ^= h >> 15; h *= 0x846CA68Bu; h ^= h >> 16;
  if (h & 1u) return;
  const uint64_t ticks = (h >> 1) % A.delay_max;
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
}

// Second half: levels A (owned slice over the XCD), B (over the XCDs) and C
// (the totals, straight into the next phase's tables).
static_assert(kXThreads == 4 * 64 && kPerXcd == 4 * 8 && kSliceMax <= 64,
              "level A: wave v sums producers v, v + 4, ...; a lane per column");
template <bool kDelay>
__device__ bool exchange_collect(Lds &L, int Lu, unsigned gen, const PArgs &A, const TabPlan &tp,
                                 int ph) {
  const int w = blockIdx.x, t = threadIdx.x;
  const int x = w % kXcd, li = w / kXcd, lane = t & 63, wv = t >> 6;
  const bool xw = t < kXThreads;
  const int sw = (Lu + kPerXcd - 1) / kPerXcd;
  const int c0 = li * sw, nsc = max(0, min(Lu, c0 + sw) - c0);
  const unsigned gw = gen + A.wait_skew;
  const bool ftest = A.wait_skew != 0;
  bool ok = true;
  // level A: wave wv, lane c sums column c0 + c over producers wv, wv + 4, ...
  // The four exchange waves meet through an LDS counter, not a workgroup
  // barrier: waves 4-7 are still issuing the next phase's copies, and
  // waiting for them would put that issue time on the critical path.
  test_delay<kDelay>(A, gen, 1);
  if (xw) {
    float v = 0.f;
    if (lane < nsc) {
      float vals[8];
      const uint64_t *pa = A.PA + (size_t)x * kPerXcd * kLuMax + c0 + lane;
      ok = spin_tagged([&](int k) { return const_cast<uint64_t *>(pa + (size_t)(wv + 4 * k) * kLuMax); },
                       [&](int) { return true; }, gw, A.err, A.herr, ftest, vals);
#pragma unroll
      for (int k = 0; k < 8; ++k) v += vals[k];
    }
    L.red[wv * 64 + lane] = v;
    // a wave's LDS operations complete in order: its sums land before its count
    if (lane == 0) atomicAdd(L.xcnt, 1);
    if (wv < 2) {
      const int target = 4 * (ph + 1);
      long sp = 0;
      while (__hip_atomic_load(L.xcnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target &&
             ++sp < kSpin) {
      }
    }
  }
  stamp(L, ph, 5);
  // level B, lane c: the XCD sum of column c0 + c is published by wave 1 and
  // summed over the XCDs by wave 0 (its own XCD's term from LDS), so the
  // polling wave never waits behind the acknowledgement of its own store;
  // the total goes to this XCD's area (level C)
  test_delay<kDelay>(A, gen, 2);
  if (wv < 2 && lane < nsc) {
    const float xs = (L.red[lane] + L.red[64 + lane]) + (L.red[128 + lane] + L.red[192 + lane]);
    uint64_t *pb = A.PB + (size_t)(gen & 1) * kXcd * kLuMax + c0 + lane;
    if (wv == 1) {
      st_tag(pb + (size_t)x * kLuMax, xs, gen);
    } else if (ok) {
      float vals[kXcd];
      ok = spin_tagged([&](int k) { return pb + (size_t)k * kLuMax; }, [&](int k) { return k != x; },
                       gw, A.err, A.herr, ftest, vals);
      float tot = 0.f;
#pragma unroll
      for (int k = 0; k < kXcd; ++k) tot += k == x ? xs : vals[k];
      st_tag_xcd(A.PC + (size_t)x * kLuMax + c0 + lane, tot, gen, A.xcd_local);
    }
  }
  stamp(L, ph, 6);
  // level C, straight into the next phase's tables: w = l * t per group
  uint64_t *pc = A.PC + (size_t)x * kLuMax;
  test_delay<kDelay>(A, gen, 3);
  {
    uint2 lraw[kGroupsPerThread];  // 4 fp16 l per group
#pragma unroll
    for (int i = 0; i < kGroupsPerThread; ++i)
      lraw[i] = i < tp.n ? *reinterpret_cast<const uint2 *>(tp.lp[i]) : make_uint2(0u, 0u);
    // every group's words in one wait, so a thread with several groups
    // polls them together rather than one round trip after another
    float tv[4 * kGroupsPerThread];
    ok = ok && spin_tagged([&](int k) { return &pc[tp.tcol[k >> 2] + (k & 3)]; },
                           [&](int k) { return (k >> 2) < tp.n && (k & 3) < tp.nval[k >> 2]; },
                           gw, A.err, A.herr, ftest, tv);
#pragma unroll
    for (int i = 0; i < kGroupsPerThread; ++i) {
      if (i >= tp.n) break;
      const float w0 = tp.nval[i] > 0 ? h2f((uint16_t)(lraw[i].x & 0xffffu)) * tv[4 * i] : 0.f;
      const float w1 = tp.nval[i] > 1 ? h2f((uint16_t)(lraw[i].x >> 16)) * tv[4 * i + 1] : 0.f;
      const float w2 = tp.nval[i] > 2 ? h2f((uint16_t)(lraw[i].y & 0xffffu)) * tv[4 * i + 2] : 0.f;
      const float w3 = tp.nval[i] > 3 ? h2f((uint16_t)(lraw[i].y >> 16)) * tv[4 * i + 3] : 0.f;
      float *tab = L.tab2 + tp.dst[i];
#pragma unroll
      for (int hi = 0; hi < 4; ++hi) table_quad(tab, w0, w1, w2, w3, hi);
    }
  }
  // one barrier ends the exchange and starts the next phase: waves 4-7 wait
  // for their copies first, and the per-wave flags are next written a
  // phase later, after the products' barriers
  if (wave_id() >= 4) __builtin_amdgcn_s_waitcnt(0);
  const int wok = __all(ok);
  if ((t & 63) == 0) L.flags8[wave_id()] = wok;
  __syncthreads();
  int all = 1;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) all &= L.flags8[i];
  return all != 0;
}

// --------------------------------------------------------------- kernel

// One 8-wave workgroup per CU (its LDS takes the CU), so two waves per
// SIMD: telling the compiler so lets it keep many table reads in flight
// (otherwise it may serialise them to fit a higher occupancy that can never
// occur).
template <bool kDelay>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_persist(PArgs A) {
  extern __shared__ __align__(16) unsigned char smem[];
  Lds L;
  {
    unsigned char *p = smem;
    L.ctx = reinterpret_cast<PhaseCtx *>(p); p += kCtxBytes;
    L.segbuf = reinterpret_cast<PSeg *>(p); p += 2 * kMaxSeg * sizeof(PSeg);
    L.stg = p; p += kStgBytes;
    L.tab2 = reinterpret_cast<float *>(p); p += kTab2Floats * 4;
    L.tab1 = reinterpret_cast<float *>(p); p += kTab1Floats * 4;
    L.acc2 = reinterpret_cast<float *>(p); p += kMaxUnitLayers * 2 * 16 * kTMax * 4;
    L.xs = reinterpret_cast<float *>(p); p += 16 * kTMax * 4;
    L.red = reinterpret_cast<float *>(p); p += kXThreads * 4;
    L.flags8 = reinterpret_cast<int *>(p);
    L.xcnt = L.flags8 + kWaves;
  }
  const int w = blockIdx.x;
  const int U = A.nunits;
  // the generation base: the tag of this workgroup's first partial word
  // (every exchange writes column 0),
  // which the previous launch's last exchange wrote as its base + U (every
  // exchange writes it; zero after a reset), so launches, captured graph
  // replays included, continue one running count
  const unsigned gen_base = __builtin_amdgcn_readfirstlane((unsigned)(
      ld_tag(&A.PA[((size_t)(w % kXcd) * kPerXcd + w / kXcd) * kLuMax]) >> 32));
  L.tl = A.timeline ? A.timeline + (size_t)w * (U + 1) * kStamps : nullptr;
  // phase 0's copy list (kMaxSeg records of two 16-byte words), then its blocks
  if (threadIdx.x == 0) *L.xcnt = 0;
  for (int i = threadIdx.x; i < kMaxSeg * 2; i += kThreads)
    reinterpret_cast<uint4 *>(L.segbuf)[i] = reinterpret_cast<const uint4 *>(A.segs)[i];
  __syncthreads();
  if (wave_id() >= 4) {
    stage_phase(A, 0, L);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  for (int ph = 0; ph <= U; ++ph) {
    stamp(L, ph, 0);
    // every context field the phase uses is read before the barrier that
    // follows the first product, after which waves 4-7 restage the context
    const int t0 = L.ctx->t0, t1 = L.ctx->t1;
    const int Lu = L.ctx->ub.Lu;
    // this thread's share of the next phase's tables (built in the
    // exchange), planned now so the reads overlap the products
    const TabPlan tp = load_tables(A, L, ph < U);
    if (ph == 0) {
      const PUnit &U0 = L.ctx->ub;
      for (int r = threadIdx.x; r < 16 * (t1 - t0); r += kThreads) {
        const int i = 16 * t0 + r;
        const uint16_t v = i < U0.a ? A.x0[i] : (uint16_t)0;
        L.xs[r] = h2f(v);
        if (A.trace && i < U0.a) A.trace[U0.trace_x + i] = v;
      }
      __syncthreads();
    } else {
      second_product(A, ph, L);
      stamp(L, ph, 2);
      if (ph == U) break;
    }
    const unsigned gen = gen_base + (unsigned)ph + 1u;
    test_delay<kDelay>(A, gen, 0);
    // the partials, on the critical path, are stored by the lookup threads
    // as they finish, before the next phase's block copies (waves 4-7),
    // which then overlap the waits; the barrier keeps the copies off the
    // LDS the lookups still read
    first_product(A, L, ph, gen);
    stamp(L, ph, 4);
    __syncthreads();
    if (wave_id() >= 4) {
      // the copy issue gets the SIMDs first while waves 0-3 only poll
      __builtin_amdgcn_s_setprio(2);
      stage_phase(A, ph + 1, L);
      __builtin_amdgcn_s_setprio(0);
    }
    if (!exchange_collect<kDelay>(L, Lu, gen, A, tp, ph)) {
      // a wait gave up: let the next phase's copies into LDS land before
      // the workgroup (and its LDS) ends
      __builtin_amdgcn_s_waitcnt(0);
      return;
    }
    stamp(L, ph, 7);
  }
}

// ------------------------------------------------------------------ host
static size_t lds_bytes() {
  return kCtxBytes + 2 * kMaxSeg * sizeof(PSeg) + (size_t)kStgBytes +
         (size_t)(kTab2Floats + kTab1Floats + kMaxUnitLayers * 2 * 16 * kTMax +
                  16 * kTMax + kXThreads + kWaves + 1) * 4 + 64;
}

int64_t persist_max_rows() { return 1; }

constexpr size_t kPaBytes = sizeof(uint64_t) * kXcd * kPerXcd * kLuMax;
constexpr size_t kPbBytes = sizeof(uint64_t) * 2 * kXcd * kLuMax;
constexpr size_t kPcBytes = sizeof(uint64_t) * kXcd * kLuMax;

__global__ void k_xcd_id(unsigned *out) {
  if (threadIdx.x == 0) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    out[blockIdx.x] = x & 15u;
  }
}

// 1 when a grid of one workgroup per CU places workgroup w on XCD w % 8 (the
// dispatcher's round robin over the XCDs), so levels A and C can stay in
// each XCD's L2; 0 otherwise (device-scope stores throughout: correct on
// any placement, slower); -1 on a HIP error.  Checked once per device.
static int xcd_placement(int device) {
  static std::mutex mu;
  static std::map<int, int> known;
  std::lock_guard<std::mutex> lk(mu);
  auto it = known.find(device);
  if (it != known.end()) return it->second;
  const int G = kXcd * kPerXcd;
  unsigned *d = nullptr;
  std::vector<unsigned> h(G, 0xffffffffu);
  int res = -1;
  if (hipMalloc(&d, G * sizeof(unsigned)) == hipSuccess) {
    hipLaunchKernelGGL(k_xcd_id, dim3(G), dim3(64), 0, 0, d);
    if (hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
        hipMemcpy(h.data(), d, G * sizeof(unsigned), hipMemcpyDeviceToHost) == hipSuccess) {
      res = 1;
      for (int w = 0; w < G; ++w)
        if (h[w] != (unsigned)(w % kXcd)) res = 0;
    }
    (void)hipFree(d);
  }
  if (res >= 0) known[device] = res;
  return res;
}

// Column-group width for the first product's lookups of a unit with Lu
// columns on nt row tiles: among 1, 2, 4 (up to maxc, which divides every
// layer's column count), the one whose busiest SIMD issues the fewest
// instructions.  Lanes are ngr lpt (lpt by the kernel's rule); passes of
// kThreads lanes; wave w runs on SIMD w % 4; a lane's pass costs about 40
// instructions plus 16 per column and word slot (two slots per step).
static int s1_width(int maxc, int Lu, int nt) {
  int best = 1;
  long best_cost = -1;
  for (int c = 1; c <= maxc; c *= 2) {
    const int ngr = Lu / c;
    int lpt = 1;
    while (lpt < 64 && lpt < nt && ngr * lpt * 2 <= kThreads) lpt *= 2;
    const int wpl = (nt + lpt - 1) / lpt, slots = (wpl + 1) / 2 * 2;
    const long per = 40 + 16L * c * slots;
    const int N = ngr * lpt;
    int worst = 0;
    for (int s = 0; s < 4; ++s) {
      int passes = 0;
      for (int w = s; w < kWaves; w += 4)
        if (N > w * 64) passes += (N - w * 64 + kThreads - 1) / kThreads;
      worst = std::max(worst, passes);
    }
    const long cost = worst * per;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

lb_status persist_build(const std::vector<lb_layer *> &layers, const std::vector<int> &unit_begin,
                        const std::vector<int> &unit_size, float kappa, int device,
                        PersistPlan **out) {
  *out = nullptr;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return LB_EHIP;
  const int G = prop.multiProcessorCount;
  if (G != kXcd * kPerXcd) return LB_EUNSUPPORTED;
  PersistPlan *P = new PersistPlan();
  P->device = device;
  P->G = G;
  P->nunits = (int)unit_begin.size();
  P->nlayers = (int)layers.size();
  int64_t tx = 0;
  for (auto *Lr : layers) tx += Lr->ly.b;
  auto unsupported = [&]() { delete P; return LB_EUNSUPPORTED; };
  for (int u = 0; u < P->nunits; ++u) {
    PUnit U{};
    U.first = unit_begin[u];
    U.n = unit_size[u];
    if (U.n > kMaxUnitLayers) return unsupported();
    const Layer &L0 = layers[U.first]->ly;
    U.a = (int)L0.a;
    U.b = (int)L0.b;
    U.c_out = kappa / std::sqrt((float)U.n);
    U.trace_x = tx;
    tx += U.a;
    int col = 0;
    int64_t yoff = 0;
    for (int i = 0; i < U.first; ++i) yoff += layers[i]->ly.b;
    for (int m = 0; m < U.n; ++m) {
      const Layer &Ly = layers[U.first + m]->ly;
      PLayer D{};
      D.su2t = Ly.su2t; D.sv16 = Ly.sv16; D.ht = Ly.ht; D.gt = Ly.gt; D.l = Ly.l;
      D.a = (int)Ly.a; D.b = (int)Ly.b; D.s = (int)Ly.s; D.P = Ly.P; D.L = (int)Ly.L;
      D.Lp = (int)Ly.Lp; D.Wk = (int)Ly.Wk; D.a16 = (int)Ly.a16; D.b16 = (int)Ly.b16;
      D.s8 = (int)Ly.s8;
      D.col0 = col;
      D.trace_y = yoff;
      yoff += Ly.b;
      col += (int)Ly.L;
      P->h_layers.push_back(D);
    }
    U.Lu = col;
    if (U.Lu > kLuMax) return unsupported();
    // column groups must divide every layer's column count P s (the
    // layers' first columns are then multiples of them too)
    int maxc = 4;
    for (int m = 0; m < U.n; ++m)
      while ((int)layers[U.first + m]->ly.L % maxc != 0) maxc /= 2;
    const int tiles = (U.a + 15) / 16, nt0 = tiles / G;
    U.cpt = s1_width(maxc, U.Lu, nt0) | (s1_width(maxc, U.Lu, nt0 + 1) << 8) | (nt0 << 16);
    for (int m = 1; m < U.n; ++m)  // the products assume one path count per unit
      if (layers[U.first + m]->ly.P != L0.P) return unsupported();
    P->h_units.push_back(U);
  }
  // table groups of every unit, in the order the tables are laid out
  // (layer-major, path, 4-column group)
  std::vector<PGroup> groups;
  std::vector<size_t> gfirst;
  for (int u = 0; u < P->nunits; ++u) {
    PUnit &U = P->h_units[u];
    gfirst.push_back(groups.size());
    int toff = 0;
    for (int m = 0; m < U.n; ++m) {
      PLayer &D = P->h_layers[U.first + m];
      D.tb2 = toff;
      for (int p = 0; p < D.P; ++p) {
        for (int rem = 0; rem < D.Wk * 8; ++rem) {
          const int nval = std::max(0, std::min(4, D.s - 4 * rem));
          PGroup g{};
          // a group past s reads nothing; its l pointer is the (valid) base
          g.lp = nval > 0 ? D.l + (size_t)p * D.s8 + 4 * rem : D.l;
          g.tcol = D.col0 + p * D.s + 4 * rem;
          g.nd = nval | ((toff + (rem >> 3) * kWordF + (rem & 7) * 16) << 4);
          groups.push_back(g);
        }
        toff += s2_set_floats(D.Wk);
      }
    }
    U.ngrp = (int)(groups.size() - gfirst.back());
    if (toff > kTab2Floats) return unsupported();
  }
  for (int u = 1; u < P->nunits; ++u)
    if (P->h_units[u].a != P->h_units[u - 1].b ||
        P->h_units[u].first != P->h_units[u - 1].first + P->h_units[u - 1].n) {
      delete P;
      return LB_EINVAL;
    }
  // per-phase capacity: tiles, staged bytes, tables
  for (int ph = 0; ph <= P->nunits; ++ph) {
    const int width = ph == 0 ? P->h_units[0].a : P->h_units[ph - 1].b;
    const int nt = ((width + 15) / 16 + G - 1) / G;
    if (nt > kTMax) return unsupported();
    long stg = 0, tab2 = 0, tab1 = 0;
    if (ph > 0) {
      const PUnit &U = P->h_units[ph - 1];
      for (int m = 0; m < U.n; ++m) {
        const PLayer &D = P->h_layers[U.first + m];
        stg += (long)D.P * ((long)D.Wk * 64 * nt + 32 * nt + 2 * D.s8);
        tab2 += (long)D.P * s2_set_floats(D.Wk);
      }
    }
    if (ph < P->nunits) {
      const PUnit &U = P->h_units[ph];
      for (int m = 0; m < U.n; ++m) {
        const PLayer &D = P->h_layers[U.first + m];
        stg += (long)nt * D.Lp * 2 + (long)D.P * 32 * nt;
        tab1 += (long)D.P * s1_set_floats(nt);
      }
    }
    if (stg > kStgBytes || tab2 > kTab2Floats || tab1 > kTab1Floats) return unsupported();
  }
  P->lds = lds_bytes();
  if (P->lds > (size_t)prop.sharedMemPerBlock) return unsupported();
  bool ok = hipMalloc(&P->d_groups, sizeof(PGroup) * std::max<size_t>(1, groups.size())) == hipSuccess &&
            hipMemcpy(P->d_groups, groups.data(), sizeof(PGroup) * groups.size(),
                      hipMemcpyHostToDevice) == hipSuccess;
  for (int u = 0; u < P->nunits && ok; ++u) P->h_units[u].grp = P->d_groups + gfirst[u];
  ok = ok && hipMalloc(&P->d_units, sizeof(PUnit) * P->nunits) == hipSuccess &&
            hipMalloc(&P->d_layers, sizeof(PLayer) * P->nlayers) == hipSuccess &&
            hipMalloc(&P->PA, kPaBytes) == hipSuccess && hipMalloc(&P->PB, kPbBytes) == hipSuccess &&
            hipMalloc(&P->PC, kPcBytes) == hipSuccess &&
            hipMalloc(&P->err, sizeof(unsigned) * 64) == hipSuccess &&
            hipHostMalloc(&P->herr, sizeof(unsigned) * 16,
                          hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
            hipHostGetDevicePointer((void **)&P->herr_dev, P->herr, 0) == hipSuccess;
  if (ok) *(volatile unsigned *)P->herr = 0u;
  ok = ok && hipMemcpy(P->d_units, P->h_units.data(), sizeof(PUnit) * P->nunits,
                       hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(P->d_layers, P->h_layers.data(), sizeof(PLayer) * P->nlayers,
                       hipMemcpyHostToDevice) == hipSuccess;
  // per-phase copy lists (device addresses of the descriptors are known now)
  std::vector<PSeg> segs((size_t)(P->nunits + 1) * kMaxSeg);
  for (int ph = 0; ph <= P->nunits && ok; ++ph) {
    PSeg *lst = &segs[(size_t)ph * kMaxSeg];
    int n = 1;
    int off_fixed = 0, off_tile = 0;  // running LDS offset = off_fixed + nt * off_tile
    auto add = [&](const void *src, long long stride, int per_tile, int fixed, int kind, int m) {
      int offp = 0;
      if (kind >= kSegS2) {
        offp = off_fixed | (off_tile << 16);
        off_fixed += fixed;
        off_tile += per_tile;
      }
      lst[n++] = PSeg{src, stride, per_tile, fixed, kind | (m << 8), offp};
    };
    const int ua = ph > 0 ? ph - 1 : 0;
    const int nun = (ph > 0) + (ph < P->nunits);
    add(P->d_units + ua, 0, 0, (int)sizeof(PUnit) * nun, kSegUnits, 0);
    int nly = 0;
    if (ph > 0) nly += P->h_units[ph - 1].n;
    if (ph < P->nunits) nly += P->h_units[ph].n;
    add(P->d_layers + P->h_units[ua].first, 0, 0, (int)sizeof(PLayer) * nly, kSegLayers, 0);
    if (ph > 0) {
      const PUnit &U = P->h_units[ph - 1];
      for (int m = 0; m < U.n; ++m) {
        const PLayer &D = P->h_layers[U.first + m];
        add(D.su2t, (long long)D.P * D.Wk * 64, D.P * D.Wk * 64, 0, kSegS2, m);
        add(D.ht, 32LL * D.P, 32 * D.P, 0, kSegH, m);
        add(D.l, 0, 0, 2 * D.P * D.s8, kSegL, m);
      }
    }
    if (ph < P->nunits) {
      const PUnit &U = P->h_units[ph];
      for (int m = 0; m < U.n; ++m) {
        const PLayer &D = P->h_layers[U.first + m];
        add(D.sv16, 2LL * D.Lp, 2 * D.Lp, 0, kSegS1, m);
        add(D.gt, 32LL * D.P, 32 * D.P, 0, kSegG, m);
      }
    }
    const int width = ph == 0 ? P->h_units[0].a : P->h_units[ph - 1].b;
    lst[0] = PSeg{nullptr, 0, width, n, kSegHeader, 0};
    for (int k = 1; k < n; ++k)
      if ((lst[k].per_tile | lst[k].fixed) % 16 != 0) ok = false;  // DMA moves 16-byte units
    if (off_fixed > 0xffff || off_tile > 0xffff) ok = false;  // offsets packed in 16 bits
  }
  ok = ok && hipMalloc(&P->d_segs, sizeof(PSeg) * segs.size()) == hipSuccess;
  ok = ok && hipMemcpy(P->d_segs, segs.data(), sizeof(PSeg) * segs.size(), hipMemcpyHostToDevice) ==
                 hipSuccess;
  ok = ok && hipMemset(P->err, 0, sizeof(unsigned) * 64) == hipSuccess;
  ok = ok && hipMemset(P->PA, 0, kPaBytes) == hipSuccess && hipMemset(P->PB, 0, kPbBytes) == hipSuccess &&
       hipMemset(P->PC, 0, kPcBytes) == hipSuccess;
  if (ok) {
    const int xl = xcd_placement(device);
    if (xl < 0) ok = false;
    P->xcd_local = xl > 0;
  }
  ok = ok && hipFuncSetAttribute((const void *)k_persist<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)P->lds) == hipSuccess;
  ok = ok && hipFuncSetAttribute((const void *)k_persist<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)P->lds) == hipSuccess;
  int occ = 0;
  int occ_d = 0;
  ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_persist<false>, kThreads, P->lds) ==
                 hipSuccess;
  ok = ok && hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_d, k_persist<true>, kThreads, P->lds) ==
                 hipSuccess;
  occ = std::min(occ, occ_d);
  if (!ok || occ < 1) {
    persist_free(P);
    return ok ? LB_EUNSUPPORTED : LB_EHIP;
  }
  *out = P;
  return LB_OK;
}

void persist_free(PersistPlan *p) {
  if (!p) return;
  if (p->d_units) (void)hipFree(p->d_units);
  if (p->d_layers) (void)hipFree(p->d_layers);
  if (p->d_segs) (void)hipFree(p->d_segs);
  if (p->d_groups) (void)hipFree(p->d_groups);
  if (p->PA) (void)hipFree(p->PA);
  if (p->PB) (void)hipFree(p->PB);
  if (p->PC) (void)hipFree(p->PC);
  if (p->err) (void)hipFree(p->err);
  if (p->herr) (void)hipHostFree(p->herr);
  delete p;
}

lb_status persist_run(PersistPlan *p, const uint16_t *x0, uint16_t *y, uint16_t *trace, int64_t M,
                      hipStream_t st, std::string *msg) {
  if (M != 1) return LB_EUNSUPPORTED;
  if (!p->broken && *(volatile unsigned *)p->herr != 0u) {
    // a finished earlier launch gave up a wait: its output was undefined.
    // Report it once; the next call resets and runs.
    p->broken = true;
    if (msg) *msg = "persistent sweep: an earlier launch gave up a device-side wait (its output is "
                    "undefined); this call did not run, the next one resets the sweep";
    return LB_ETIMEOUT;
  }
  if (p->broken) {
    // a previous launch gave up a wait: clear the error word and every tag
    // (synchronous: the launch that failed has finished before the reset)
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemset(p->err, 0, sizeof(unsigned) * 64) != hipSuccess ||
        hipMemset(p->PA, 0, kPaBytes) != hipSuccess || hipMemset(p->PB, 0, kPbBytes) != hipSuccess ||
        hipMemset(p->PC, 0, kPcBytes) != hipSuccess)
      return LB_EHIP;
    *(volatile unsigned *)p->herr = 0u;
    p->broken = false;
  }
  PArgs A{};
  A.units = p->d_units;
  A.layers = p->d_layers;
  A.nunits = p->nunits;
  A.x0 = x0;
  A.y = y;
  A.trace = trace;
  A.PA = p->PA;
  A.PB = p->PB;
  A.PC = p->PC;
  A.xcd_local = p->xcd_local;
  A.err = p->err;
  A.herr = p->herr_dev;
  A.timeline = p->timeline;
  A.segs = p->d_segs;
  A.grp0 = p->d_groups;
  A.wait_skew = p->fail_test ? 0x40000000u : 0u;
  A.delay_seed = p->delay_seed;
  A.delay_max = p->delay_max;
  if (p->delay_max)
    hipLaunchKernelGGL(k_persist<true>, dim3(p->G), dim3(kThreads), p->lds, st, A);
  else
    hipLaunchKernelGGL(k_persist<false>, dim3(p->G), dim3(kThreads), p->lds, st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    if (msg) *msg = std::string("persistent launch: ") + hipGetErrorString(e);
    return LB_EHIP;
  }
  return LB_OK;
}

void persist_set_timeline(PersistPlan *p, uint64_t *buf) { p->timeline = buf; }
void persist_set_fail_test(PersistPlan *p, bool on) { p->fail_test = on; }
void persist_set_delay(PersistPlan *p, unsigned seed, unsigned max_ticks) {
  p->delay_seed = seed;
  p->delay_max = max_ticks;
}
int persist_grid(const PersistPlan *p) { return p->G; }
int persist_phases(const PersistPlan *p) { return p->nunits + 1; }
int persist_stamps() { return kStamps; }

lb_status persist_check(PersistPlan *p, std::string *msg) {
  unsigned e = 0;
  if (hipMemcpy(&e, p->err, sizeof(unsigned),
                hipMemcpyDeviceToHost) !=
      hipSuccess)
    return LB_EHIP;
  if (e) {
    p->broken = true;
    if (msg) *msg = "persistent sweep: a device-side wait timed out (err=" + std::to_string(e) + ")";
    return LB_ETIMEOUT;
  }
  return LB_OK;
}

}  // namespace lbi
