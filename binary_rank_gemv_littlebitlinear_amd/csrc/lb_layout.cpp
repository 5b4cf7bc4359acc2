// Host re-layout of the sign bits (layouts defined in lb_layout.h).
#include "lb_layout.h"

namespace lbl {

namespace {

// Valid bits of word q of a row of rank s.
inline uint32_t tail_mask(int64_t s, int64_t q) {
  const int64_t n = s - 32 * q;
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// Columns of word q that exist (s - 32 q, at most 32).
inline int64_t word_cols(int64_t s, int64_t q) { return (s - 32 * q) < 32 ? (s - 32 * q) : 32; }

uint32_t mfma_bit_order_slow(uint32_t w) {
  uint32_t o = 0;
  for (int g = 0; g < 4; ++g)
    for (int e = 0; e < 8; ++e) {
      const uint32_t flip = ((w >> (8 * g + e)) & 1u) ^ 1u;
      const int pos = (e & 1) ? 31 - (e >> 1) - 4 * g : 15 - (e >> 1) - 4 * g;
      o |= flip << pos;
    }
  return o;
}

// The permutation is bytewise: byte g of w fills its own bit positions, so
// a table per byte position gives the word in four lookups.
struct MfmaOrderTable {
  uint32_t t[4][256];
  MfmaOrderTable() {
    for (int g = 0; g < 4; ++g)
      for (uint32_t v = 0; v < 256; ++v)
        // the other bytes set to all ones contribute no flips
        t[g][v] = mfma_bit_order_slow((0xffffffffu & ~(0xffu << (8 * g))) | (v << (8 * g)));
  }
};
const MfmaOrderTable g_order;

// The 32-row word of row group r, latent column c, joined from sv16.
inline uint32_t sv16_word(const Dims &d, const uint16_t *sv16, int64_t r, int64_t c) {
  return (uint32_t)sv16[(size_t)(2 * r) * d.Lp + c] |
         ((uint32_t)sv16[(size_t)(2 * r + 1) * d.Lp + c] << 16);
}

}  // namespace

Dims dims(int64_t a, int64_t b, int64_t s, int P) {
  Dims d;
  d.a = a; d.b = b; d.s = s; d.P = P;
  d.Wk = (s + 31) / 32;
  d.L = P * s;
  d.Lp = (d.L + 7) / 8 * 8;
  d.R1 = (a + 31) / 32;
  d.T16a = (a + 15) / 16;
  d.T16v = 2 * d.R1;
  d.T16b = (b + 15) / 16;
  d.a16 = d.T16a * 16;
  d.b16 = d.T16b * 16;
  return d;
}

void transpose32(uint32_t m[32]) {
  // swap the off-diagonal j x j blocks for j = 16, 8, 4, 2, 1
  uint32_t mask = 0x0000ffffu;
  for (int j = 16; j != 0; j >>= 1, mask ^= (mask << j)) {
    for (int k = 0; k < 32; k = ((k | j) + 1) & ~j) {
      const uint32_t t = ((m[k] >> j) ^ m[k | j]) & mask;
      m[k] ^= t << j;
      m[k | j] ^= t;
    }
  }
}

uint32_t mfma_bit_order(uint32_t w) {
  return g_order.t[0][w & 0xff] | g_order.t[1][(w >> 8) & 0xff] | g_order.t[2][(w >> 16) & 0xff] |
         g_order.t[3][w >> 24];
}

void put_sv16(const Dims &d, int path, const uint32_t *sv, uint16_t *sv16) {
  uint32_t blk[32];
  for (int64_t r = 0; r < d.R1; ++r)
    for (int64_t q = 0; q < d.Wk; ++q) {
      const uint32_t msk = tail_mask(d.s, q);
      for (int e = 0; e < 32; ++e) {
        const int64_t i = 32 * r + e;
        blk[e] = i < d.a ? (sv[(size_t)i * d.Wk + q] & msk) : 0u;
      }
      transpose32(blk);  // blk[kk] bit e = S_V[32 r + e, 32 q + kk]
      const int64_t nk = word_cols(d.s, q);
      for (int64_t kk = 0; kk < nk; ++kk) {
        const int64_t c = path * d.s + 32 * q + kk;
        sv16[(size_t)(2 * r) * d.Lp + c] = (uint16_t)(blk[kk] & 0xffffu);
        sv16[(size_t)(2 * r + 1) * d.Lp + c] = (uint16_t)(blk[kk] >> 16);
      }
    }
}

void get_sv16(const Dims &d, int path, const uint16_t *sv16, uint32_t *sv) {
  uint32_t blk[32];
  for (int64_t r = 0; r < d.R1; ++r)
    for (int64_t q = 0; q < d.Wk; ++q) {
      const int64_t nk = word_cols(d.s, q);
      for (int64_t kk = 0; kk < 32; ++kk)
        blk[kk] = kk < nk ? sv16_word(d, sv16, r, path * d.s + 32 * q + kk) : 0u;
      transpose32(blk);  // blk[e] bit kk = S_V[32 r + e, 32 q + kk]
      for (int e = 0; e < 32; ++e) {
        const int64_t i = 32 * r + e;
        if (i < d.a) sv[(size_t)i * d.Wk + q] = blk[e];
      }
    }
}

void put_su2t(const Dims &d, int path, const uint32_t *su, uint32_t *su2t) {
  for (int64_t j = 0; j < d.b16; ++j)
    for (int64_t q = 0; q < d.Wk; ++q) {
      const uint32_t wd = j < d.b ? (su[(size_t)j * d.Wk + q] & tail_mask(d.s, q)) : 0u;
      su2t[((size_t)((j >> 4) * d.P + path) * d.Wk + q) * 16 + (j & 15)] = wd;
    }
}

void get_su2t(const Dims &d, int path, const uint32_t *su2t, uint32_t *su) {
  for (int64_t j = 0; j < d.b; ++j)
    for (int64_t q = 0; q < d.Wk; ++q)
      su[(size_t)j * d.Wk + q] = su2t[((size_t)((j >> 4) * d.P + path) * d.Wk + q) * 16 + (j & 15)];
}

void sv1m_from_sv16(const Dims &d, const uint16_t *sv16, uint32_t *sv1m) {
  for (int64_t r = 0; r < d.R1; ++r)
    for (int64_t c = 0; c < d.L; ++c) sv1m[(size_t)r * d.L + c] = mfma_bit_order(sv16_word(d, sv16, r, c));
}

void su2m_from_su2t(const Dims &d, const uint32_t *su2t, uint32_t *su2m) {
  for (int p = 0; p < d.P; ++p)
    for (int64_t q = 0; q < d.Wk; ++q)
      for (int64_t j = 0; j < d.b16; ++j)
        su2m[((size_t)p * d.Wk + q) * d.b16 + j] =
            mfma_bit_order(su2t[((size_t)((j >> 4) * d.P + p) * d.Wk + q) * 16 + (j & 15)]);
}

void put_tile16(int64_t n, int64_t n16, int P, int path, const uint16_t *v, uint16_t *t) {
  for (int64_t j = 0; j < n16; ++j)
    t[((size_t)(j >> 4) * P + path) * 16 + (j & 15)] = j < n ? v[j] : (uint16_t)0;
}

}  // namespace lbl
