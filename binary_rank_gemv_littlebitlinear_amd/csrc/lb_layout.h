// Host re-layout of a layer's sign bits: pure functions on host arrays, no
// HIP and no device memory, so they build with any C++17 compiler (the
// library links them; a sanitizer build checks them on the CPU).
//
// The canonical layout is the C ABI's (include/lb.h): a factor with `rows`
// rows is rows x Wk uint32 words, row-major, entry k of a row at bit k % 32
// of word k / 32, bit 1 = +1 ([LB news] Sec. 2: S_U in {+-1}^(b x s),
// S_V in {+-1}^(a x s)).  Bits past s are ignored on input.
//
// Device layouts (P paths, latent column c = p * s + k, L = P * s):
//
//   sv16[gi * Lp + c]   (uint16, T16v x Lp)  bit (i % 16) = S_V,p[i, k] for
//       i = 16 gi + bit.  The first product's bits by 16-row tiles of the
//       input; T16v = 2 R1 = the tiles rounded up to an even count, so that
//       rows 2 r and 2 r + 1 together give the 32-row word of row group r.
//       Lp = L rounded up to 8.
//   su2t[((tau * P + p) * Wk + q) * 16 + r]   (uint32, T16b x P x Wk x 16)
//       = word q of S_U,p row 16 tau + r: the second product's bits by
//       16-row tiles of the output, each tile one contiguous block.
//   sv1m[r * L + c], su2m[(p * Wk + q) * b16 + j]   (uint32)  the
//       matrix-core copies: the same words as sv16 (two halves joined) and
//       su2t, column- and row-major, with every word's bits inverted
//       (1 = sign -1) and permuted so that the sign of element 8 g + e
//       (g = 0..3, e = 0..7) sits at bit 15 - e/2 - 4 g for even e and
//       31 - (e - 1)/2 - 4 g for odd e.
//   tile16[(tau * P + p) * 16 + r] = v_p[16 tau + r]   (fp16 bits) the
//       per-path scales h and g by 16-row tiles.
//
// Padding bits and padding scales are zero.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace lbl {

struct Dims {
  int64_t a = 0, b = 0, s = 0;
  int P = 1;
  int64_t Wk = 0, L = 0, Lp = 0, R1 = 0, T16a = 0, T16v = 0, T16b = 0, a16 = 0, b16 = 0;
};

// The derived sizes of a layer with input width a, output width b, rank s
// and P paths (1 or 2).
Dims dims(int64_t a, int64_t b, int64_t s, int P);

inline size_t sv16_elems(const Dims &d) { return (size_t)d.T16v * d.Lp; }
inline size_t su2t_elems(const Dims &d) { return (size_t)d.T16b * d.P * d.Wk * 16; }
inline size_t sv1m_elems(const Dims &d) { return (size_t)d.R1 * d.L; }
inline size_t su2m_elems(const Dims &d) { return (size_t)d.P * d.Wk * d.b16; }
inline size_t tile16_elems(int64_t n16, int P) { return (size_t)n16 * P; }

// In-place transpose of a 32 x 32 bit matrix: bit c of m[r] <-> bit r of m[c].
void transpose32(uint32_t m[32]);

// One word in the matrix-core bit order.
uint32_t mfma_bit_order(uint32_t w);

// Path `path` of the canonical S_V (a x Wk words) into / out of sv16; the
// other path's columns are left as they are.
void put_sv16(const Dims &d, int path, const uint32_t *sv, uint16_t *sv16);
void get_sv16(const Dims &d, int path, const uint16_t *sv16, uint32_t *sv);

// Path `path` of the canonical S_U (b x Wk words) into / out of su2t.
void put_su2t(const Dims &d, int path, const uint32_t *su, uint32_t *su2t);
void get_su2t(const Dims &d, int path, const uint32_t *su2t, uint32_t *su);

// The matrix-core copies of every path, from the tile layouts.
void sv1m_from_sv16(const Dims &d, const uint16_t *sv16, uint32_t *sv1m);
void su2m_from_su2t(const Dims &d, const uint32_t *su2t, uint32_t *su2m);

// Path `path` of an n-long per-row scale into the tile layout of n16
// (n rounded up to 16) rows.
void put_tile16(int64_t n, int64_t n16, int P, int path, const uint16_t *v, uint16_t *t);

}  // namespace lbl
