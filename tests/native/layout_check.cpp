// Driver of the host sign re-layout (csrc/lb_layout.cpp) for the CPU tests:
// built together with it under AddressSanitizer and UndefinedBehaviorSanitizer.
//
//   layout_check IN OUT
//
// IN:  int64 a, b, s, P, order (0: paths packed 0 then 1; 1: the reverse);
//      then for each path p: su (b x Wk uint32), sv (a x Wk uint32),
//      h (b uint16), g (a uint16).
// OUT: sv16, su2t, sv1m, su2m, ht, gt (the device layouts, in that order),
//      then for each path p the canonical words read back: su, sv.
// The layout buffers start zeroed, as the device storage does.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../binary_rank_gemv_littlebitlinear_amd/csrc/lb_layout.h"

template <class T>
static void read_n(FILE *f, std::vector<T> &v, size_t n) {
  v.resize(n);
  if (n && fread(v.data(), sizeof(T), n, f) != n) {
    fprintf(stderr, "short read\n");
    exit(2);
  }
}

template <class T>
static void write_v(FILE *f, const std::vector<T> &v) {
  if (!v.empty() && fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) {
    fprintf(stderr, "short write\n");
    exit(2);
  }
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: layout_check IN OUT\n");
    return 2;
  }
  FILE *in = fopen(argv[1], "rb");
  if (!in) return 2;
  std::vector<int64_t> hdr;
  read_n(in, hdr, 5);
  const int64_t a = hdr[0], b = hdr[1], s = hdr[2];
  const int P = (int)hdr[3], order = (int)hdr[4];
  if (a < 1 || b < 1 || s < 1 || (P != 1 && P != 2)) return 2;
  const lbl::Dims d = lbl::dims(a, b, s, P);
  std::vector<uint32_t> su[2], sv[2];
  std::vector<uint16_t> h[2], g[2];
  for (int p = 0; p < P; ++p) {
    read_n(in, su[p], (size_t)b * d.Wk);
    read_n(in, sv[p], (size_t)a * d.Wk);
    read_n(in, h[p], (size_t)b);
    read_n(in, g[p], (size_t)a);
  }
  fclose(in);

  std::vector<uint16_t> sv16(lbl::sv16_elems(d), 0), ht(lbl::tile16_elems(d.b16, P), 0),
      gt(lbl::tile16_elems(d.a16, P), 0);
  std::vector<uint32_t> su2t(lbl::su2t_elems(d), 0u), sv1m(lbl::sv1m_elems(d), 0u),
      su2m(lbl::su2m_elems(d), 0u);
  for (int k = 0; k < P; ++k) {
    const int p = order ? P - 1 - k : k;
    lbl::put_sv16(d, p, sv[p].data(), sv16.data());
    lbl::put_su2t(d, p, su[p].data(), su2t.data());
    lbl::put_tile16(b, d.b16, P, p, h[p].data(), ht.data());
    lbl::put_tile16(a, d.a16, P, p, g[p].data(), gt.data());
  }
  lbl::sv1m_from_sv16(d, sv16.data(), sv1m.data());
  lbl::su2m_from_su2t(d, su2t.data(), su2m.data());

  FILE *out = fopen(argv[2], "wb");
  if (!out) return 2;
  write_v(out, sv16);
  write_v(out, su2t);
  write_v(out, sv1m);
  write_v(out, su2m);
  write_v(out, ht);
  write_v(out, gt);
  for (int p = 0; p < P; ++p) {
    std::vector<uint32_t> bu((size_t)b * d.Wk, 0xdeadbeefu), bv((size_t)a * d.Wk, 0xdeadbeefu);
    lbl::get_su2t(d, p, su2t.data(), bu.data());
    lbl::get_sv16(d, p, sv16.data(), bv.data());
    write_v(out, bu);
    write_v(out, bv);
  }
  fclose(out);
  return 0;
}
