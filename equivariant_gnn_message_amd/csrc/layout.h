// Compile-time description of one irrep layout of the convolution
//   m_b = (1/N) sum_{a->b} (x_a (x) y_ab) (.) s_ab
// (e3j Convolution page, class formula and plain implementation).
//
// A layout is (C, x blocks, SH lmax L, output blocks).  Blocks are encoded in a
// 32-bit "block code": 2 bits per l = 0..15, 0 = absent, 1 = even, 2 = odd;
// blocks are stored in ascending l.  Paths are every (x block, l2 = 0..L,
// output block) triple, in that nesting order, with |l1-l2| <= l3 <= l1+l2 and
// p3 = p1 (-1)^l2 (the edge features are spherical harmonics of parity (-1)^l2).
// The path index is the scalar axis of s (the "third source space" that the
// page infers from the two inputs).
//
// The nonzero pattern of each real Clebsch-Gordan tensor C[m1,m2,m3] (real
// basis, m = -l..l) follows the selection rule
//   |m3| in { |m1|+|m2|, ||m1|-|m2|| }  and  #(m < 0) = l1+l2+l3 (mod 2),
// which is exact up to entries that vanish by accident (the host builder fills
// the values and checks that nothing outside the pattern is nonzero).
//
// Everything here is constexpr so that kernels can be fully unrolled with the
// pattern known at compile time, while the coefficient VALUES are produced at
// run time by the host builder in exactly this enumeration order.
#pragma once

#include <cstdint>

namespace e3c {

constexpr int kMaxL = 15;
constexpr int kMaxPaths = 48;
constexpr int kMaxNnz = 1024;
constexpr int kMaxComps = 64;

constexpr int iabs(int v) { return v < 0 ? -v : v; }

constexpr int block_parity(uint32_t code, int l) {
  const uint32_t b = (code >> (2 * l)) & 3u;
  return b == 1u ? 1 : (b == 2u ? -1 : 0);
}

// number of components per channel of a block list
constexpr int code_dim(uint32_t code) {
  int d = 0;
  for (int l = 0; l <= kMaxL; ++l)
    if (block_parity(code, l) != 0) d += 2 * l + 1;
  return d;
}

constexpr int code_offset(uint32_t code, int lq) {
  int d = 0;
  for (int l = 0; l < lq; ++l)
    if (block_parity(code, l) != 0) d += 2 * l + 1;
  return d;
}

// selection rule for a real-basis CG entry (see header comment)
constexpr bool cg_allowed(int l1, int l2, int l3, int m1, int m2, int m3) {
  if (iabs(l1 - l2) > l3 || l3 > l1 + l2) return false;
  const int a = iabs(m1), b = iabs(m2), c = iabs(m3);
  if (!(c == a + b || c == iabs(a - b))) return false;
  const int neg = (m1 < 0) + (m2 < 0) + (m3 < 0);
  return (neg & 1) == ((l1 + l2 + l3) & 1);
}

struct PathInfo {
  int l1, o1, l2, o2, l3, o3;
  int nnz_begin, nnz_end;   // range in the entry list
};

struct Entry {
  int8_t m1, m2, m3;        // 0-based indices inside the blocks (m + l)
};

struct LayoutTables {
  int num_x, num_y, num_out, num_paths, nnz;
  PathInfo path[kMaxPaths];
  Entry entry[kMaxNnz];
};

constexpr LayoutTables make_tables(uint32_t xcode, int lmax, uint32_t ocode) {
  LayoutTables t{};
  t.num_x = code_dim(xcode);
  t.num_y = (lmax + 1) * (lmax + 1);
  t.num_out = code_dim(ocode);
  int np = 0, nnz = 0;
  for (int l1 = 0; l1 <= kMaxL; ++l1) {
    const int p1 = block_parity(xcode, l1);
    if (p1 == 0) continue;
    for (int l2 = 0; l2 <= lmax; ++l2) {
      for (int l3 = 0; l3 <= kMaxL; ++l3) {
        const int p3 = block_parity(ocode, l3);
        if (p3 == 0) continue;
        if (iabs(l1 - l2) > l3 || l3 > l1 + l2) continue;
        if (p3 != p1 * ((l2 & 1) ? -1 : 1)) continue;
        PathInfo& P = t.path[np++];
        P.l1 = l1; P.o1 = code_offset(xcode, l1);
        P.l2 = l2; P.o2 = l2 * l2;
        P.l3 = l3; P.o3 = code_offset(ocode, l3);
        P.nnz_begin = nnz;
        for (int i = 0; i < 2 * l1 + 1; ++i)
          for (int j = 0; j < 2 * l2 + 1; ++j)
            for (int k = 0; k < 2 * l3 + 1; ++k)
              if (cg_allowed(l1, l2, l3, i - l1, j - l2, k - l3)) {
                t.entry[nnz].m1 = (int8_t)i;
                t.entry[nnz].m2 = (int8_t)j;
                t.entry[nnz].m3 = (int8_t)k;
                ++nnz;
              }
        P.nnz_end = nnz;
      }
    }
  }
  t.num_paths = np;
  t.nnz = nnz;
  return t;
}

// True if K^p[m3][m1] = sum_m2 C[m1,m2,m3] y[m2] has a structurally nonzero term.
constexpr bool k_nonzero(const LayoutTables& t, int p, int m3, int m1) {
  for (int e = t.path[p].nnz_begin; e < t.path[p].nnz_end; ++e)
    if (t.entry[e].m3 == m3 && t.entry[e].m1 == m1) return true;
  return false;
}

// Compile-time layout: channels and block codes.
template <int C_, uint32_t XCODE_, int L_, uint32_t OCODE_>
struct Layout {
  static constexpr int C = C_;
  static constexpr uint32_t XCODE = XCODE_;
  static constexpr int L = L_;
  static constexpr uint32_t OCODE = OCODE_;
  static constexpr LayoutTables T = make_tables(XCODE_, L_, OCODE_);
  static constexpr int NX = T.num_x;
  static constexpr int NY = T.num_y;
  static constexpr int NO = T.num_out;
  static constexpr int NP = T.num_paths;
  static constexpr int NNZ = T.nnz;
};

// natural-parity block code for l = 0..lmax (0e + 1o + 2e + ...)
constexpr uint32_t natural_code(int lmax) {
  uint32_t c = 0;
  for (int l = 0; l <= lmax; ++l) c |= ((l & 1) ? 2u : 1u) << (2 * l);
  return c;
}

}  // namespace e3c
