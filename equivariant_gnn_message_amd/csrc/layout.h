// Compile-time description of one irrep layout of the convolution
//   m_b = (1/N) sum_{a->b} (x_a (x) y_ab) (.) s_ab
// (e3j Convolution page: class formula, and the unfused implementation
// described beneath it).
//
// A layout is (C, x blocks, SH lmax L, output blocks).  Blocks are encoded in a
// 32-bit "block code": 2 bits per l = 0..15, 0 = absent, 1 = even, 2 = odd;
// blocks are stored in ascending l.  Paths are every (x block, l2 = 0..L,
// output block) triple, in that nesting order, with |l1-l2| <= l3 <= l1+l2 and
// p3 = p1 (-1)^l2 (the edge features are spherical harmonics of parity (-1)^l2).
// The path index is the scalar axis of s (the page derives the space of the
// mixing scalars from the spaces of the two inputs).
//
// The nonzero pattern of each real Clebsch-Gordan tensor C[m1,m2,m3] (real
// basis, m = -l..l) follows the selection rule
//   |m3| in { |m1|+|m2|, ||m1|-|m2|| }  and  #(m < 0) = l1+l2+l3 (mod 2),
// which is exact up to entries that vanish by accident (the host builder fills
// the values and checks that nothing outside the pattern is nonzero).
//
// Everything here is constexpr so that kernels can be fully unrolled with the
// pattern and the coefficient values known at compile time; the host plan
// builder produces the same values at run time, in this enumeration order, and
// checks the two tables against each other.
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

// ------------------------------------------------ compile-time CG values --
//
// The kernels take the real CG values as compile-time constants (instruction
// literals), evaluated here from the same definitions the host plan builder
// uses: Racah's formula in binomial form (exact 64-bit integer sums), the
// complex -> real spherical-harmonic basis change (Y_real = U Y_complex,
// Condon-Shortley phases), one global phase, and the sign rule (first nonzero
// entry in (m1, m2, m3) order positive).  The plan checks these tables against
// its runtime tables before binding a layout to its kernels.

constexpr double cx_sqrt(double v) {
  if (!(v > 0.0)) return 0.0;
  double r = v > 1.0 ? v : 1.0;
  for (int i = 0; i < 200; ++i) {
    const double n = 0.5 * (r + v / r);
    if (n == r) break;
    r = n;
  }
  return r;
}

constexpr int64_t cx_binom(int n, int k) {
  if (k < 0 || k > n) return 0;
  if (k > n - k) k = n - k;
  int64_t r = 1;
  for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
  return r;
}

constexpr double cx_complex_cg(int j1, int m1, int j2, int m2, int J, int M) {
  if (M != m1 + m2 || J < iabs(j1 - j2) || J > j1 + j2) return 0.0;
  if (iabs(m1) > j1 || iabs(m2) > j2 || iabs(M) > J) return 0.0;
  const int a = j1 + j2 - J, b = j1 - j2 + J, c = -j1 + j2 + J;
  int64_t S = 0;
  for (int k = 0; k <= a; ++k) {
    const int i1 = j1 - m1 - k, i2 = j2 + m2 - k;
    if (i1 < 0 || i1 > b || i2 < 0 || i2 > c) continue;
    const int64_t term = cx_binom(a, k) * cx_binom(b, i1) * cx_binom(c, i2);
    S += (k & 1) ? -term : term;
  }
  const int64_t num = (2 * J + 1) * cx_binom(2 * j1, a) * cx_binom(2 * j2, a);
  const int64_t den = (int64_t)(a + b + c + 1) * cx_binom(a + b + c, a) * cx_binom(2 * j1, j1 - m1) *
                      cx_binom(2 * j2, j2 - m2) * cx_binom(2 * J, J - M);
  return (double)S * cx_sqrt((double)num / (double)den);
}

struct Cplx {
  double re, im;
};
constexpr Cplx cmul(Cplx a, Cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
constexpr Cplx cconj(Cplx a) { return {a.re, -a.im}; }

// Row m of U (Y_real = U Y_complex): up to two (mu, value) entries.
struct BasisRow {
  int n;
  int mu[2];
  Cplx v[2];
};

constexpr BasisRow basis_row(int m) {
  const double r = 0.70710678118654752440;
  BasisRow row{};
  if (m == 0) {
    row.n = 1;
    row.mu[0] = 0;
    row.v[0] = {1.0, 0.0};
    return row;
  }
  const double sgn = (iabs(m) & 1) ? -1.0 : 1.0;
  row.n = 2;
  if (m > 0) {
    row.mu[0] = m;  row.v[0] = {sgn * r, 0.0};
    row.mu[1] = -m; row.v[1] = {r, 0.0};
  } else {
    row.mu[0] = m;  row.v[0] = {0.0, r};
    row.mu[1] = -m; row.v[1] = {0.0, -sgn * r};
  }
  return row;
}

constexpr Cplx real_cg_complex_entry(int l1, int l2, int l3, int i, int j, int k) {
  const BasisRow r1 = basis_row(i - l1), r2 = basis_row(j - l2), r3 = basis_row(k - l3);
  Cplx s{0.0, 0.0};
  for (int x = 0; x < r1.n; ++x)
    for (int y = 0; y < r2.n; ++y)
      for (int z = 0; z < r3.n; ++z) {
        const double cg = cx_complex_cg(l1, r1.mu[x], l2, r2.mu[y], l3, r3.mu[z]);
        if (cg == 0.0) continue;
        const Cplx t = cmul(cmul(r3.v[z], cconj(r1.v[x])), cconj(r2.v[y]));
        s.re += cg * t.re;
        s.im += cg * t.im;
      }
  return s;
}

template <int NNZ>
struct CGValues {
  float v[NNZ > 0 ? NNZ : 1];
};

// Real CG values of every pattern entry, path by path.  The pattern lists
// (m1, m2, m3) in lexicographic order and contains every nonzero entry, so
// the global phase (from the largest entry) and the sign (first nonzero entry
// positive) can be taken over the pattern alone.
template <int NNZ>
constexpr CGValues<NNZ> make_cg_values(const LayoutTables& t) {
  CGValues<NNZ> out{};
  Cplx z[kMaxNnz]{};
  for (int p = 0; p < t.num_paths; ++p) {
    const PathInfo& P = t.path[p];
    Cplx big{0.0, 0.0};
    double amax = 0.0;
    for (int q = P.nnz_begin; q < P.nnz_end; ++q) {
      z[q] = real_cg_complex_entry(P.l1, P.l2, P.l3, t.entry[q].m1, t.entry[q].m2, t.entry[q].m3);
      const double m2 = z[q].re * z[q].re + z[q].im * z[q].im;
      if (m2 > amax) { amax = m2; big = z[q]; }
    }
    const double mag = cx_sqrt(amax);
    const Cplx unphase{big.re / mag, -big.im / mag};
    double sign = 0.0;
    for (int q = P.nnz_begin; q < P.nnz_end && sign == 0.0; ++q) {
      const double v = cmul(z[q], unphase).re;
      if (v > 1e-14 * mag) sign = 1.0;
      if (v < -1e-14 * mag) sign = -1.0;
    }
    for (int q = P.nnz_begin; q < P.nnz_end; ++q) {
      const double v = cmul(z[q], unphase).re;
      out.v[q] = (v > -1e-14 * mag && v < 1e-14 * mag) ? 0.0f : (float)(sign * v);
    }
  }
  return out;
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
  static constexpr CGValues<NNZ> CG = make_cg_values<NNZ>(T);
};

// SENDER graph ordering (e3j Convolution page, note on graph_ordering): with
// the edges grouped by sender, node b's message is assembled from its
// outgoing edges e = (b -> a) as (x_a (x) p.y_e) (.) s_e, i.e. from the
// reverse edges' features under the page's symmetry assumptions
// y_ab = (-1)^l y_ba (per l block) and s_ab = s_ba.  The parity (-1)^l2 of the
// edge-feature block is folded into the path's CG constants; everything else
// is the RECEIVER kernel with the roles of the two endpoints exchanged.
template <int NNZ>
constexpr CGValues<NNZ> parity_flipped(const LayoutTables& t, const CGValues<NNZ>& cg) {
  CGValues<NNZ> r = cg;
  for (int p = 0; p < t.num_paths; ++p)
    if (t.path[p].l2 & 1)
      for (int q = t.path[p].nnz_begin; q < t.path[p].nnz_end; ++q) r.v[q] = -r.v[q];
  return r;
}

template <class LY>
struct SenderOrdered : LY {
  static constexpr CGValues<LY::NNZ> CG = parity_flipped<LY::NNZ>(LY::T, LY::CG);
};

// natural-parity block code for l = 0..lmax (0e + 1o + 2e + ...)
constexpr uint32_t natural_code(int lmax) {
  uint32_t c = 0;
  for (int l = 0; l <= lmax; ++l) c |= ((l & 1) ? 2u : 1u) << (2 * l);
  return c;
}

}  // namespace e3c
