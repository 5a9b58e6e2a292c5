// Host core: irreps strings, paths, real Clebsch-Gordan tensors.
//
// CG values: Racah's closed formula for the complex (Condon-Shortley)
// coefficients, rearranged so that the alternating sum is a sum of products
// of binomial coefficients (exact in 64-bit integers for l <= 6) and the
// square-root factor is a ratio of two exact integers:
//   <j1 m1 j2 m2|J M> = S * sqrt(R),  a = j1+j2-J, b = j1-j2+J, c = -j1+j2+J,
//   S = sum_k (-1)^k binom(a,k) binom(b, j1-m1-k) binom(c, j2+m2-k),
//   R = (2J+1) binom(2j1,a) binom(2j2,a) /
//       ((a+b+c+1) binom(a+b+c,a) binom(2j1,j1-m1) binom(2j2,j2-m2) binom(2J,J-M)).
// The real tensor is the complex one conjugated into the real spherical-harmonic
// basis (Y_real = U Y_complex), made real by one global phase, with the sign of
// the first nonzero entry (in m1, m2, m3 order) positive.  The e3nn_mlx README
// promises real CG coefficients, and the e3j Convolution page names a
// "SQRT_DIM_OUT" normalization, without formulas; the orthonormal reading above
// is the one this library uses.
#include "host_core.h"

#include <cctype>
#include <cmath>
#include <complex>
#include <cstdint>

namespace e3c {

// ------------------------------------------------------------------ irreps --

namespace {

void strip_spaces(const std::string& in, std::string* out) {
  out->clear();
  for (char ch : in)
    if (!std::isspace(static_cast<unsigned char>(ch))) out->push_back(ch);
}

bool split_top(const std::string& s, std::vector<std::string>* parts) {
  int depth = 0;
  std::string cur;
  for (char ch : s) {
    if (ch == '(') ++depth;
    if (ch == ')') {
      if (--depth < 0) return false;
    }
    if (ch == '+' && depth == 0) {
      parts->push_back(cur);
      cur.clear();
    } else {
      cur.push_back(ch);
    }
  }
  if (depth != 0) return false;
  parts->push_back(cur);
  return true;
}

bool parse_uint(const std::string& s, size_t* pos, long* val) {
  size_t p = *pos;
  long v = 0;
  while (p < s.size() && std::isdigit(static_cast<unsigned char>(s[p]))) {
    v = v * 10 + (s[p] - '0');
    if (v > 1000000) return false;
    ++p;
  }
  if (p == *pos) return false;
  *pos = p;
  *val = v;
  return true;
}

bool parse_into(const std::string& s, int mul_scale, std::vector<Irrep>* out, std::string* err) {
  std::vector<std::string> parts;
  if (!split_top(s, &parts)) {
    *err = "unbalanced parentheses";
    return false;
  }
  for (const std::string& part : parts) {
    if (part.empty()) {
      *err = "empty block";
      return false;
    }
    size_t pos = 0;
    long mul = 1;
    long num = 0;
    if (!parse_uint(part, &pos, &num)) {
      *err = "block '" + part + "' does not start with a number";
      return false;
    }
    if (pos < part.size() && part[pos] == 'x') {
      mul = num;
      ++pos;
      if (pos < part.size() && part[pos] == '(') {
        if (part.back() != ')') {
          *err = "block '" + part + "' has an unclosed group";
          return false;
        }
        if (!parse_into(part.substr(pos + 1, part.size() - pos - 2), mul_scale * (int)mul, out, err))
          return false;
        continue;
      }
      if (!parse_uint(part, &pos, &num)) {
        *err = "block '" + part + "' has no l after 'x'";
        return false;
      }
    }
    if (pos + 1 != part.size() || (part[pos] != 'e' && part[pos] != 'o')) {
      *err = "block '" + part + "' must end in e or o";
      return false;
    }
    out->push_back(Irrep{(int)mul * mul_scale, (int)num, part[pos] == 'e' ? 1 : -1});
  }
  return true;
}

}  // namespace

bool parse_irreps(const std::string& text, std::vector<Irrep>* out, std::string* err) {
  out->clear();
  std::string s;
  strip_spaces(text, &s);
  if (s.empty()) {
    *err = "empty irreps string";
    return false;
  }
  return parse_into(s, 1, out, err);
}

std::vector<HostPath> enumerate_paths(const std::vector<Irrep>& xin, int lmax,
                                      const std::vector<Irrep>& out) {
  std::vector<int> ox(xin.size()), oo(out.size());
  int acc = 0;
  for (size_t i = 0; i < xin.size(); ++i) { ox[i] = acc; acc += 2 * xin[i].l + 1; }
  acc = 0;
  for (size_t i = 0; i < out.size(); ++i) { oo[i] = acc; acc += 2 * out[i].l + 1; }
  std::vector<HostPath> paths;
  for (size_t i1 = 0; i1 < xin.size(); ++i1) {
    for (int l2 = 0; l2 <= lmax; ++l2) {
      const int py = (l2 % 2) ? -1 : 1;
      for (size_t i3 = 0; i3 < out.size(); ++i3) {
        const int l1 = xin[i1].l, l3 = out[i3].l;
        if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) continue;
        if (out[i3].parity != xin[i1].parity * py) continue;
        paths.push_back(HostPath{(int)i1, l1, xin[i1].parity, ox[i1], l2, l2 * l2, (int)i3, l3,
                                 out[i3].parity, oo[i3]});
      }
    }
  }
  return paths;
}

// -------------------------------------------------------------- CG values --

namespace {

int64_t binom(int n, int k) {
  if (k < 0 || k > n) return 0;
  if (k > n - k) k = n - k;
  int64_t r = 1;
  for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;  // exact at every step
  return r;
}

long double complex_cg(int j1, int m1, int j2, int m2, int J, int M) {
  if (M != m1 + m2) return 0.0L;
  if (J < std::abs(j1 - j2) || J > j1 + j2) return 0.0L;
  if (std::abs(m1) > j1 || std::abs(m2) > j2 || std::abs(M) > J) return 0.0L;
  const int a = j1 + j2 - J, b = j1 - j2 + J, c = -j1 + j2 + J;
  int64_t S = 0;
  for (int k = 0; k <= a; ++k) {
    const int i1 = j1 - m1 - k, i2 = j2 + m2 - k;
    if (i1 < 0 || i1 > b || i2 < 0 || i2 > c) continue;
    const int64_t term = binom(a, k) * binom(b, i1) * binom(c, i2);
    S += (k % 2) ? -term : term;
  }
  const int64_t num = (2 * J + 1) * binom(2 * j1, a) * binom(2 * j2, a);
  const int64_t den = (int64_t)(a + b + c + 1) * binom(a + b + c, a) * binom(2 * j1, j1 - m1) *
                      binom(2 * j2, j2 - m2) * binom(2 * J, J - M);
  return (long double)S * std::sqrt((long double)num / (long double)den);
}

using cld = std::complex<long double>;

// Y_real[m] = sum_mu U[m][mu] Y_complex[mu]; returns the (at most two) nonzero
// entries of row m as (mu, value) pairs.
int basis_row(int m, int* mu, cld* val) {
  const long double r = 1.0L / std::sqrt(2.0L);
  if (m == 0) {
    mu[0] = 0;
    val[0] = cld(1.0L, 0.0L);
    return 1;
  }
  const long double sgn = (std::abs(m) % 2) ? -1.0L : 1.0L;
  if (m > 0) {
    mu[0] = m;  val[0] = cld(sgn * r, 0.0L);
    mu[1] = -m; val[1] = cld(r, 0.0L);
  } else {
    mu[0] = m;  val[0] = cld(0.0L, r);
    mu[1] = -m; val[1] = cld(0.0L, -sgn * r);
  }
  return 2;
}

}  // namespace

bool real_cg(int l1, int l2, int l3, std::vector<double>* out) {
  if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > 6 || l2 > 6 || l3 > 6) return false;
  if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return false;
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  std::vector<cld> T((size_t)n1 * n2 * n3);
  // out_r = U3 CG(U1^H x_r, U2^H y_r):  T[i][j][k] = sum U3[k][c] CG[a][b][c] conj(U1[i][a]) conj(U2[j][b])
  for (int i = 0; i < n1; ++i) {
    int mu1[2]; cld v1[2];
    const int c1 = basis_row(i - l1, mu1, v1);
    for (int j = 0; j < n2; ++j) {
      int mu2[2]; cld v2[2];
      const int c2 = basis_row(j - l2, mu2, v2);
      for (int k = 0; k < n3; ++k) {
        int mu3[2]; cld v3[2];
        const int c3 = basis_row(k - l3, mu3, v3);
        cld sum(0.0L, 0.0L);
        for (int x = 0; x < c1; ++x)
          for (int y = 0; y < c2; ++y)
            for (int z = 0; z < c3; ++z) {
              const long double cg = complex_cg(l1, mu1[x], l2, mu2[y], l3, mu3[z]);
              if (cg == 0.0L) continue;
              sum += v3[z] * cg * std::conj(v1[x]) * std::conj(v2[y]);
            }
        T[((size_t)i * n2 + j) * n3 + k] = sum;
      }
    }
  }
  size_t imax = 0;
  long double amax = 0.0L;
  for (size_t q = 0; q < T.size(); ++q) {
    if (std::abs(T[q]) > amax) { amax = std::abs(T[q]); imax = q; }
  }
  if (amax == 0.0L) return false;
  const cld phase = T[imax] / amax;
  out->assign(T.size(), 0.0);
  for (size_t q = 0; q < T.size(); ++q) {
    const cld v = T[q] / phase;
    if (std::abs(v.imag()) > 1e-12L * amax) return false;   // not real: formula error
    (*out)[q] = std::abs(v.real()) < 1e-14L * amax ? 0.0 : (double)v.real();
  }
  for (size_t q = 0; q < out->size(); ++q) {
    if ((*out)[q] != 0.0) {
      if ((*out)[q] < 0.0)
        for (double& v : *out) v = -v;
      break;
    }
  }
  return true;
}

// ---------------------------------------------------------- scheduling --

void receiver_order(const int* row_ptr, const int* src, int num_nodes, int cluster, int* order) {
  std::vector<char> seen((size_t)num_nodes, 0);
  std::vector<int> queue;
  queue.reserve((size_t)cluster * 64);
  int out = 0;
  for (int seed = 0; seed < num_nodes; ++seed) {
    if (seen[seed]) continue;
    queue.clear();
    queue.push_back(seed);
    seen[seed] = 1;
    int taken = 0;
    size_t head = 0;
    while (head < queue.size() && taken < cluster) {
      const int v = queue[head++];
      order[out++] = v;
      ++taken;
      for (int e = row_ptr[v]; e < row_ptr[v + 1]; ++e) {
        const int a = src[e];
        if (!seen[a]) {
          seen[a] = 1;
          queue.push_back(a);
        }
      }
    }
    // nodes queued but not taken go back to the pool
    for (size_t i = head; i < queue.size(); ++i) seen[queue[i]] = 0;
  }
}

}  // namespace e3c
