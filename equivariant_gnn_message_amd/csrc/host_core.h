// Host-side core of the plan: irreps parsing, path enumeration and real
// Clebsch-Gordan tensors.  Pure C++17, no device calls.
#pragma once

#include <string>
#include <vector>

namespace e3c {

struct Irrep {
  int mul;
  int l;
  int parity;  // +1 even, -1 odd
};

// Parses "8x0e+8x1o", "0e + 2x1o", "64x(0e+1o+2e)".  Returns false and sets
// *err on a malformed string.
bool parse_irreps(const std::string& text, std::vector<Irrep>* out, std::string* err);

struct HostPath {
  int i1, l1, p1, o1;   // x block
  int l2, o2;           // edge harmonic
  int i3, l3, p3, o3;   // output block
};

// Paths in s-axis order: x block (as listed), l2 = 0..lmax, output block (as
// listed); kept iff |l1-l2| <= l3 <= l1+l2 and p3 = p1 (-1)^l2.
std::vector<HostPath> enumerate_paths(const std::vector<Irrep>& xin, int lmax,
                                      const std::vector<Irrep>& out);

// Real CG tensor of (l1, l2, l3) flattened as [m1][m2][m3] (m = -l..l -> 0..2l),
// real basis with z polar and l=1 ordered (y, z, x), orthonormal over (m1, m2),
// first nonzero entry positive.  Requires l1, l2, l3 <= 6 and the triangle
// rule; returns false otherwise.
bool real_cg(int l1, int l2, int l3, std::vector<double>* out);

// Receiver processing order for gather locality: greedy breadth-first clusters
// of about `cluster` receivers over the in-neighbour graph (CSR row_ptr/src),
// seeds taken in index order.  Writes a permutation of 0..N-1 into order.
void receiver_order(const int* row_ptr, const int* src, int num_nodes, int cluster, int* order);

}  // namespace e3c
