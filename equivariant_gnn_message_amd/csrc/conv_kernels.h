// Fused HIP kernels for the equivariant message-passing convolution, gfx950
// (device templates and launchers; each layout file instantiates them).
//
//   out[b] = (1/N) sum_{e=(a->b)} (x[a] (x) y[e]) (.) s[e]
// (e3j Convolution page: class formula.  The unfused implementation the page
// describes runs over all edges four times -- sender rows, product with the
// harmonics, weighting by the scalars, accumulation at the receivers; here
// the four happen in one pass per receiver.)
//
// Design (wave64):
// * Receiver-sorted CSR: a wave owns one or more receivers, so the scatter-add
//   becomes a register-resident segmented sum with a single coalesced store
//   per output row and no atomics (the e3j page's RECEIVER ordering: every
//   receiver's messages are summed where they arrive).
// * Trailing channels: lanes map to channels.  A "group" of LPG = C/CPL lanes
//   covers all C channels of one edge, CPL channels per lane; a wave holds
//   64/LPG groups, GPR of which split the edges of one receiver and are summed
//   by cross-lane shuffles at the end of the segment.
// * Per edge: y (channel-less, shared by the group) builds the per-path
//   matrices K^p[m3][m1] = sum_m2 C^p[m1,m2,m3] y[o2+m2] in registers from the
//   compile-time nonzero pattern (the CG values are compile-time constants,
//   emitted as instruction literals); then per channel either
//   acc[o3+m3] += sum_m1 K^p[m3][m1] (s[p] x[a][o1+m1])   (2l1+1 <= 2l3+1) or
//   acc[o3+m3] += s[p] * sum_m1 K^p[m3][m1] x[a][o1+m1]   (otherwise),
//   whichever needs fewer products.
// * The pipelined kernels keep the next edge's rows in flight while the
//   current edge is contracted (two register buffers).
// * s and y are streamed with non-temporal loads so the gathered x rows stay
//   cache resident; out is written with non-temporal stores.
// * Work-group b runs logical block (b mod 8) * (grid / 8) + b / 8, so each of
//   the 8 XCDs (each with its own L2) runs a contiguous range of the receiver
//   processing order.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"

namespace e3c {
namespace {

template <int B, int E, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    sfor<B + 1, E>(static_cast<F&&>(f));
  }
}

// ------------------------------------------------- compile-time pattern -----

constexpr bool first_term(const LayoutTables& t, int p, int q) {
  for (int e = t.path[p].nnz_begin; e < q; ++e)
    if (t.entry[e].m3 == t.entry[q].m3 && t.entry[e].m1 == t.entry[q].m1) return false;
  return true;
}

constexpr int first_m1(const LayoutTables& t, int p, int m3) {
  for (int m1 = 0; m1 < 2 * t.path[p].l1 + 1; ++m1)
    if (k_nonzero(t, p, m3, m1)) return m1;
  return -1;
}

constexpr int first_m3(const LayoutTables& t, int p, int m1) {
  for (int m3 = 0; m3 < 2 * t.path[p].l3 + 1; ++m3)
    if (k_nonzero(t, p, m3, m1)) return m3;
  return -1;
}

constexpr int pow2_ceil(int v) {
  int r = 1;
  while (r < v) r <<= 1;
  return r;
}

constexpr int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}


// Wave index in processing order.  Work-groups are dealt round-robin to the
// 8 XCDs (8 L2 caches); remapping so that XCD k runs a contiguous range of
// logical blocks keeps receivers that are processed together (neighbours in
// the receiver order) on one L2, where their shared senders' rows are reused.
// The grid is a multiple of 8 work-groups of 4 waves.
__device__ __forceinline__ int logical_wave() {
  const int per_xcd = (int)(gridDim.x >> 3);
  const int bid = (int)blockIdx.x;
  const int lb = (bid & 7) * per_xcd + (bid >> 3);
  return __builtin_amdgcn_readfirstlane(lb * 4 + (int)(threadIdx.x >> 6));
}

// --------------------------------------------------------------- loads ------

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short bf16_bits;

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

template <class T, bool NT>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

// CPL consecutive channel values starting at p.
template <typename IN, int CPL, bool NT>
__device__ __forceinline__ void load_ch(const IN* p, float (&v)[CPL]) {
  if constexpr (std::is_same<IN, float>::value) {
    if constexpr (CPL == 4) {
      const f32x4 t = ld<f32x4, NT>(reinterpret_cast<const f32x4*>(p));
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (CPL == 2) {
      const f32x2 t = ld<f32x2, NT>(reinterpret_cast<const f32x2*>(p));
      v[0] = t.x; v[1] = t.y;
    } else {
      static_assert(CPL == 1, "fp32 lanes hold 1, 2 or 4 channels");
      v[0] = ld<float, NT>(p);
    }
  } else {
    if constexpr (CPL == 8) {
      const u32x4 t = ld<u32x4, NT>(reinterpret_cast<const u32x4*>(p));
      v[0] = bf_lo(t.x); v[1] = bf_hi(t.x); v[2] = bf_lo(t.y); v[3] = bf_hi(t.y);
      v[4] = bf_lo(t.z); v[5] = bf_hi(t.z); v[6] = bf_lo(t.w); v[7] = bf_hi(t.w);
    } else if constexpr (CPL == 4) {
      const u32x2 t = ld<u32x2, NT>(reinterpret_cast<const u32x2*>(p));
      v[0] = bf_lo(t.x); v[1] = bf_hi(t.x); v[2] = bf_lo(t.y); v[3] = bf_hi(t.y);
    } else if constexpr (CPL == 2) {
      const unsigned t = ld<unsigned, NT>(reinterpret_cast<const unsigned*>(p));
      v[0] = bf_lo(t); v[1] = bf_hi(t);
    } else {
      static_assert(CPL == 1, "bf16 lanes hold 1, 2, 4 or 8 channels");
      v[0] = __uint_as_float(static_cast<unsigned>(ld<bf16_bits, NT>(p)) << 16);
    }
  }
}

// A row of N values (edge features), widest loads the row alignment allows.
template <typename IN, int N>
__device__ __forceinline__ void load_row(const IN* p, float (&v)[N]) {
  constexpr int bytes = N * (int)sizeof(IN);
  if constexpr (std::is_same<IN, float>::value) {
    if constexpr (bytes % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + i);
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = __builtin_nontemporal_load(p + i);
    }
  } else {
    if constexpr (bytes % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
        v[8 * i] = bf_lo(t.x); v[8 * i + 1] = bf_hi(t.x); v[8 * i + 2] = bf_lo(t.y);
        v[8 * i + 3] = bf_hi(t.y); v[8 * i + 4] = bf_lo(t.z); v[8 * i + 5] = bf_hi(t.z);
        v[8 * i + 6] = bf_lo(t.w); v[8 * i + 7] = bf_hi(t.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i)
        v[i] = __uint_as_float(static_cast<unsigned>(__builtin_nontemporal_load(p + i)) << 16);
    }
  }
}

// ----------------------------------------------------- shared edge math -----

// K^p[m3][m1] = sum_m2 C^p[m1,m2,m3] y[o2+m2] over the compile-time pattern.
template <class LY, int p, int D3, int D1>
__device__ __forceinline__ void build_k(const float (&yv)[LY::NY], float (&K)[D3][D1]) {
  constexpr PathInfo P = LY::T.path[p];
  sfor<P.nnz_begin, P.nnz_end>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    constexpr Entry en = LY::T.entry[q];
    constexpr float c = LY::CG.v[q];
    const float yy = yv[P.o2 + en.m2];
    if constexpr (first_term(LY::T, p, q)) {
      K[en.m3][en.m1] = c * yy;
    } else {
      K[en.m3][en.m1] = __builtin_fmaf(c, yy, K[en.m3][en.m1]);
    }
  });
}

// ------------------------------------------------------------ forward -------

template <class LY, typename IN, int CPL, int GPR>
__global__ void __launch_bounds__(256) conv_fwd(FwdParams prm) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NO = LY::NO, NP = LY::NP;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;

  const IN* __restrict__ x = static_cast<const IN*>(prm.x);
  const IN* __restrict__ y = static_cast<const IN*>(prm.y);
  const IN* __restrict__ s = static_cast<const IN*>(prm.s);
  const int* __restrict__ src = prm.src;
  const int* __restrict__ row_ptr = prm.row_ptr;

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const int gi = grp % GPR;
  const int slot = grp / GPR;
  const int bl = logical_wave() * RPW + slot;
  const bool valid = bl < prm.num_nodes;
  const int b = valid ? (prm.order ? prm.order[bl] : bl) : 0;

  float acc[NO][CPL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[o][c] = 0.0f;

  int beg = 0, end = 0;
  if (valid) {
    beg = row_ptr[b];
    end = b < prm.num_real ? row_ptr[b + 1] : beg;   // padding receivers: no messages
  }
  const int c0 = li * CPL;

  for (int e = beg + gi; e < end; e += GPR) {
    const int a = src[e];
    float yv[NY];
    load_row<IN, NY>(y + (size_t)e * NY, yv);
    float xv[NX][CPL];
#pragma unroll
    for (int i = 0; i < NX; ++i) load_ch<IN, CPL, false>(x + ((size_t)a * NX + i) * C + c0, xv[i]);
    const IN* srow = s + (size_t)e * NP * C + c0;

    sfor<0, NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr PathInfo P = LY::T.path[p];
      constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
      float sv[CPL];
      load_ch<IN, CPL, true>(srow + p * C, sv);
      float K[D3][D1];
      build_k<LY, p, D3, D1>(yv, K);
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        static_assert(first_m1(LY::T, p, m3) >= 0, "every output row has a term");
        float t[CPL];
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              if constexpr (first_m1(LY::T, p, m3) == m1) {
                t[c] = K[m3][m1] * xv[P.o1 + m1][c];
              } else {
                t[c] = __builtin_fmaf(K[m3][m1], xv[P.o1 + m1][c], t[c]);
              }
            }
          }
        });
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          acc[P.o3 + m3][c] = __builtin_fmaf(sv[c], t[c], acc[P.o3 + m3][c]);
      });
    });
  }

  if constexpr (GPR > 1) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int d = LPG; d < LPG * GPR; d <<= 1) acc[o][c] += __shfl_xor(acc[o][c], d, 64);
  }

  if (valid) {
    float* orow = prm.out + (size_t)b * NO * C + c0;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      if (o % GPR != gi) continue;
      float* dst = orow + (size_t)o * C;
      if constexpr (CPL == 4) {
        f32x4 v = {acc[o][0] * prm.inv_avg, acc[o][1] * prm.inv_avg, acc[o][2] * prm.inv_avg,
                   acc[o][3] * prm.inv_avg};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
      } else if constexpr (CPL == 2) {
        f32x2 v = {acc[o][0] * prm.inv_avg, acc[o][1] * prm.inv_avg};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x2*>(dst));
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(acc[o][c] * prm.inv_avg, dst + c);
      }
    }
  }
}

// ------------------------------------------------- pipelined forward --------
//
// Same mapping as conv_fwd, with the edge loop software-pipelined: the loads
// of edge i+1 (y row, s rows, gathered x row) are in flight while edge i is
// computed, and the sender index is fetched two edges ahead so the gather's
// address is known when its loads are issued.  Two register buffers alternate
// (the loop body is unrolled twice), so no per-edge register copies.  Raw
// values (bf16 words) are kept until use.  Per path the contraction is
// reassociated as acc[o3+m3] += sum_m1 K[m3][m1] (s[p] x[o1+m1]), which needs
// (2 l1 + 1) products per path instead of (2 l3 + 1) mixing FMAs; paths with
// l1 > l3 keep the mixing form, which is then the cheaper one.

template <typename IN, int N>
struct RawVec;

template <int N>
struct RawVec<float, N> {
  float v[N];
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};

template <int N>
struct RawVec<bf16_bits, N> {
  unsigned w[(N + 1) / 2];
  __device__ __forceinline__ float get(int i) const {
    return (i & 1) ? bf_hi(w[i >> 1]) : bf_lo(w[i >> 1]);
  }
};

// N consecutive elements at p into raw registers (p aligned to the row size).
template <typename IN, int N, bool NT>
__device__ __forceinline__ void load_raw(const IN* p, RawVec<IN, N>& r) {
  if constexpr (std::is_same<IN, float>::value) {
    constexpr int bytes = N * 4;
    if constexpr (bytes % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const f32x4 t = ld<f32x4, NT>(reinterpret_cast<const f32x4*>(p) + i);
        r.v[4 * i] = t.x; r.v[4 * i + 1] = t.y; r.v[4 * i + 2] = t.z; r.v[4 * i + 3] = t.w;
      }
    } else if constexpr (bytes % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const f32x2 t = ld<f32x2, NT>(reinterpret_cast<const f32x2*>(p) + i);
        r.v[2 * i] = t.x; r.v[2 * i + 1] = t.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) r.v[i] = ld<float, NT>(p + i);
    }
  } else {
    constexpr int bytes = N * 2;
    if constexpr (bytes % 16 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        const u32x4 t = ld<u32x4, NT>(reinterpret_cast<const u32x4*>(p) + i);
        r.w[4 * i] = t.x; r.w[4 * i + 1] = t.y; r.w[4 * i + 2] = t.z; r.w[4 * i + 3] = t.w;
      }
    } else if constexpr (bytes % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const u32x2 t = ld<u32x2, NT>(reinterpret_cast<const u32x2*>(p) + i);
        r.w[2 * i] = t.x; r.w[2 * i + 1] = t.y;
      }
    } else if constexpr (bytes % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) r.w[i] = ld<unsigned, NT>(reinterpret_cast<const unsigned*>(p) + i);
    } else {
#pragma unroll
      for (int i = 0; i < (N + 1) / 2; ++i) r.w[i] = 0u;
#pragma unroll
      for (int i = 0; i < N; ++i)
        r.w[i >> 1] |= static_cast<unsigned>(ld<bf16_bits, NT>(p + i)) << (16 * (i & 1));
    }
  }
}

template <class LY, typename IN, int CPL>
struct EdgeBuf {
  RawVec<IN, LY::NY> y;
  RawVec<IN, CPL> x[LY::NX];
  RawVec<IN, CPL> s[LY::NP];
};

template <class LY, typename IN, int CPL>
__device__ __forceinline__ void load_edge(EdgeBuf<LY, IN, CPL>& buf, const IN* __restrict__ x,
                                          const IN* __restrict__ y, const IN* __restrict__ s, int e,
                                          int a, int c0) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP;
  load_raw<IN, NY, true>(y + (size_t)e * NY, buf.y);
  const IN* srow = s + (size_t)e * NP * C + c0;
#pragma unroll
  for (int p = 0; p < NP; ++p) load_raw<IN, CPL, true>(srow + p * C, buf.s[p]);
  const IN* xrow = x + (size_t)a * NX * C + c0;
#pragma unroll
  for (int i = 0; i < NX; ++i) load_raw<IN, CPL, false>(xrow + i * C, buf.x[i]);
}

template <class LY, typename IN, int CPL>
__device__ __forceinline__ void edge_accumulate(const EdgeBuf<LY, IN, CPL>& buf,
                                                float (&acc)[LY::NO][CPL]) {
  constexpr int NY = LY::NY, NP = LY::NP;
  float yv[NY];
#pragma unroll
  for (int j = 0; j < NY; ++j) yv[j] = buf.y.get(j);
  sfor<0, NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr PathInfo P = LY::T.path[p];
    constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
    float K[D3][D1];
    build_k<LY, p, D3, D1>(yv, K);
    if constexpr (D1 <= D3) {
      // acc += K (s x): 2 l1 + 1 products per channel
      float u[D1][CPL];
      sfor<0, D1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        if constexpr (first_m3(LY::T, p, m1) >= 0) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) u[m1][c] = buf.s[p].get(c) * buf.x[P.o1 + m1].get(c);
        }
      });
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              acc[P.o3 + m3][c] = __builtin_fmaf(K[m3][m1], u[m1][c], acc[P.o3 + m3][c]);
          }
        });
      });
    } else {
      // acc += s (K x): 2 l3 + 1 mixing products per channel
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        float tv[CPL];
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              if constexpr (first_m1(LY::T, p, m3) == m1) {
                tv[c] = K[m3][m1] * buf.x[P.o1 + m1].get(c);
              } else {
                tv[c] = __builtin_fmaf(K[m3][m1], buf.x[P.o1 + m1].get(c), tv[c]);
              }
            }
          }
        });
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          acc[P.o3 + m3][c] = __builtin_fmaf(buf.s[p].get(c), tv[c], acc[P.o3 + m3][c]);
      });
    }
  });
}

// UL: the sender index two edges ahead and the next edge's rows are loaded
// unconditionally, clamped to the receiver's last edge past its end (a
// conditional load, merged into the loop variable, makes the compiler wait
// for every load in flight, the next edge's rows included). Which form is
// faster depends on the layout.
template <class LY, typename IN, int CPL, int GPR, bool UL = false>
__global__ void __launch_bounds__(256) conv_fwd_pipe(FwdParams prm) {
  constexpr int C = LY::C, NO = LY::NO;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;

  const IN* __restrict__ x = static_cast<const IN*>(prm.x);
  const IN* __restrict__ y = static_cast<const IN*>(prm.y);
  const IN* __restrict__ s = static_cast<const IN*>(prm.s);
  const int* __restrict__ src = prm.src;
  const int* __restrict__ row_ptr = prm.row_ptr;

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const int gi = grp % GPR;
  const int slot = grp / GPR;
  const int bl = logical_wave() * RPW + slot;
  const bool valid = bl < prm.num_nodes;
  const int b = valid ? (prm.order ? prm.order[bl] : bl) : 0;
  const int c0 = li * CPL;

  float acc[NO][CPL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[o][c] = 0.0f;

  int beg = 0, end = 0;
  if (valid) {
    beg = row_ptr[b];
    end = b < prm.num_real ? row_ptr[b + 1] : beg;   // padding receivers: no messages
  }

  EdgeBuf<LY, IN, CPL> b0, b1;
  int e = beg + gi;
  if (e < end) load_edge<LY, IN, CPL>(b0, x, y, s, e, src[e], c0);
  int en = e + GPR;
  int an = en < end ? src[en] : 0;
  while (e < end) {
    int en2 = en + GPR;
    int an2;
    if constexpr (UL) {
      an2 = src[en2 < end ? en2 : end - 1];
      load_edge<LY, IN, CPL>(b1, x, y, s, en < end ? en : end - 1, an, c0);
    } else {
      if (en < end) load_edge<LY, IN, CPL>(b1, x, y, s, en, an, c0);
      an2 = en2 < end ? src[en2] : 0;
    }
    edge_accumulate<LY, IN, CPL>(b0, acc);
    e = en;
    en = en2;
    an = an2;
    if (e >= end) break;
    en2 = en + GPR;
    if constexpr (UL) {
      an2 = src[en2 < end ? en2 : end - 1];
      load_edge<LY, IN, CPL>(b0, x, y, s, en < end ? en : end - 1, an, c0);
    } else {
      if (en < end) load_edge<LY, IN, CPL>(b0, x, y, s, en, an, c0);
      an2 = en2 < end ? src[en2] : 0;
    }
    edge_accumulate<LY, IN, CPL>(b1, acc);
    e = en;
    en = en2;
    an = an2;
  }

  if constexpr (GPR > 1) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int d = LPG; d < LPG * GPR; d <<= 1) acc[o][c] += __shfl_xor(acc[o][c], d, 64);
  }

  if (valid) {
    float* orow = prm.out + (size_t)b * NO * C + c0;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      if (o % GPR != gi) continue;
      float* dst = orow + (size_t)o * C;
      if constexpr (CPL == 4) {
        f32x4 v = {acc[o][0] * prm.inv_avg, acc[o][1] * prm.inv_avg, acc[o][2] * prm.inv_avg,
                   acc[o][3] * prm.inv_avg};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
      } else if constexpr (CPL == 2) {
        f32x2 v = {acc[o][0] * prm.inv_avg, acc[o][1] * prm.inv_avg};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x2*>(dst));
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(acc[o][c] * prm.inv_avg, dst + c);
      }
    }
  }
}

// ------------------------------------------------------ forward-mode (JVP) --
//
// The convolution is trilinear in (x, y, s), so its derivative along a
// tangent (dx, dy, ds) is, per path and channel,
//   d out = K(y) dx (.) s  +  K(dy) x (.) s  +  K(y) x (.) ds     (divided by N).
// One pass reads both the primal and the tangent operands, builds K from y
// and from dy, and accumulates the primal output (stored when out != NULL)
// and the tangent output together.

template <int CPL>
__device__ __forceinline__ void store_row(float* dst, const float (&v)[CPL], float scale) {
  if constexpr (CPL == 4) {
    f32x4 w = {v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(dst));
  } else if constexpr (CPL == 2) {
    f32x2 w = {v[0] * scale, v[1] * scale};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x2*>(dst));
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(v[c] * scale, dst + c);
  }
}

template <class LY, typename IN, int CPL, int GPR>
__global__ void __launch_bounds__(256) conv_jvp(JvpParams prm) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NO = LY::NO, NP = LY::NP;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;

  const IN* __restrict__ x = static_cast<const IN*>(prm.x);
  const IN* __restrict__ y = static_cast<const IN*>(prm.y);
  const IN* __restrict__ s = static_cast<const IN*>(prm.s);
  const IN* __restrict__ dx = static_cast<const IN*>(prm.dx);
  const IN* __restrict__ dy = static_cast<const IN*>(prm.dy);
  const IN* __restrict__ ds = static_cast<const IN*>(prm.ds);
  const int* __restrict__ src = prm.src;
  const int* __restrict__ row_ptr = prm.row_ptr;

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const int gi = grp % GPR;
  const int slot = grp / GPR;
  const int bl = logical_wave() * RPW + slot;
  const bool valid = bl < prm.num_nodes;
  const int b = valid ? (prm.order ? prm.order[bl] : bl) : 0;

  float acc[NO][CPL], dacc[NO][CPL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      acc[o][c] = 0.0f;
      dacc[o][c] = 0.0f;
    }

  int beg = 0, end = 0;
  if (valid) {
    beg = row_ptr[b];
    end = b < prm.num_real ? row_ptr[b + 1] : beg;
  }
  const int c0 = li * CPL;

  for (int e = beg + gi; e < end; e += GPR) {
    const int a = src[e];
    float yv[NY], dyv[NY];
    load_row<IN, NY>(y + (size_t)e * NY, yv);
    load_row<IN, NY>(dy + (size_t)e * NY, dyv);
    float xv[NX][CPL], dxv[NX][CPL];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      load_ch<IN, CPL, false>(x + ((size_t)a * NX + i) * C + c0, xv[i]);
      load_ch<IN, CPL, false>(dx + ((size_t)a * NX + i) * C + c0, dxv[i]);
    }
    const IN* srow = s + (size_t)e * NP * C + c0;
    const IN* dsrow = ds + (size_t)e * NP * C + c0;

    sfor<0, NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr PathInfo P = LY::T.path[p];
      constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
      float sv[CPL], dsv[CPL];
      load_ch<IN, CPL, true>(srow + p * C, sv);
      load_ch<IN, CPL, true>(dsrow + p * C, dsv);
      float K[D3][D1], dK[D3][D1];
      build_k<LY, p, D3, D1>(yv, K);
      build_k<LY, p, D3, D1>(dyv, dK);
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        float t[CPL], dt[CPL];
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              if constexpr (first_m1(LY::T, p, m3) == m1) {
                t[c] = K[m3][m1] * xv[P.o1 + m1][c];
                dt[c] = __builtin_fmaf(dK[m3][m1], xv[P.o1 + m1][c], K[m3][m1] * dxv[P.o1 + m1][c]);
              } else {
                t[c] = __builtin_fmaf(K[m3][m1], xv[P.o1 + m1][c], t[c]);
                dt[c] = __builtin_fmaf(K[m3][m1], dxv[P.o1 + m1][c], dt[c]);
                dt[c] = __builtin_fmaf(dK[m3][m1], xv[P.o1 + m1][c], dt[c]);
              }
            }
          }
        });
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          acc[P.o3 + m3][c] = __builtin_fmaf(sv[c], t[c], acc[P.o3 + m3][c]);
          dacc[P.o3 + m3][c] = __builtin_fmaf(sv[c], dt[c], __builtin_fmaf(dsv[c], t[c], dacc[P.o3 + m3][c]));
        }
      });
    });
  }

  if constexpr (GPR > 1) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int d = LPG; d < LPG * GPR; d <<= 1) {
          acc[o][c] += __shfl_xor(acc[o][c], d, 64);
          dacc[o][c] += __shfl_xor(dacc[o][c], d, 64);
        }
  }

  if (valid) {
    const size_t row = (size_t)b * NO * C + c0;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      if (o % GPR != gi) continue;
      store_row<CPL>(prm.out_dot + row + (size_t)o * C, dacc[o], prm.inv_avg);
      if (prm.out) store_row<CPL>(prm.out + row + (size_t)o * C, acc[o], prm.inv_avg);
    }
  }
}

// conv_jvp with the edge loop software-pipelined like conv_fwd_pipe: the
// primal and tangent rows of the next edge are loaded while the current edge
// is accumulated (the non-pipelined kernel spends most of its time waiting for
// its loads).
template <class LY, typename IN, int CPL>
struct JvpBuf {
  EdgeBuf<LY, IN, CPL> p, t;   // (x, y, s) and (dx, dy, ds)
};

template <class LY, typename IN, int CPL>
__device__ __forceinline__ void jvp_accumulate(const JvpBuf<LY, IN, CPL>& buf, float (&acc)[LY::NO][CPL],
                                               float (&dacc)[LY::NO][CPL]) {
  constexpr int NY = LY::NY, NP = LY::NP;
  float yv[NY], dyv[NY];
#pragma unroll
  for (int j = 0; j < NY; ++j) {
    yv[j] = buf.p.y.get(j);
    dyv[j] = buf.t.y.get(j);
  }
  sfor<0, NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr PathInfo P = LY::T.path[p];
    constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
    float K[D3][D1], dK[D3][D1];
    build_k<LY, p, D3, D1>(yv, K);
    build_k<LY, p, D3, D1>(dyv, dK);
    sfor<0, D3>([&](auto m3c) {
      constexpr int m3 = decltype(m3c)::value;
      float t[CPL], dt[CPL];
      sfor<0, D1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float xv = buf.p.x[P.o1 + m1].get(c), dxv = buf.t.x[P.o1 + m1].get(c);
            if constexpr (first_m1(LY::T, p, m3) == m1) {
              t[c] = K[m3][m1] * xv;
              dt[c] = __builtin_fmaf(dK[m3][m1], xv, K[m3][m1] * dxv);
            } else {
              t[c] = __builtin_fmaf(K[m3][m1], xv, t[c]);
              dt[c] = __builtin_fmaf(K[m3][m1], dxv, dt[c]);
              dt[c] = __builtin_fmaf(dK[m3][m1], xv, dt[c]);
            }
          }
        }
      });
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float sv = buf.p.s[p].get(c), dsv = buf.t.s[p].get(c);
        acc[P.o3 + m3][c] = __builtin_fmaf(sv, t[c], acc[P.o3 + m3][c]);
        dacc[P.o3 + m3][c] = __builtin_fmaf(sv, dt[c], __builtin_fmaf(dsv, t[c], dacc[P.o3 + m3][c]));
      }
    });
  });
}

// PX: the sender rows (x, dx) are prefetched with the rest; without it they
// are loaded just before their edge is accumulated (fewer registers).
template <class LY, typename IN, int CPL, int GPR, bool PX>
__global__ void __launch_bounds__(256) conv_jvp_pipe(JvpParams prm) {
  constexpr int C = LY::C, NO = LY::NO;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;

  const IN* __restrict__ x = static_cast<const IN*>(prm.x);
  const IN* __restrict__ y = static_cast<const IN*>(prm.y);
  const IN* __restrict__ s = static_cast<const IN*>(prm.s);
  const IN* __restrict__ dx = static_cast<const IN*>(prm.dx);
  const IN* __restrict__ dy = static_cast<const IN*>(prm.dy);
  const IN* __restrict__ ds = static_cast<const IN*>(prm.ds);
  const int* __restrict__ src = prm.src;
  const int* __restrict__ row_ptr = prm.row_ptr;

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const int gi = grp % GPR;
  const int slot = grp / GPR;
  const int bl = logical_wave() * RPW + slot;
  const bool valid = bl < prm.num_nodes;
  const int b = valid ? (prm.order ? prm.order[bl] : bl) : 0;
  const int c0 = li * CPL;

  float acc[NO][CPL], dacc[NO][CPL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      acc[o][c] = 0.0f;
      dacc[o][c] = 0.0f;
    }

  int beg = 0, end = 0;
  if (valid) {
    beg = row_ptr[b];
    end = b < prm.num_real ? row_ptr[b + 1] : beg;
  }

  constexpr int NX = LY::NX, NY = LY::NY, NP = LY::NP;
  // the edge's rows: y, dy, s, ds (and x, dx of sender a when PX)
  auto load = [&](JvpBuf<LY, IN, CPL>& buf, int e, int a) {
    load_raw<IN, NY, true>(y + (size_t)e * NY, buf.p.y);
    load_raw<IN, NY, true>(dy + (size_t)e * NY, buf.t.y);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      load_raw<IN, CPL, true>(s + ((size_t)e * NP + p) * C + c0, buf.p.s[p]);
      load_raw<IN, CPL, true>(ds + ((size_t)e * NP + p) * C + c0, buf.t.s[p]);
    }
    if constexpr (PX) {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        load_raw<IN, CPL, false>(x + ((size_t)a * NX + i) * C + c0, buf.p.x[i]);
        load_raw<IN, CPL, false>(dx + ((size_t)a * NX + i) * C + c0, buf.t.x[i]);
      }
    }
  };
  auto load_x = [&](JvpBuf<LY, IN, CPL>& buf, int a) {
    if constexpr (!PX) {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        load_raw<IN, CPL, false>(x + ((size_t)a * NX + i) * C + c0, buf.p.x[i]);
        load_raw<IN, CPL, false>(dx + ((size_t)a * NX + i) * C + c0, buf.t.x[i]);
      }
    }
  };
  JvpBuf<LY, IN, CPL> b0, b1;
  int e = beg + gi;
  int a = e < end ? src[e] : 0;
  if (e < end) load(b0, e, a);
  int en = e + GPR;
  int an = en < end ? src[en] : 0;
  // Unconditional loads, clamped to the receiver's last edge past its end
  // (a conditional load makes the compiler wait for all loads in flight).
  while (e < end) {
    int en2 = en + GPR;
    int an2 = src[en2 < end ? en2 : end - 1];
    load_x(b0, a);
    load(b1, en < end ? en : end - 1, an);
    jvp_accumulate<LY, IN, CPL>(b0, acc, dacc);
    e = en;
    a = an;
    en = en2;
    an = an2;
    if (e >= end) break;
    en2 = en + GPR;
    an2 = src[en2 < end ? en2 : end - 1];
    load_x(b1, a);
    load(b0, en < end ? en : end - 1, an);
    jvp_accumulate<LY, IN, CPL>(b1, acc, dacc);
    e = en;
    a = an;
    en = en2;
    an = an2;
  }

  if constexpr (GPR > 1) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int d = LPG; d < LPG * GPR; d <<= 1) {
          acc[o][c] += __shfl_xor(acc[o][c], d, 64);
          dacc[o][c] += __shfl_xor(dacc[o][c], d, 64);
        }
  }

  if (valid) {
    const size_t row = (size_t)b * NO * C + c0;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      if (o % GPR != gi) continue;
      store_row<CPL>(prm.out_dot + row + (size_t)o * C, dacc[o], prm.inv_avg);
      if (prm.out) store_row<CPL>(prm.out + row + (size_t)o * C, acc[o], prm.inv_avg);
    }
  }
}

// ----------------------------------------------------------- backward -------

// Edges into a padding receiver (node mask) carry no gradient: their grad_y
// and grad_s rows are zero and nothing reaches grad_x.
template <class LY>
__device__ __forceinline__ void zero_edge_grads(const BwdParams& prm, int e0, int end, int step,
                                                int li, int lpg) {
  constexpr int PC = LY::NP * LY::C, NY = LY::NY;
  const bool zs = prm.gs && !(prm.flags & kAccumulateS);   // an accumulated zero is a no-op
  const bool zy = prm.gy && !(prm.flags & kAccumulateY);
  for (int e = e0; e < end; e += step) {
    if (zs)
      for (int k = li; k < PC; k += lpg) __builtin_nontemporal_store(0.0f, prm.gs + (size_t)e * PC + k);
    if (zy)
      for (int k = li; k < NY; k += lpg) prm.gy[(size_t)e * NY + k] = 0.0f;
  }
}
//
// Reverse pass of L = <g, out>, receiver ordered: the cotangent row g[b] is
// loaded once per receiver; per incoming edge the narrow sender row x[a] is
// gathered (the reason the e3j page gives for preferring RECEIVER ordering:
// the reverse pass then reads x rows per edge, narrower than cotangent rows).  With t^p = K^p x[a] and
// h^p = s^p * g[b] / N (per channel):
//   grad_s[e,p] = sum_m3 g[b][o3+m3] t^p[m3] / N
//   grad_y[e,o2+m2] = sum_p sum_c sum_{m1,m3} C^p[m1,m2,m3] x[a][o1+m1] h^p[m3]
//   grad_x[a][o1+m1] += sum_p sum_m3 K^p[m3][m1] h^p[m3]      (device atomics)
// Lanes hold channels li, li+LPG, ... so every atomic and store instruction of
// a group touches consecutive floats.

template <class LY, int CPL, int GPR>
__global__ void __launch_bounds__(256) conv_bwd(BwdParams prm) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NO = LY::NO, NP = LY::NP;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;
  constexpr int NYP = pow2_ceil(NY);
  constexpr int STEPS = ilog2(LPG);

  const float* __restrict__ x = prm.x;
  const float* __restrict__ y = prm.y;
  const float* __restrict__ s = prm.s;
  const int* __restrict__ src = prm.src;
  const int* __restrict__ row_ptr = prm.row_ptr;

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const int gi = grp % GPR;
  const int slot = grp / GPR;
  const int bl = logical_wave() * RPW + slot;
  if (bl >= prm.num_nodes) return;   // whole slots only: no cross-lane work follows an early exit
  const int b = prm.order ? prm.order[bl] : bl;

  const int beg = row_ptr[b];
  const int end = row_ptr[b + 1];
  if (b >= prm.num_real) {
    zero_edge_grads<LY>(prm, beg + gi, end, GPR, li, LPG);
    return;
  }

  float gv[NO][CPL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      gv[o][c] = prm.g[((size_t)b * NO + o) * C + li + c * LPG] * prm.inv_avg;

  for (int e = beg + gi; e < end; e += GPR) {
    const int a = src[e];
    float yv[NY];
    load_row<float, NY>(y + (size_t)e * NY, yv);
    float xv[NX][CPL];
#pragma unroll
    for (int i = 0; i < NX; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) xv[i][c] = x[((size_t)a * NX + i) * C + li + c * LPG];

    float dxp[NX][CPL];
#pragma unroll
    for (int i = 0; i < NX; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) dxp[i][c] = 0.0f;
    float dyp[NYP];
#pragma unroll
    for (int j = 0; j < NYP; ++j) dyp[j] = 0.0f;

    const float* srow = s + (size_t)e * NP * C + li;
    float* gsrow = prm.gs + (size_t)e * NP * C + li;

    sfor<0, NP>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      constexpr PathInfo P = LY::T.path[p];
      constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
      float sv[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) sv[c] = __builtin_nontemporal_load(srow + p * C + c * LPG);
      float K[D3][D1];
      build_k<LY, p, D3, D1>(yv, K);

      // t = K x, grad_s = <g, t>
      float ds[CPL];
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        float t[CPL];
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              if constexpr (first_m1(LY::T, p, m3) == m1) {
                t[c] = K[m3][m1] * xv[P.o1 + m1][c];
              } else {
                t[c] = __builtin_fmaf(K[m3][m1], xv[P.o1 + m1][c], t[c]);
              }
            }
          }
        });
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if constexpr (m3 == 0) {
            ds[c] = gv[P.o3][c] * t[c];
          } else {
            ds[c] = __builtin_fmaf(gv[P.o3 + m3][c], t[c], ds[c]);
          }
        }
      });
#pragma unroll
      for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(ds[c], gsrow + p * C + c * LPG);

      // h = s * g / N
      float h[D3][CPL];
#pragma unroll
      for (int m3 = 0; m3 < D3; ++m3)
#pragma unroll
        for (int c = 0; c < CPL; ++c) h[m3][c] = sv[c] * gv[P.o3 + m3][c];

      // grad_x contribution: K^T h
      sfor<0, D1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        sfor<0, D3>([&](auto m3c) {
          constexpr int m3 = decltype(m3c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              dxp[P.o1 + m1][c] = __builtin_fmaf(K[m3][m1], h[m3][c], dxp[P.o1 + m1][c]);
          }
        });
      });

      // grad_y: per (m1, m3) pair q = sum_c x h, then dy[o2+m2] += C q
      sfor<0, D1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        sfor<0, D3>([&](auto m3c) {
          constexpr int m3 = decltype(m3c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
            float q = xv[P.o1 + m1][0] * h[m3][0];
#pragma unroll
            for (int c = 1; c < CPL; ++c) q = __builtin_fmaf(xv[P.o1 + m1][c], h[m3][c], q);
            sfor<P.nnz_begin, P.nnz_end>([&](auto ec) {
              constexpr int qi = decltype(ec)::value;
              constexpr Entry en = LY::T.entry[qi];
              if constexpr (en.m1 == m1 && en.m3 == m3) {
                dyp[P.o2 + en.m2] = __builtin_fmaf(LY::CG.v[qi], q, dyp[P.o2 + en.m2]);
              }
            });
          }
        });
      });
    });

    // grad_x: fp32 device atomics (consecutive lanes, consecutive floats)
#pragma unroll
    for (int i = 0; i < NX; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        unsafeAtomicAdd(prm.gx + ((size_t)a * NX + i) * C + li + c * LPG, dxp[i][c]);

    // grad_y: reduce the per-lane partials over the group's LPG lanes
    // (reduce-scatter: each halving step keeps half of the components).
    sfor<0, STEPS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int d = LPG >> (k + 1);
      constexpr int n = (NYP >> k) > 1 ? (NYP >> k) : 1;
      if constexpr (n > 1) {
        const bool upper = (li & d) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
          const float send = upper ? dyp[i] : dyp[i + n / 2];
          const float keep = upper ? dyp[i + n / 2] : dyp[i];
          dyp[i] = keep + __shfl_xor(send, d, 64);
        }
      } else {
        dyp[0] += __shfl_xor(dyp[0], d, 64);
      }
    });
    constexpr int NF = (NYP >> STEPS) > 1 ? (NYP >> STEPS) : 1;   // components left per lane
    constexpr int REP = LPG > NYP ? LPG / NYP : 1;                  // lanes holding the same ones
    if ((li & (REP - 1)) == 0) {
      int base = 0;
#pragma unroll
      for (int k = 0; k < STEPS; ++k) {
        const int d = LPG >> (k + 1);
        const int n = (NYP >> k) > 1 ? (NYP >> k) : 1;
        if (n > 1 && (li & d)) base += n / 2;
      }
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int comp = base + j;
        if (comp < NY) prm.gy[(size_t)e * NY + comp] = dyp[j];
      }
    }
  }
}

// ------------------------------------------------- pipelined backward -------
//
// conv_bwd with the edge loop software-pipelined like conv_fwd_pipe: the next
// edge's y, s and gathered x values are loaded while the current edge is
// processed.  Same per-edge arithmetic and output writes as conv_bwd.

template <class LY, int CPL>
struct BwdBuf {
  float y[LY::NY];
  float x[LY::NX][CPL];
  float s[LY::NP][CPL];
};

template <class LY, int CPL, int LPG>
__device__ __forceinline__ void load_bwd_edge(BwdBuf<LY, CPL>& buf, const float* __restrict__ x,
                                              const float* __restrict__ y,
                                              const float* __restrict__ s, int e, int a, int li) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP;
  load_row<float, NY>(y + (size_t)e * NY, buf.y);
  const float* xrow = x + (size_t)a * NX * C + li;
#pragma unroll
  for (int i = 0; i < NX; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) buf.x[i][c] = xrow[i * C + c * LPG];
  const float* srow = s + (size_t)e * NP * C + li;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int c = 0; c < CPL; ++c) buf.s[p][c] = __builtin_nontemporal_load(srow + p * C + c * LPG);
}

// GEN: honour optional outputs (nullptr: not computed) and accumulation flags;
// the default instantiations assume all three outputs, overwritten.
template <class LY, int CPL, int LPG, bool GEN = false>
__device__ __forceinline__ void bwd_edge(const BwdBuf<LY, CPL>& buf, const float (&gv)[LY::NO][CPL],
                                         const BwdParams& prm, int e, int a, int li) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP;
  constexpr int NYP = pow2_ceil(NY);
  constexpr int STEPS = ilog2(LPG);
  float dxp[NX][CPL];
#pragma unroll
  for (int i = 0; i < NX; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) dxp[i][c] = 0.0f;
  float dyp[NYP];
#pragma unroll
  for (int j = 0; j < NYP; ++j) dyp[j] = 0.0f;
  const bool want_s = !GEN || prm.gs;
  const bool want_y = !GEN || prm.gy;
  const bool want_x = !GEN || prm.gx;
  float* gsrow = want_s ? prm.gs + (size_t)e * NP * C + li : nullptr;
  // Accumulating into grad_s: fetch the edge's rows up front, in one batch,
  // rather than one dependent load per path before its store.
  float gs_prev[GEN ? NP : 1][CPL];
  const bool acc_s = GEN && want_s && (prm.flags & kAccumulateS);
  if constexpr (GEN) {
    if (acc_s) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int c = 0; c < CPL; ++c) gs_prev[p][c] = __builtin_nontemporal_load(gsrow + p * C + c * LPG);
    }
  }

  // Per path, with w = K^T g (g already divided by N):
  //   grad_s = sum_m1 x[o1+m1] w[m1]            (= <g, K x>)
  //   grad_x += s w                             (= K^T (s g))
  //   grad_y[o2+m2] += sum_{m1,m3} C[m1,m2,m3] sum_c (s x[o1+m1]) g[o3+m3]
  sfor<0, NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr PathInfo P = LY::T.path[p];
    constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
    float K[D3][D1];
    build_k<LY, p, D3, D1>(buf.y, K);
    float ds[CPL];
    sfor<0, D1>([&](auto m1c) {
      constexpr int m1 = decltype(m1c)::value;
      float w[CPL];
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            if constexpr (first_m3(LY::T, p, m1) == m3) {
              w[c] = K[m3][m1] * gv[P.o3 + m3][c];
            } else {
              w[c] = __builtin_fmaf(K[m3][m1], gv[P.o3 + m3][c], w[c]);
            }
          }
        }
      });
      if constexpr (first_m3(LY::T, p, m1) >= 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if constexpr (m1 == 0) {
            ds[c] = buf.x[P.o1][c] * w[c];
          } else {
            ds[c] = __builtin_fmaf(buf.x[P.o1 + m1][c], w[c], ds[c]);
          }
          dxp[P.o1 + m1][c] = __builtin_fmaf(buf.s[p][c], w[c], dxp[P.o1 + m1][c]);
        }
      } else if constexpr (m1 == 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) ds[c] = 0.0f;
      }
    });
    if constexpr (GEN) {
      if (want_s) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          __builtin_nontemporal_store(acc_s ? ds[c] + gs_prev[p][c] : ds[c], gsrow + p * C + c * LPG);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(ds[c], gsrow + p * C + c * LPG);
    }

    if (want_y) sfor<0, D1>([&](auto m1c) {
      constexpr int m1 = decltype(m1c)::value;
      if constexpr (first_m3(LY::T, p, m1) >= 0) {
        float u[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) u[c] = buf.s[p][c] * buf.x[P.o1 + m1][c];
        sfor<0, D3>([&](auto m3c) {
          constexpr int m3 = decltype(m3c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
            float q = u[0] * gv[P.o3 + m3][0];
#pragma unroll
            for (int c = 1; c < CPL; ++c) q = __builtin_fmaf(u[c], gv[P.o3 + m3][c], q);
            sfor<P.nnz_begin, P.nnz_end>([&](auto ec) {
              constexpr int qi = decltype(ec)::value;
              constexpr Entry en = LY::T.entry[qi];
              if constexpr (en.m1 == m1 && en.m3 == m3) {
                dyp[P.o2 + en.m2] = __builtin_fmaf(LY::CG.v[qi], q, dyp[P.o2 + en.m2]);
              }
            });
          }
        });
      }
    });
  });

  if (want_x) {
#pragma unroll
    for (int i = 0; i < NX; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        unsafeAtomicAdd(prm.gx + ((size_t)a * NX + i) * C + li + c * LPG, dxp[i][c]);
  }
  if (!want_y) return;

  sfor<0, STEPS>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int d = LPG >> (k + 1);
    constexpr int n = (NYP >> k) > 1 ? (NYP >> k) : 1;
    if constexpr (n > 1) {
      const bool upper = (li & d) != 0;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float send = upper ? dyp[i] : dyp[i + n / 2];
        const float keep = upper ? dyp[i + n / 2] : dyp[i];
        dyp[i] = keep + __shfl_xor(send, d, 64);
      }
    } else {
      dyp[0] += __shfl_xor(dyp[0], d, 64);
    }
  });
  constexpr int NF = (NYP >> STEPS) > 1 ? (NYP >> STEPS) : 1;
  constexpr int REP = LPG > NYP ? LPG / NYP : 1;
  if ((li & (REP - 1)) == 0) {
    int base = 0;
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
      const int d = LPG >> (k + 1);
      const int n = (NYP >> k) > 1 ? (NYP >> k) : 1;
      if (n > 1 && (li & d)) base += n / 2;
    }
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int comp = base + j;
      if (comp < NY) {
        float* dst = prm.gy + (size_t)e * NY + comp;
        *dst = (GEN && (prm.flags & kAccumulateY)) ? dyp[j] + *dst : dyp[j];
      }
    }
  }
}

template <class LY, int CPL, int GPR, bool GEN = false>
__global__ void __launch_bounds__(256) conv_bwd_pipe(BwdParams prm) {
  constexpr int C = LY::C, NO = LY::NO;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;

  const float* __restrict__ x = prm.x;
  const float* __restrict__ y = prm.y;
  const float* __restrict__ s = prm.s;
  const int* __restrict__ src = prm.src;

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const int gi = grp % GPR;
  const int slot = grp / GPR;
  const int bl = logical_wave() * RPW + slot;
  if (bl >= prm.num_nodes) return;   // whole slots only: no cross-lane work follows an early exit
  const int b = prm.order ? prm.order[bl] : bl;

  const int beg = prm.row_ptr[b];
  const int end = prm.row_ptr[b + 1];
  if (b >= prm.num_real) {
    zero_edge_grads<LY>(prm, beg + gi, end, GPR, li, LPG);
    return;
  }

  float gv[NO][CPL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      gv[o][c] = prm.g[((size_t)b * NO + o) * C + li + c * LPG] * prm.inv_avg;

  BwdBuf<LY, CPL> b0, b1;
  int e = beg + gi;
  int a = 0;
  if (e < end) {
    a = src[e];
    load_bwd_edge<LY, CPL, LPG>(b0, x, y, s, e, a, li);
  }
  int en = e + GPR;
  int an = en < end ? src[en] : 0;
  // The sender index two edges ahead and the next edge's rows are loaded
  // unconditionally, clamped to the receiver's last edge past its end: a
  // conditional load, merged into the loop variable, makes the compiler wait
  // for every memory operation in flight, this edge's gradient stores included.
  while (e < end) {
    int en2 = en + GPR;
    int an2 = src[en2 < end ? en2 : end - 1];
    load_bwd_edge<LY, CPL, LPG>(b1, x, y, s, en < end ? en : end - 1, an, li);
    bwd_edge<LY, CPL, LPG, GEN>(b0, gv, prm, e, a, li);
    e = en;
    a = an;
    en = en2;
    an = an2;
    if (e >= end) break;
    en2 = en + GPR;
    an2 = src[en2 < end ? en2 : end - 1];
    load_bwd_edge<LY, CPL, LPG>(b0, x, y, s, en < end ? en : end - 1, an, li);
    bwd_edge<LY, CPL, LPG, GEN>(b1, gv, prm, e, a, li);
    e = en;
    a = an;
    en = en2;
    an = an2;
  }
}

__global__ void fill_zero(float* __restrict__ p, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0.0f;
}

// ------------------------------------------------------------- launchers ----


template <class LY, typename IN, int CPL, int GPR>
hipError_t launch_fwd(const FwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_fwd<LY, IN, CPL, GPR>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class LY, typename IN, int CPL, int GPR, bool UL = false>
hipError_t launch_fwd_pipe(const FwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_fwd_pipe<LY, IN, CPL, GPR, UL>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class LY, int CPL, int GPR>
hipError_t launch_bwd(const BwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  const size_t nx = (size_t)p.num_nodes * LY::NX * LY::C;
  const unsigned zb = (unsigned)((nx + 255) / 256 < 8192 ? (nx + 255) / 256 : 8192);
  hipLaunchKernelGGL(fill_zero, dim3(zb), dim3(256), 0, st, p.gx, nx);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_bwd<LY, CPL, GPR>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class LY, int CPL, int GPR, bool GEN = false>
hipError_t launch_bwd_pipe(const BwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  if (p.gx && !(p.flags & kAccumulateX)) {
    const size_t nx = (size_t)p.num_nodes * LY::NX * LY::C;
    const unsigned zb = (unsigned)((nx + 255) / 256 < 8192 ? (nx + 255) / 256 : 8192);
    hipLaunchKernelGGL(fill_zero, dim3(zb), dim3(256), 0, st, p.gx, nx);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_bwd_pipe<LY, CPL, GPR, GEN>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class LY, typename IN, int CPL, int GPR, bool PX>
hipError_t launch_jvp_pipe(const JvpParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_jvp_pipe<LY, IN, CPL, GPR, PX>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class LY, typename IN, int CPL, int GPR>
hipError_t launch_jvp(const JvpParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_jvp<LY, IN, CPL, GPR>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace e3c
