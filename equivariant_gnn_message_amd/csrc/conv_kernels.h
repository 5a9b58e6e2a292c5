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
// The grid is a multiple of 8 work-groups of WPB waves.
template <int WPB = 4>
__device__ __forceinline__ int logical_wave() {
  const int per_xcd = (int)(gridDim.x >> 3);
  const int bid = (int)blockIdx.x;
  const int lb = (bid & 7) * per_xcd + (bid >> 3);
  return __builtin_amdgcn_readfirstlane(lb * WPB + (WPB > 1 ? (int)(threadIdx.x >> 6) : 0));
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

// Entries of one path's K^p that are equal up to sign.  Within a path many
// entries K[m3][m1] = sum_m2 C[m1,m2,m3] y[m2] have the same terms (the same
// m2, coefficients of equal magnitude) up to one common sign; the table below
// finds them at compile time from the coefficient values.  Each entry is
// mapped to the first entry (in the order of the entry list) with the same
// terms up to sign; only those representatives are computed, and the others
// are their copies or negations, which the compiler folds into the source
// modifiers of the instructions that use them.
struct KRefTable {
  int8_t rm3[kMaxNnz];   // representative of the K entry of CG entry q
  int8_t rm1[kMaxNnz];
  int8_t sgn[kMaxNnz];   // +1 or -1
};

// True if the K entries of CG entries qa and qb (same path) have the same
// terms up to one common sign, returned in sgn.
constexpr bool k_terms_match(const LayoutTables& t, const float* v, int p, int qa, int qb, int& sgn) {
  const int a3 = t.entry[qa].m3, a1 = t.entry[qa].m1, b3 = t.entry[qb].m3, b1 = t.entry[qb].m1;
  int na = 0, nb = 0;
  sgn = 0;
  for (int q = t.path[p].nnz_begin; q < t.path[p].nnz_end; ++q) {
    if (t.entry[q].m3 == b3 && t.entry[q].m1 == b1) ++nb;
    if (t.entry[q].m3 != a3 || t.entry[q].m1 != a1) continue;
    ++na;
    int r = -1;
    for (int q2 = t.path[p].nnz_begin; q2 < t.path[p].nnz_end; ++q2)
      if (t.entry[q2].m3 == b3 && t.entry[q2].m1 == b1 && t.entry[q2].m2 == t.entry[q].m2) r = q2;
    if (r < 0) return false;
    const float va = v[q], vb = v[r];
    const float aa = va < 0.0f ? -va : va, ab = vb < 0.0f ? -vb : vb;
    if (aa == 0.0f && ab == 0.0f) continue;
    const float d = aa > ab ? aa - ab : ab - aa;
    if (aa == 0.0f || ab == 0.0f || d > 1e-6f * aa) return false;
    const int s = (va < 0.0f) != (vb < 0.0f) ? -1 : 1;
    if (sgn == 0) sgn = s;
    if (sgn != s) return false;
  }
  if (sgn == 0) sgn = 1;
  return na == nb;
}

template <class LY>
constexpr KRefTable make_kref() {
  KRefTable r{};
  const LayoutTables& t = LY::T;
  for (int p = 0; p < t.num_paths; ++p)
    for (int q = t.path[p].nnz_begin; q < t.path[p].nnz_end; ++q) {
      r.rm3[q] = t.entry[q].m3;
      r.rm1[q] = t.entry[q].m1;
      r.sgn[q] = 1;
      for (int q2 = t.path[p].nnz_begin; q2 < q; ++q2) {
        if (!first_term(t, p, q2)) continue;
        if (t.entry[q2].m3 == t.entry[q].m3 && t.entry[q2].m1 == t.entry[q].m1) break;
        int sg = 0;
        if (k_terms_match(t, LY::CG.v, p, q, q2, sg)) {
          r.rm3[q] = t.entry[q2].m3;
          r.rm1[q] = t.entry[q2].m1;
          r.sgn[q] = (int8_t)sg;
          break;
        }
      }
    }
  return r;
}

template <class LY>
struct KRefs {
  static constexpr KRefTable R = make_kref<LY>();
};

// K^p[m3][m1] = sum_m2 C^p[m1,m2,m3] y[o2+m2] over the compile-time pattern,
// each class of entries equal up to sign computed once.
template <class LY, int p, int D3, int D1>
__device__ __forceinline__ void build_k(const float (&yv)[LY::NY], float (&K)[D3][D1]) {
  constexpr PathInfo P = LY::T.path[p];
  sfor<P.nnz_begin, P.nnz_end>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    constexpr Entry en = LY::T.entry[q];
    if constexpr (KRefs<LY>::R.rm3[q] == en.m3 && KRefs<LY>::R.rm1[q] == en.m1) {
      constexpr float c = LY::CG.v[q];
      const float yy = yv[P.o2 + en.m2];
      if constexpr (first_term(LY::T, p, q)) {
        K[en.m3][en.m1] = c * yy;
      } else {
        K[en.m3][en.m1] = __builtin_fmaf(c, yy, K[en.m3][en.m1]);
      }
    }
  });
  sfor<P.nnz_begin, P.nnz_end>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    constexpr Entry en = LY::T.entry[q];
    constexpr int r3 = KRefs<LY>::R.rm3[q], r1 = KRefs<LY>::R.rm1[q];
    if constexpr (first_term(LY::T, p, q) && !(r3 == en.m3 && r1 == en.m1)) {
      if constexpr (KRefs<LY>::R.sgn[q] > 0) {
        K[en.m3][en.m1] = K[r3][r1];
      } else {
        K[en.m3][en.m1] = -K[r3][r1];
      }
    }
  });
}

// Orders a wave's LDS accesses around an exchange between its lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Adds a group's partial rows v into dst (NR rows of C floats) with fp32
// atomics.  Lane li holds channels li*CPL .. li*CPL+CPL-1 of each row; the
// rows are re-laid through the group's LDS rows xt (NR * C floats) so that
// lane li adds channels li + c*LPG, and each atomic instruction of the group
// covers consecutive channels.
template <int C, int NR, int CPL, int LPG>
__device__ __forceinline__ void atomic_add_rows(float* dst, const float (&v)[NR][CPL], float* xt,
                                                int li) {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if constexpr (CPL == 4) {
      *reinterpret_cast<f32x4*>(xt + i * C + li * 4) = f32x4{v[i][0], v[i][1], v[i][2], v[i][3]};
    } else if constexpr (CPL == 2) {
      *reinterpret_cast<f32x2*>(xt + i * C + li * 2) = f32x2{v[i][0], v[i][1]};
    } else {
      xt[i * C + li] = v[i][0];
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) unsafeAtomicAdd(dst + i * C + li + c * LPG, xt[i * C + li + c * LPG]);
  wave_lds_sync();
}

// Sums the group's per-lane partial edge-feature gradients dyp (NY used of
// pow2_ceil(NY)) over its LPG lanes and writes the row dst[0 .. NY), or adds
// it when acc.  Each butterfly step halves the components a lane keeps, so
// the sum costs NYP - 1 shuffles rather than NY log2(LPG).
template <int NY, int LPG>
__device__ __forceinline__ void store_dy(float (&dyp)[pow2_ceil(NY)], float* dst, int li, bool acc) {
  constexpr int NYP = pow2_ceil(NY);
  constexpr int STEPS = ilog2(LPG);
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
      if (comp < NY) dst[comp] = acc ? dyp[j] + dst[comp] : dyp[j];
    }
  }
}

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

// A lane's CPL consecutive floats in LDS (its own channels: no exchange).
template <int CPL>
__device__ __forceinline__ void lds_store_ch(float* p, const float (&v)[CPL], float scale) {
  if constexpr (CPL == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale};
  } else if constexpr (CPL == 2) {
    *reinterpret_cast<f32x2*>(p) = f32x2{v[0] * scale, v[1] * scale};
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) p[c] = v[c] * scale;
  }
}

template <int CPL>
__device__ __forceinline__ void lds_load_ch(const float* p, float (&v)[CPL]) {
  if constexpr (CPL == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else if constexpr (CPL == 2) {
    const f32x2 t = *reinterpret_cast<const f32x2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = p[c];
  }
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

// ------------------------------------------------ fused output linear ------

// Output blocks of a block code.
constexpr int num_blocks(uint32_t code) {
  int n = 0;
  for (int l = 0; l <= kMaxL; ++l) n += block_parity(code, l) != 0;
  return n;
}

// The output channels v0 .. v0+VL-1 of every component of receiver b from its
// summed row (LDS) and the weights (LDS).
template <class LY, int VL>
__device__ __forceinline__ void lin_rows(const float* w, const float* row, const FwdParams& prm,
                                         int b, int v0) {
  constexpr int C = LY::C, NO = LY::NO;
  float res[NO][VL];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int c = 0; c < VL; ++c) res[o][c] = 0.0f;
  int k = 0;
  sfor<0, kMaxL + 1>([&](auto lc) {
    constexpr int l = decltype(lc)::value;
    if constexpr (block_parity(LY::OCODE, l) != 0) {
      constexpr int ob = code_offset(LY::OCODE, l);
      const float* wk = w + k * C * C + v0;
#pragma unroll 2
      for (int u = 0; u < C; u += 4) {
        float wv[4][VL];
#pragma unroll
        for (int q = 0; q < 4; ++q) lds_load_ch<VL>(wk + (u + q) * C, wv[q]);
#pragma unroll
        for (int m = 0; m < 2 * l + 1; ++m) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(row + (ob + m) * C + u);
#pragma unroll
          for (int c = 0; c < VL; ++c) {
            res[ob + m][c] = __builtin_fmaf(a.x, wv[0][c], res[ob + m][c]);
            res[ob + m][c] = __builtin_fmaf(a.y, wv[1][c], res[ob + m][c]);
            res[ob + m][c] = __builtin_fmaf(a.z, wv[2][c], res[ob + m][c]);
            res[ob + m][c] = __builtin_fmaf(a.w, wv[3][c], res[ob + m][c]);
          }
        }
      }
      ++k;
    }
  });
  float* orow = prm.out + (size_t)b * NO * C + v0;
#pragma unroll
  for (int o = 0; o < NO; ++o) store_row<VL>(orow + (size_t)o * C, res[o], prm.lin_alpha);
}

// Fused output linear (the step after the convolution, cuEquivariance page,
// Flax NNX layers, IrrepsLinear: each output irrep block mixed over its
// channels by a C x C weight matrix, scaled by scale / sqrt(C)).  The receiver's summed row goes through the wave's LDS
// row; then the GPR * LPG lanes of the receiver each produce C / (GPR * LPG)
// output channels of every component,
//   out[b, o, v] = lin_alpha * sum_u row[o, u] W_k(o)[u, v]
// (lin_alpha = scale / sqrt(C) / N), W staged in LDS once per work-group.
template <class LY, int CPL, int GPR>
__device__ __forceinline__ void lin_epilogue(const float (&acc)[LY::NO][CPL], const float* w,
                                             float* row, const FwdParams& prm, int b, bool valid,
                                             int li, int gi) {
  constexpr int C = LY::C, NO = LY::NO;
  constexpr int LPG = C / CPL;
  constexpr int EL = LPG * GPR;                 // lanes of one receiver
  constexpr int VL = C / EL > 0 ? C / EL : 1;   // output channels per lane
  static_assert(C % 4 == 0, "rows are read four channels at a time");
  if (gi == 0) {
#pragma unroll
    for (int o = 0; o < NO; ++o) lds_store_ch<CPL>(row + o * C + li * CPL, acc[o], 1.0f);
  }
  wave_lds_sync();
  const int v0 = (gi * LPG + li) * VL;
  if (valid && v0 < C) lin_rows<LY, VL>(w, row, prm, b, v0);
  wave_lds_sync();   // the row is rewritten for the wave's next receiver
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

// A row of N floats at a wave-uniform address, read through the scalar cache.
template <int N>
__device__ __forceinline__ void load_row_uniform(const float* p, float (&v)[N]) {
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* q = (cfloat*)(uintptr_t)p;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = q[i];
}

template <class LY, typename IN, int CPL>
struct EdgeBuf {
  RawVec<IN, LY::NY> y;
  RawVec<IN, CPL> x[LY::NX];
  RawVec<IN, CPL> s[LY::NP];
  float ysg;              // pair-stored rows: -1 when the edge is its pair's reverse (P y)
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

// Pair-stored edge data (PR; the symmetry of the e3j Convolution page's note
// on SENDER ordering): the edge's y and s rows are its pair's, read at row
// |p| of the pair arrays, with the odd-l blocks of y negated when the edge is
// the reverse of the stored one (p < 0: ~p is the pair).
template <class LY, typename IN, int CPL>
__device__ __forceinline__ void load_edge_pair(EdgeBuf<LY, IN, CPL>& buf, const IN* __restrict__ x,
                                               const IN* __restrict__ y, const IN* __restrict__ s,
                                               int p, int a, int c0) {
  load_edge<LY, IN, CPL>(buf, x, y, s, p >= 0 ? p : ~p, a, c0);
  buf.ysg = p >= 0 ? 1.0f : -1.0f;
}

template <class LY, typename IN, int CPL, bool PR = false>
__device__ __forceinline__ void edge_accumulate(const EdgeBuf<LY, IN, CPL>& buf,
                                                float (&acc)[LY::NO][CPL]) {
  constexpr int NY = LY::NY, NP = LY::NP;
  float yv[NY];
#pragma unroll
  for (int j = 0; j < NY; ++j) yv[j] = buf.y.get(j);
  if constexpr (PR) {
#pragma unroll
    for (int l = 1; l * l < NY; l += 2)
#pragma unroll
      for (int j = l * l; j < (l + 1) * (l + 1); ++j) yv[j] *= buf.ysg;
  }
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
// The receivers of wave slot ws (RPW of them): one per GPR groups.
template <class LY, typename IN, int CPL, int GPR, bool UL, bool LIN, bool PR>
__device__ __forceinline__ void fwd_pipe_receivers(const FwdParams& prm, int ws, const float* lin_w,
                                                   float* lin_row) {
  constexpr int C = LY::C, NO = LY::NO;
  constexpr int LPG = C / CPL;
  constexpr int G = 64 / LPG;
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
  const int bl = ws * RPW + slot;
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

  // PR: the pair map entry of an edge is fetched with its sender index
  const int* __restrict__ emap = prm.emap;
  auto pmap = [&](int ee) { return PR ? emap[ee] : 0; };
  auto ld = [&](EdgeBuf<LY, IN, CPL>& buf, int ee, int a, int pm) {
    if constexpr (PR) {
      load_edge_pair<LY, IN, CPL>(buf, x, y, s, pm, a, c0);
    } else {
      load_edge<LY, IN, CPL>(buf, x, y, s, ee, a, c0);
    }
  };
  EdgeBuf<LY, IN, CPL> b0, b1;
  int e = beg + gi;
  if (e < end) ld(b0, e, src[e], pmap(e));
  int en = e + GPR;
  int an = en < end ? src[en] : 0;
  int pn = en < end ? pmap(en) : 0;
  while (e < end) {
    int en2 = en + GPR;
    int an2, pn2;
    if constexpr (UL) {
      an2 = src[en2 < end ? en2 : end - 1];
      pn2 = pmap(en2 < end ? en2 : end - 1);
      ld(b1, en < end ? en : end - 1, an, pn);
    } else {
      if (en < end) ld(b1, en, an, pn);
      an2 = en2 < end ? src[en2] : 0;
      pn2 = en2 < end ? pmap(en2) : 0;
    }
    edge_accumulate<LY, IN, CPL, PR>(b0, acc);
    e = en;
    en = en2;
    an = an2;
    pn = pn2;
    if (e >= end) break;
    en2 = en + GPR;
    if constexpr (UL) {
      an2 = src[en2 < end ? en2 : end - 1];
      pn2 = pmap(en2 < end ? en2 : end - 1);
      ld(b0, en < end ? en : end - 1, an, pn);
    } else {
      if (en < end) ld(b0, en, an, pn);
      an2 = en2 < end ? src[en2] : 0;
      pn2 = en2 < end ? pmap(en2) : 0;
    }
    edge_accumulate<LY, IN, CPL, PR>(b1, acc);
    e = en;
    en = en2;
    an = an2;
    pn = pn2;
  }

  if constexpr (GPR > 1) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int d = LPG; d < LPG * GPR; d <<= 1) acc[o][c] += __shfl_xor(acc[o][c], d, 64);
  }

  if constexpr (LIN) {
    lin_epilogue<LY, CPL, GPR>(acc, lin_w, lin_row + slot * NO * C, prm, b, valid, li, gi);
    return;
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

// LIN: the output linear fused into the epilogue.  Its weights (NB blocks of
// C x C) are staged in LDS once per work-group, so the work-groups loop over
// contiguous ranges of wave slots rather than taking one each.
template <class LY, typename IN, int CPL, int GPR, bool UL = false, bool LIN = false, bool PR = false,
          int WPB = 4>
__global__ void __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(PR ? 2 : 1)))
conv_fwd_pipe(FwdParams prm) {
  constexpr int C = LY::C, NO = LY::NO;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  static_assert(G % GPR == 0, "groups per receiver must divide groups per wave");
  constexpr int RPW = G / GPR;
  if constexpr (!LIN) {
    fwd_pipe_receivers<LY, IN, CPL, GPR, UL, false, PR>(prm, logical_wave<WPB>(), nullptr, nullptr);
  } else {
    constexpr int NB = num_blocks(LY::OCODE);
    __shared__ float lin_w[NB * C * C];
    __shared__ float lin_row[4][RPW * NO * C];    // one row per receiver slot of each wave
    for (int i = threadIdx.x; i < NB * C * C; i += blockDim.x) lin_w[i] = prm.lin_w[i];
    __syncthreads();
    const int waves = (int)gridDim.x * 4;
    const int slots = (prm.num_nodes + RPW - 1) / RPW;
    const int per = (slots + waves - 1) / waves;
    const int w0 = logical_wave() * per;
    const int w1 = w0 + per < slots ? w0 + per : slots;
    for (int ws = w0; ws < w1; ++ws)
      fwd_pipe_receivers<LY, IN, CPL, GPR, UL, true, PR>(prm, ws, lin_w, lin_row[threadIdx.x >> 6]);
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
template <class LY, typename IN, int CPL, int GPR, bool PX, int WPB = 4>
__global__ void __launch_bounds__(64 * WPB) conv_jvp_pipe(JvpParams prm) {
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
  const int bl = logical_wave<WPB>() * RPW + slot;
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

    store_dy<NY, LPG>(dyp, prm.gy + (size_t)e * NY, li, false);
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

// The lane holds channels li, li+LPG, ... (one 4-byte access per channel).
// With one group per wave (LPG = 64) the edge is wave-uniform and its y row
// is read through the scalar cache.
template <class LY, int CPL, int LPG>
__device__ __forceinline__ void load_bwd_edge(BwdBuf<LY, CPL>& buf, const float* __restrict__ x,
                                              const float* __restrict__ y,
                                              const float* __restrict__ s, int e, int a, int li) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP;
  if constexpr (LPG == 64) {
    load_row_uniform<NY>(y + (size_t)__builtin_amdgcn_readfirstlane(e) * NY, buf.y);
  } else {
    load_row<float, NY>(y + (size_t)e * NY, buf.y);
  }
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
// Q: contiguous channel quads (see load_bwd_edge); the grad_x partials are
// then re-laid through the group's LDS rows xt (NX * C floats) so that each
// atomic instruction of the group covers consecutive channels.
// after(p) runs once path p's last use of the edge's s[p] is done (the tiled
// kernel reloads s[p] with the next edge's row there).
struct NoAfterPath {
  template <class P>
  __device__ __forceinline__ void operator()(P) const {}
};

template <class LY, int CPL, int LPG, bool GEN = false, bool Q = false, class After = NoAfterPath>
__device__ __forceinline__ void bwd_edge(const BwdBuf<LY, CPL>& buf, const float (&gv)[LY::NO][CPL],
                                         const BwdParams& prm, int e, int a, int li,
                                         float* xt = nullptr, After after = After{}) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP;
  constexpr int NYP = pow2_ceil(NY);
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
  float* gsrow = want_s ? prm.gs + (size_t)e * NP * C + (Q ? li * CPL : li) : nullptr;
  // Accumulating into grad_s: fetch the edge's rows up front, in one batch,
  // rather than one dependent load per path before its store.
  float gs_prev[GEN ? NP : 1][CPL];
  const bool acc_s = GEN && want_s && (prm.flags & kAccumulateS);
  if constexpr (GEN) {
    if (acc_s) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if constexpr (Q) {
          load_ch<float, CPL, true>(gsrow + p * C, gs_prev[p]);
        } else {
#pragma unroll
          for (int c = 0; c < CPL; ++c) gs_prev[p][c] = __builtin_nontemporal_load(gsrow + p * C + c * LPG);
        }
      }
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
    if (want_s) {
      if constexpr (GEN) {
        if (acc_s) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) ds[c] += gs_prev[p][c];
        }
      }
      if constexpr (Q) {
        store_row<CPL>(gsrow + p * C, ds, 1.0f);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) __builtin_nontemporal_store(ds[c], gsrow + p * C + c * LPG);
      }
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
    after(pc);
  });

  if (want_x) {
    if constexpr (Q) {
      atomic_add_rows<C, NX, CPL, LPG>(prm.gx + (size_t)a * NX * C, dxp, xt, li);
    } else {
#pragma unroll
      for (int i = 0; i < NX; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          unsafeAtomicAdd(prm.gx + ((size_t)a * NX + i) * C + li + c * LPG, dxp[i][c]);
    }
  }
  if (!want_y) return;
  store_dy<NY, LPG>(dyp, prm.gy + (size_t)e * NY, li, GEN && (prm.flags & kAccumulateY));
}

template <class LY, int CPL, int GPR, bool GEN = false, int WPB = 4>
__global__ void __launch_bounds__(64 * WPB) conv_bwd_pipe(BwdParams prm) {
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
  const int bl = logical_wave<WPB>() * RPW + slot;
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

// ------------------------------------------------- edge-tiled backward ------
//
// The reverse pass sums nothing at the receivers (every output is per edge, or
// per sender through grad_x), so it need not walk receivers: the edges are cut
// into tiles of about T consecutive edges in storage order, one per wave.  The
// waves resident at one time then sweep a narrow, advancing window of the s
// and grad_s rows (the largest streams), which the memory system serves faster
// than one separate stream per receiver (measured on MI355X: this order beats
// the receiver-locality order even though its sender rows then miss L2).  A
// wave holds 64/LPG groups, each on its own edge (tile edges grp, grp + G,
// ...); a lane holds CPL consecutive channels, so s and grad_s move in 16-byte
// accesses, and the grad_x partials are re-laid through LDS so that each atomic
// instruction covers consecutive channels.  Each group tracks the receiver of
// its edge (found once by a wave-parallel search of row_ptr, then advanced edge
// by edge) and reloads the cotangent row g[b]/N when it changes.

// Largest b in [0, num_nodes) with row_ptr[b] <= e (the receiver of edge e when
// e < row_ptr[num_nodes] = num_edges), by 64 probes per round.  The first
// round probes the 64 receivers around e * num_nodes / num_edges (where the
// answer lies when degrees do not drift far from their mean); otherwise the
// search narrows [0, num_nodes) by 64x per round.
__device__ __forceinline__ int find_receiver(const int* __restrict__ row_ptr, int num_nodes,
                                             int num_edges, int e) {
  const int lane = threadIdx.x & 63;
  long lo = 0, hi = num_nodes;
  {
    long g0 = (long)e * num_nodes / num_edges - 31;
    g0 = g0 < 0 ? 0 : (g0 + 64 > num_nodes ? (num_nodes > 64 ? num_nodes - 64 : 0) : g0);
    const long k = g0 + lane;
    const bool le = k < num_nodes && row_ptr[k < num_nodes ? k : 0] <= e;
    const unsigned long long m = __ballot(le);
    const int cnt = __popcll(m);
    // the guess brackets e when probe g0 is <= e and the probe after the last
    // true one (if inside the window) is > e
    // (the probes <= e are a prefix of the lanes: row_ptr is non-decreasing)
    if ((m & 1ull) && (cnt < 64 || g0 + 64 >= num_nodes)) {
      lo = g0 + cnt - 1;          // the next receiver starts after e, or there is none
      hi = lo + 1;
    } else if (m & 1ull) {
      lo = g0 + 63;               // all 64 probes <= e: the answer lies above
    } else {
      hi = g0;                    // row_ptr[g0] > e (so g0 > 0): the answer lies below
    }
  }
  while (hi - lo > 1) {
    const long step = (hi - lo + 63) / 64;
    const long k = lo + (long)lane * step;
    const bool le = k < hi && row_ptr[k < hi ? k : lo] <= e;
    const int cnt = __popcll(__ballot(le));
    lo += (long)(cnt - 1) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return __builtin_amdgcn_readfirstlane((int)lo);
}


// One tile: the edges [e0, e1).
template <class LY, int CPL, bool GEN, bool SY = false, bool SS = false>
__device__ __forceinline__ void bwd_tile(const BwdParams& prm, long e0, int e1, float* xt, int li,
                                         int grp) {
  constexpr int C = LY::C, NX = LY::NX, NO = LY::NO;
  constexpr int LPG = C / CPL;
  constexpr int G = 64 / LPG;
  // edges of padding receivers (b >= num_real) carry no gradient
  const int e_real = prm.num_real < prm.num_nodes ? prm.row_ptr[prm.num_real] : prm.num_edges;
  const int e_lim = e1 < e_real ? e1 : e_real;

  if ((int)e0 < e_lim) {
    int e = (int)e0 + grp;
    BwdBuf<LY, CPL> b0, b1;
    {
      // the first edge's y and s rows do not depend on the receiver search:
      // in flight while it runs (measured on MI355X: -0.7 % on the training
      // graph)
      const int ef = e < e_lim - 1 ? e : e_lim - 1;
      load_row<float, LY::NY>(prm.y + (size_t)ef * LY::NY, b0.y);
      const float* sf = prm.s + (size_t)ef * LY::NP * C + li * CPL;
#pragma unroll
      for (int p = 0; p < LY::NP; ++p) load_ch<float, CPL, true>(sf + p * C, b0.s[p]);
    }
    int b = find_receiver(prm.row_ptr, prm.num_nodes, prm.num_edges, (int)e0);
    while (prm.row_ptr[b + 1] <= (e < e_lim ? e : e_lim - 1)) ++b;   // this group's first edge
    int bend = prm.row_ptr[b + 1];
    float gv[NO][CPL];
    auto load_g = [&]() {
      const float* grow = prm.g + (size_t)b * NO * C + li * CPL;
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        load_ch<float, CPL, false>(grow + o * C, gv[o]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) gv[o][c] *= prm.inv_avg;
      }
    };
    load_g();
    const int last = e_lim - 1;
    // y and x rows: two buffers (the next edge's load while this one is used);
    // s rows: one buffer, s[p] replaced by the next edge's row as soon as path
    // p is done with it, which keeps a whole edge of s in flight at the cost
    // of one row of registers.
    int a = prm.src[e < last ? e : last];
#pragma unroll
    for (int i = 0; i < NX; ++i)
      load_ch<float, CPL, false>(prm.x + ((size_t)a * NX + i) * C + li * CPL, b0.x[i]);
    int en = e + G;
    int an = prm.src[en < last ? en : last];
    auto step = [&](BwdBuf<LY, CPL>& cur, BwdBuf<LY, CPL>& nxt) {
      // the next edge's rows (and the sender two edges ahead) are loaded
      // unconditionally, clamped to the tile's last edge
      const int en2 = en + G;
      int an2;
      if constexpr (SS) {
        // both groups' senders two edges ahead through the scalar cache
        static_assert(G == 2, "two groups per wave");
        typedef const __attribute__((address_space(4))) int cint;
        cint* sp = (cint*)(uintptr_t)prm.src;
        const int e0n2 = __builtin_amdgcn_readfirstlane(en2 - grp);
        const int sa = sp[e0n2 < last ? e0n2 : last];
        const int sb = sp[e0n2 + 1 < last ? e0n2 + 1 : last];
        an2 = grp ? sb : sa;
      } else {
        an2 = prm.src[en2 < last ? en2 : last];
      }
      const int ec = en < last ? en : last;
      // SY: the two groups' next y rows through the scalar cache (two scalar
      // loads instead of four vector loads per group), each group taking its
      // own at the end of the step
      float ya[SY ? LY::NY : 1], yb[SY ? LY::NY : 1];
      if constexpr (SY) {
        static_assert(G == 2, "two groups per wave");
        const int e0n = __builtin_amdgcn_readfirstlane(en - grp);
        load_row_uniform<LY::NY>(prm.y + (size_t)(e0n < last ? e0n : last) * LY::NY, ya);
        load_row_uniform<LY::NY>(prm.y + (size_t)(e0n + 1 < last ? e0n + 1 : last) * LY::NY, yb);
      } else {
        load_row<float, LY::NY>(prm.y + (size_t)ec * LY::NY, nxt.y);
      }
#pragma unroll
      for (int i = 0; i < NX; ++i)
        load_ch<float, CPL, false>(prm.x + ((size_t)an * NX + i) * C + li * CPL, nxt.x[i]);
      const float* snext = prm.s + (size_t)ec * LY::NP * C + li * CPL;
      auto reload = [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        load_ch<float, CPL, true>(snext + p * C, cur.s[p]);
      };
      if (e <= last) {
        if (e >= bend) {
          do { ++b; } while (prm.row_ptr[b + 1] <= e);
          bend = prm.row_ptr[b + 1];
          load_g();
        }
        bwd_edge<LY, CPL, LPG, GEN, true>(cur, gv, prm, e, a, li, xt, reload);
      } else {
        sfor<0, LY::NP>(reload);
      }
#pragma unroll
      for (int p = 0; p < LY::NP; ++p)
#pragma unroll
        for (int c = 0; c < CPL; ++c) nxt.s[p][c] = cur.s[p][c];
      if constexpr (SY) {
#pragma unroll
        for (int j = 0; j < LY::NY; ++j) nxt.y[j] = grp ? yb[j] : ya[j];
      }
      e = en;
      a = an;
      en = en2;
      an = an2;
    };
    // wave-uniform trip count: steps of G edges until the tile is done
    for (int k0 = (int)e0; k0 <= last; k0 += 2 * G) {
      step(b0, b1);
      if (k0 + G > last) break;
      step(b1, b0);
    }
  }
  // padding edges of this tile
  if (e_lim < e1) {
    const int z0 = e_lim > (int)e0 ? e_lim : (int)e0;
    zero_edge_grads<LY>(prm, z0 + grp, e1, G, li, LPG);
  }
}

// The edges are cut into prm.tiles ranges of nearly equal length (differing by
// at most one edge); wave w runs range w.
template <class LY, int CPL, bool GEN = false, int WPB = 4, bool SY = false, bool SS = false>
__global__ void __launch_bounds__(64 * WPB) conv_bwd_tile(BwdParams prm) {
  constexpr int C = LY::C, NX = LY::NX;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  __shared__ float xt_all[WPB][G][NX * C];

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const long w = logical_wave<WPB>();
  if (w >= prm.tiles) return;
  const long e0 = w * prm.num_edges / prm.tiles;
  const int e1 = (int)((w + 1) * prm.num_edges / prm.tiles);
  if (e0 >= e1) return;
  bwd_tile<LY, CPL, GEN, SY, SS>(prm, e0, e1, xt_all[WPB > 1 ? threadIdx.x >> 6 : 0][grp], li, grp);
}

// ------------------------------------------------ pair-stored backward ------
//
// On a graph that holds b -> a whenever it holds a -> b, with edge features
// y_ba = P y_ab (P: (-1)^l on each l block) and scalars s_ba = s_ab (the
// assumptions of the e3j Convolution page's note on SENDER ordering), one row
// of y and s per undirected pair suffices: a stored edge e = (a -> b) stands
// for itself and for its reverse (b -> a), whose per-path matrix is
// (-1)^l2 K^p(y[e]).  One pass over the stored edges takes both directions,
// reading s[e] and writing grad_s[e] once for the two (per path and channel,
// with w = K^T g[b] / N, w' = (-1)^l2 K^T g[a] / N):
//   grad_s[e] = <x[a], w> + <x[b], w'>
//   grad_x[a] += s w,      grad_x[b] += s w'
//   grad_y[e] = dy(a -> b) + P dy(b -> a)
// The stored edges come grouped by b (runs of equal dst), so a group keeps
// g[b], x[b] and the grad_x[b] sum of its run on chip and adds that sum with
// one set of atomics when the run ends; g[a] and x[a] are gathered per edge
// and grad_x[a] takes atomics per edge, as in the directed pass.  Any order of
// the stored edges gives the same result up to the fp32 summation order;
// grouping saves atomics, and an order in which nearby receivers follow each
// other keeps the gathered rows in L2 (measured on MI355X: it removes about
// 40 % of the gather traffic of the training graph).  Tiles of consecutive
// stored edges, one per wave, as in the edge-tiled pass; a lane holds CPL
// consecutive channels.
//
// Registers (two waves per SIMD need at most 256 per lane): g[b] / N of the
// current run is kept in LDS, in the lane's own slots, and read path by path;
// the paths are visited by output block, so the rows of g[a] that one block
// uses are replaced by the next edge's as soon as that block's paths are done
// (one buffer of g[a] in flight rather than two), as s is replaced path by
// path.  1/N is folded into g[b] and x[b] (and the grad_x[b] sum scaled by 1/N
// when added), so the gathered g[a] needs no scaling.  With one group per wave
// the edge's y row is wave-uniform and read through the scalar cache.

// The j-th path in order of output block (then path index).
constexpr int path_by_out(const LayoutTables& t, int j) {
  for (int p = 0; p < t.num_paths; ++p) {
    int r = 0;
    for (int q = 0; q < t.num_paths; ++q)
      if (t.path[q].o3 < t.path[p].o3 || (t.path[q].o3 == t.path[p].o3 && q < p)) ++r;
    if (r == j) return p;
  }
  return -1;
}

// True if no later path in that order writes the same output block.
constexpr bool last_into_block(const LayoutTables& t, int j) {
  return j + 1 >= t.num_paths || t.path[path_by_out(t, j + 1)].o3 != t.path[path_by_out(t, j)].o3;
}


template <class LY, int CPL>
struct PairBuf {
  float y[LY::NY];
  float xa[LY::NX][CPL];
};

template <class LY, int CPL>
struct PairRun {
  float xb[LY::NX][CPL];     // x[b] / N
  float dxb[LY::NX][CPL];    // N times this group's part of grad_x[b] over the run so far
};

template <class LY, int CPL, int LPG, class After>
__device__ __forceinline__ void bwd_pair_edge(const PairBuf<LY, CPL>& buf,
                                              const float (&ga)[LY::NO][CPL],
                                              const float (&s)[LY::NP][CPL], PairRun<LY, CPL>& run,
                                              const float* gbs, const BwdParams& prm, int e, int a,
                                              int li, float* xt, After after) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP;
  constexpr int NYP = pow2_ceil(NY);
  float dxa[NX][CPL];
#pragma unroll
  for (int i = 0; i < NX; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) dxa[i][c] = 0.0f;
  float dyp[NYP];
#pragma unroll
  for (int j = 0; j < NYP; ++j) dyp[j] = 0.0f;
  float* gsrow = prm.gs + (size_t)e * NP * C + li * CPL;

  sfor<0, NP>([&](auto jc) {
    constexpr int p = path_by_out(LY::T, decltype(jc)::value);
    constexpr PathInfo P = LY::T.path[p];
    constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
    constexpr float sg = (P.l2 & 1) ? -1.0f : 1.0f;   // the reverse edge's K is sg K
    float K[D3][D1];
    build_k<LY, p, D3, D1>(buf.y, K);
    float gb[D3][CPL];                                // this path's rows of g[b] / N
#pragma unroll
    for (int m3 = 0; m3 < D3; ++m3) lds_load_ch<CPL>(gbs + (P.o3 + m3) * C, gb[m3]);
    float ds[CPL];
    sfor<0, D1>([&](auto m1c) {
      constexpr int m1 = decltype(m1c)::value;
      float w1[CPL], w2[CPL];
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            if constexpr (first_m3(LY::T, p, m1) == m3) {
              w1[c] = K[m3][m1] * gb[m3][c];
              w2[c] = K[m3][m1] * ga[P.o3 + m3][c];
            } else {
              w1[c] = __builtin_fmaf(K[m3][m1], gb[m3][c], w1[c]);
              w2[c] = __builtin_fmaf(K[m3][m1], ga[P.o3 + m3][c], w2[c]);
            }
          }
        }
      });
      if constexpr (first_m3(LY::T, p, m1) >= 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if constexpr (m1 == 0) {
            ds[c] = buf.xa[P.o1][c] * w1[c];
          } else {
            ds[c] = __builtin_fmaf(buf.xa[P.o1 + m1][c], w1[c], ds[c]);
          }
          ds[c] = __builtin_fmaf(sg * run.xb[P.o1 + m1][c], w2[c], ds[c]);
          dxa[P.o1 + m1][c] = __builtin_fmaf(s[p][c], w1[c], dxa[P.o1 + m1][c]);
          run.dxb[P.o1 + m1][c] = __builtin_fmaf(sg * s[p][c], w2[c], run.dxb[P.o1 + m1][c]);
        }
      } else if constexpr (m1 == 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) ds[c] = 0.0f;
      }
    });
    store_row<CPL>(gsrow + p * C, ds, 1.0f);

    // grad_y[o2+m2] += sum_{m1,m3} C[m1,m2,m3] sum_c s (x[a] g[b] + sg x[b] g[a]) / N
    sfor<0, D1>([&](auto m1c) {
      constexpr int m1 = decltype(m1c)::value;
      if constexpr (first_m3(LY::T, p, m1) >= 0) {
        float u1[CPL], u2[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          u1[c] = s[p][c] * buf.xa[P.o1 + m1][c];
          u2[c] = sg * s[p][c] * run.xb[P.o1 + m1][c];
        }
        sfor<0, D3>([&](auto m3c) {
          constexpr int m3 = decltype(m3c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
            float q = u1[0] * gb[m3][0];
            q = __builtin_fmaf(u2[0], ga[P.o3 + m3][0], q);
#pragma unroll
            for (int c = 1; c < CPL; ++c) {
              q = __builtin_fmaf(u1[c], gb[m3][c], q);
              q = __builtin_fmaf(u2[c], ga[P.o3 + m3][c], q);
            }
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
    after(jc);
  });

  atomic_add_rows<C, NX, CPL, LPG>(prm.gx + (size_t)a * NX * C, dxa, xt, li);
  store_dy<NY, LPG>(dyp, prm.gy + (size_t)e * NY, li, false);
}

// One tile: the stored edges [e0, e1); group grp takes e0 + grp, e0 + grp + G, ...
template <class LY, int CPL>
__device__ __forceinline__ void bwd_pair_tile(const BwdParams& prm, int e0, int e1, float* xt,
                                              float* gbs, int li, int grp) {
  constexpr int C = LY::C, NX = LY::NX, NO = LY::NO, NP = LY::NP;
  constexpr int LPG = C / CPL;
  constexpr int G = 64 / LPG;
  const int last = e1 - 1;
  const float inv = prm.inv_avg;
  const int* __restrict__ dst = prm.dst;

  PairRun<LY, CPL> run;
  int b = -1;                               // node of the current run (none yet)
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < NX; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) run.dxb[i][c] *= inv;
    atomic_add_rows<C, NX, CPL, LPG>(prm.gx + (size_t)b * NX * C, run.dxb, xt, li);
  };
  auto start_run = [&](int nb) {
    b = nb;
    const float* grow = prm.g + (size_t)b * NO * C + li * CPL;
    const float* xrow = prm.x + (size_t)b * NX * C + li * CPL;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      float v[CPL];
      load_ch<float, CPL, false>(grow + o * C, v);
      lds_store_ch<CPL>(gbs + o * C, v, inv);
    }
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      load_ch<float, CPL, false>(xrow + i * C, run.xb[i]);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        run.xb[i][c] *= inv;
        run.dxb[i][c] = 0.0f;
      }
    }
  };
  auto load_edge = [&](PairBuf<LY, CPL>& nb, int ec, int a) {
    if constexpr (G == 1) {
      load_row_uniform<LY::NY>(prm.y + (size_t)ec * LY::NY, nb.y);
    } else {
      load_row<float, LY::NY>(prm.y + (size_t)ec * LY::NY, nb.y);
    }
    const float* xrow = prm.x + (size_t)a * NX * C + li * CPL;
#pragma unroll
    for (int i = 0; i < NX; ++i) load_ch<float, CPL, false>(xrow + i * C, nb.xa[i]);
  };

  // s and g[a]: one buffer each, refilled with the next edge's rows as the
  // paths finish with them; y and x[a]: two buffers.
  float s[NP][CPL], ga[NO][CPL];
  PairBuf<LY, CPL> b0, b1;
  int e = e0 + grp;
  int ec = e < last ? e : last;
  int a = prm.src[ec];
  int bc = dst[ec];
  load_edge(b0, ec, a);
  {
    const float* srow = prm.s + (size_t)ec * NP * C + li * CPL;
    const float* grow = prm.g + (size_t)a * NO * C + li * CPL;
#pragma unroll
    for (int p = 0; p < NP; ++p) load_ch<float, CPL, true>(srow + p * C, s[p]);
#pragma unroll
    for (int o = 0; o < NO; ++o) load_ch<float, CPL, false>(grow + o * C, ga[o]);
  }
  int en = e + G;
  int an = prm.src[en < last ? en : last];
  int bn = dst[en < last ? en : last];
  auto step = [&](PairBuf<LY, CPL>& cur, PairBuf<LY, CPL>& nxt) {
    // the next edge's rows (and the indices two edges ahead) are loaded
    // unconditionally, clamped to the tile's last edge
    const int en2 = en + G;
    const int ec2 = en2 < last ? en2 : last;
    const int an2 = prm.src[ec2];
    const int bn2 = dst[ec2];
    const int ecn = en < last ? en : last;
    load_edge(nxt, ecn, an);
    const float* snext = prm.s + (size_t)ecn * NP * C + li * CPL;
    const float* gnext = prm.g + (size_t)an * NO * C + li * CPL;
    auto reload = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int p = path_by_out(LY::T, j);
      load_ch<float, CPL, true>(snext + p * C, s[p]);
      if constexpr (last_into_block(LY::T, j)) {
        constexpr PathInfo P = LY::T.path[p];
#pragma unroll
        for (int m3 = 0; m3 < 2 * P.l3 + 1; ++m3)
          load_ch<float, CPL, false>(gnext + (P.o3 + m3) * C, ga[P.o3 + m3]);
      }
    };
    if (e <= last) {
      if (bc != b) {
        if (b >= 0) flush();
        start_run(bc);
      }
      bwd_pair_edge<LY, CPL, LPG>(cur, ga, s, run, gbs, prm, e, a, li, xt, reload);
    } else {
      sfor<0, NP>(reload);
    }
    e = en;
    a = an;
    bc = bn;
    en = en2;
    an = an2;
    bn = bn2;
  };
  // wave-uniform trip count: steps of G edges until the tile is done
  for (int k0 = e0; k0 <= last; k0 += 2 * G) {
    step(b0, b1);
    if (k0 + G > last) break;
    step(b1, b0);
  }
  if (b >= 0) flush();
}

// The stored edges are cut into prm.tiles ranges of nearly equal length; wave
// w runs range w.
template <class LY, int CPL, int WPB = 4>
__global__ void __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(2)))
conv_bwd_pairs(BwdParams prm) {
  constexpr int C = LY::C, NX = LY::NX;
  constexpr int LPG = C / CPL;
  static_assert(C % CPL == 0 && 64 % LPG == 0, "a group must tile a wave");
  constexpr int G = 64 / LPG;
  __shared__ float xt_all[WPB][G][NX * C];
  __shared__ float gb_all[WPB][G][LY::NO * C];

  const int lane = threadIdx.x & 63;
  const int li = lane % LPG;
  const int grp = lane / LPG;
  const long w = logical_wave<WPB>();
  if (w >= prm.tiles) return;
  const int e0 = (int)(w * prm.num_edges / prm.tiles);
  const int e1 = (int)((w + 1) * prm.num_edges / prm.tiles);
  if (e0 >= e1) return;
  bwd_pair_tile<LY, CPL>(prm, e0, e1, xt_all[WPB > 1 ? threadIdx.x >> 6 : 0][grp],
                         gb_all[WPB > 1 ? threadIdx.x >> 6 : 0][grp] + li * CPL, li, grp);
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

// LIN: the output linear fused into the epilogue (p.lin_w, p.lin_alpha).
// PR: y and s read from pair-stored rows through p.emap.
template <class LY, typename IN, int CPL, int GPR, bool UL = false, bool LIN = false, bool PR = false,
          int WPB = 4>
hipError_t launch_fwd_pipe(const FwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  static_assert(WPB == 4 || !LIN, "the fused linear runs work-groups of four waves");
  if (p.num_nodes <= 0) return hipSuccess;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + WPB - 1) / WPB + 7) / 8 * 8;
  // the fused linear's work-groups loop over receivers: at most 1024 of them,
  // each staging the weights once
  const long grid = LIN && blocks > 1024 ? 1024 : blocks;
  hipLaunchKernelGGL((conv_fwd_pipe<LY, IN, CPL, GPR, UL, LIN, PR, WPB>), dim3((unsigned)grid), dim3(64 * WPB),
                     0, st, p);
  return hipGetLastError();
}

template <class LY, int CPL, int GPR>
hipError_t launch_bwd(const BwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  hipError_t err = launch_fill_zero(p.gx, (size_t)p.num_nodes * LY::NX * LY::C, st);
  if (err != hipSuccess) return err;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + 3) / 4 + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_bwd<LY, CPL, GPR>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <class LY, int CPL, int GPR, bool GEN = false, int WPB = 4>
hipError_t launch_bwd_pipe(const BwdParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  if (p.gx && !(p.flags & kAccumulateX)) {
    const hipError_t err = launch_fill_zero(p.gx, (size_t)p.num_nodes * LY::NX * LY::C, st);
    if (err != hipSuccess) return err;
  }
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + WPB - 1) / WPB + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_bwd_pipe<LY, CPL, GPR, GEN, WPB>), dim3((unsigned)blocks), dim3(64 * WPB), 0, st, p);
  return hipGetLastError();
}

// One wave per tile of about T edges.
template <class LY, int CPL, int T, bool GEN = false, int WPB = 4, bool SY = false, bool SS = false>
hipError_t launch_bwd_tile(const BwdParams& prm, hipStream_t st) {
  BwdParams p = prm;
  if (p.num_nodes <= 0) return hipSuccess;
  if (p.gx && !(p.flags & kAccumulateX)) {
    const hipError_t err = launch_fill_zero(p.gx, (size_t)p.num_nodes * LY::NX * LY::C, st);
    if (err != hipSuccess) return err;
  }
  if (p.num_edges <= 0) return hipSuccess;
  const auto kernel = conv_bwd_tile<LY, CPL, GEN, WPB, SY, SS>;
  const long tiles = ((long)p.num_edges + T - 1) / T;
  p.tiles = (int)tiles;
  const long blocks = ((tiles + WPB - 1) / WPB + 7) / 8 * 8;   // whole rounds of the 8 XCDs (logical_wave)
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * WPB), 0, st, p);
  return hipGetLastError();
}

// Pair-stored reverse pass: grad_x zeroed, then one wave per tile of about T
// stored edges (prm.num_edges of them, prm.dst their receivers).
template <class LY, int CPL, int T, int WPB = 4>
hipError_t launch_bwd_pairs(const BwdParams& prm, hipStream_t st) {
  BwdParams p = prm;
  if (p.num_nodes <= 0) return hipSuccess;
  const hipError_t err = launch_fill_zero(p.gx, (size_t)p.num_nodes * LY::NX * LY::C, st);
  if (err != hipSuccess) return err;
  if (p.num_edges <= 0) return hipSuccess;
  const long tiles = ((long)p.num_edges + T - 1) / T;
  p.tiles = (int)tiles;
  const long blocks = ((tiles + WPB - 1) / WPB + 7) / 8 * 8;   // whole rounds of the 8 XCDs (logical_wave)
  hipLaunchKernelGGL((conv_bwd_pairs<LY, CPL, WPB>), dim3((unsigned)blocks), dim3(64 * WPB), 0, st, p);
  return hipGetLastError();
}

template <class LY, typename IN, int CPL, int GPR, bool PX, int WPB = 4>
hipError_t launch_jvp_pipe(const JvpParams& p, hipStream_t st) {
  constexpr int RPW = (64 / (LY::C / CPL)) / GPR;
  if (p.num_nodes <= 0) return hipSuccess;
  const long waves = (p.num_nodes + RPW - 1) / RPW;
  const long blocks = ((waves + WPB - 1) / WPB + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_jvp_pipe<LY, IN, CPL, GPR, PX, WPB>), dim3((unsigned)blocks), dim3(64 * WPB), 0, st, p);
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
