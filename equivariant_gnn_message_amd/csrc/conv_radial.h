// Convolution with the edge scalars computed in the kernel from the edge
// lengths (gate-points page: radial embedding of the edge length, then a
// fully connected network whose outputs weight the convolution's paths and
// channels), for layouts of 32 channels, fp32.
//
//   f_k(r) = exp(-((r - mu_k) / sigma)^2) (1 + cos(pi r / r_max)) / 2 (0 for r >= r_max),
//   s[e]   = silu(f(r_e) W1) W2   -> (NP, C),
//   out[b] = (1/N) sum_{e=(a->b)} (x[a] (x) y[e]) (.) s[e].
//
// The scalars never reach memory: the (E, NP, C) tensor that would otherwise
// be written by the network and read back by the convolution is formed per
// edge in registers.
//
// Per tile of 16 edges (one wave): four quads, each up to four consecutive
// edges of one receiver (quads of different receivers can share a tile):
// * lane (m, q) = (lane % 16, lane / 16) evaluates the basis for edge m of the
//   tile (slot m % 4 of quad m / 4) and the hidden units u = 32 j + 4 i + q
//   (i < 8) of contraction step j, which is the A operand of
//   v_mfma_f32_16x16x32_f16 (A[m][8 q + i]);
// * s (16 edges x NP*C) = h W2 is accumulated over hidden/32 steps in NP*C/16
//   accumulator tiles, from two-part fp16 operands (fp32-level accuracy, see
//   the kernel); W2 is staged once per work-group in LDS;
// * the accumulator layout hands lane (g, n) = (lane / 16, lane % 16) the
//   scalars of edges 4g .. 4g+3 of the tile, i.e. quad g, for channels n and
//   n + 16 of every path (column p*C + c lies in tile 2p + c/16), so each lane
//   runs the tensor product and mixing of its quad for those two channels;
// * the four groups' partial sums are combined per receiver by a segmented
//   scan across the groups and added to the receiver's row in LDS; a row is
//   written once, when the receiver's last quad has been added (by the wave
//   holding its first quad when neighbouring waves share the receiver).
#pragma once

#include "conv_kernels.h"

namespace e3c {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kRadialWaves = 8;          // waves per work-group (one W2 copy in LDS)
constexpr int kRadialMaxHidden = 128;
constexpr int kRadialMaxBasis = 8;

template <class LY>
struct RadialShape {
  static constexpr int C = LY::C, NP = LY::NP;
  static constexpr int NT = NP * C / 16;   // accumulator tiles of 16 columns
  static_assert(C == 32, "radial kernel: 32 channels (two per lane)");
  static_assert(NT <= 16 && NT % 4 == 0, "radial kernel: at most 8 paths, an even number");
};

// First b in [0, n] with row_ptr[b] + 8 b >= v (requires v <= row_ptr[n] + 8 n),
// searched by the whole wave: each round reads 64 samples of the range and
// keeps the interval between the last sample below v and the first at or above
// it, so a range of n shrinks to one entry in about log64(n) + 1 dependent loads.
__device__ __forceinline__ int radial_lower_bound(const int* row_ptr, int n, long v, int lane) {
  int lo = 0, hi = n;   // the answer lies in [lo, hi]; hi always satisfies the condition
  while (hi - lo >= 64) {
    const int step = (hi - lo + 63) >> 6;
    const long cand = lo + (long)(lane + 1) * step;
    const int idx = cand < hi ? (int)cand : hi;   // lane 63 samples hi
    const unsigned long long m = __ballot((long)row_ptr[idx] + 8L * idx >= v);
    const int k = (int)__builtin_ctzll(m);
    const int nhi = __builtin_amdgcn_readlane(idx, k);
    const int nlo = k == 0 ? lo : __builtin_amdgcn_readlane(idx, k - 1) + 1;
    lo = nlo;
    hi = nhi;
  }
  const int idx = lo + lane;
  const unsigned long long m = __ballot(idx <= hi && (long)row_ptr[idx] + 8L * idx >= v);
  return lo + (int)__builtin_ctzll(m);
}

// The tensor product and mixing of one edge for a lane's two channels, with
// the scalars sv[p][ch] already in registers (same contraction forms as
// edge_accumulate).
template <class LY>
__device__ __forceinline__ void radial_edge(const float (&yv)[LY::NY], const float (&xv)[LY::NX][2],
                                            const float (&sv)[LY::NP][2], float (&acc)[LY::NO][2]) {
  constexpr int NP = LY::NP;
  sfor<0, NP>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    constexpr PathInfo P = LY::T.path[p];
    constexpr int D1 = 2 * P.l1 + 1, D3 = 2 * P.l3 + 1;
    float K[D3][D1];
    build_k<LY, p, D3, D1>(yv, K);
    if constexpr (D1 <= D3) {
      float u[D1][2];
      sfor<0, D1>([&](auto m1c) {
        constexpr int m1 = decltype(m1c)::value;
        if constexpr (first_m3(LY::T, p, m1) >= 0) {
#pragma unroll
          for (int c = 0; c < 2; ++c) u[m1][c] = sv[p][c] * xv[P.o1 + m1][c];
        }
      });
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[P.o3 + m3][c] = __builtin_fmaf(K[m3][m1], u[m1][c], acc[P.o3 + m3][c]);
          }
        });
      });
    } else {
      sfor<0, D3>([&](auto m3c) {
        constexpr int m3 = decltype(m3c)::value;
        float tv[2];
        sfor<0, D1>([&](auto m1c) {
          constexpr int m1 = decltype(m1c)::value;
          if constexpr (k_nonzero(LY::T, p, m3, m1)) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              if constexpr (first_m1(LY::T, p, m3) == m1) {
                tv[c] = K[m3][m1] * xv[P.o1 + m1][c];
              } else {
                tv[c] = __builtin_fmaf(K[m3][m1], xv[P.o1 + m1][c], tv[c]);
              }
            }
          }
        });
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[P.o3 + m3][c] = __builtin_fmaf(sv[p][c], tv[c], acc[P.o3 + m3][c]);
      });
    }
  });
}

// The rows one lane needs for one edge: y and its two channels of x[src].
template <class LY>
struct RadialRows {
  f32x4 y[LY::NY / 4];
  float x[LY::NX][2];
};

template <class LY>
__device__ __forceinline__ void radial_load(RadialRows<LY>& R, const RadialParams& prm, int e, int a, int n) {
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY;
  static_assert(NY % 4 == 0, "y rows load as float4");
  const f32x4* yr = reinterpret_cast<const f32x4*>(prm.y + (size_t)e * NY);
#pragma unroll
  for (int i = 0; i < NY / 4; ++i) R.y[i] = yr[i];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    R.x[i][0] = prm.x[((size_t)a * NX + i) * C + n];
    R.x[i][1] = prm.x[((size_t)a * NX + i) * C + n + 16];
  }
}

template <class LY>
__global__ void __launch_bounds__(64 * kRadialWaves) conv_fwd_radial(RadialParams prm) {
  using SH = RadialShape<LY>;
  constexpr int C = LY::C, NY = LY::NY, NO = LY::NO, NP = LY::NP, NT = SH::NT;
  // The second layer (hidden -> NP * C) runs on the fp16 matrix instruction
  // with each operand split into two fp16 parts, v = hi + lo with
  // |v - hi - lo| <= 2^-22 |v|, and three products per term (hi hi + hi lo +
  // lo hi; the dropped lo lo is below 2^-22 of the term), accumulated in fp32:
  // fp32-level accuracy at a small fraction of the fp32 matrix instruction's
  // cycles.  Powers of two keep both operands inside the fp16 range: hidden
  // unit u is scaled by 2^-g_u, with sum_b |W1[b, u]| (a bound of |silu(z_u)|,
  // since 0 <= f_b <= 1) in [2^(13 + g_u), 2^(14 + g_u)); W2 row u by 2^g_u;
  // the columns of channel c (one per path) by 2^-e_c so that their largest
  // entry lies in [2^13, 2^14).  Channels do not mix in the convolution, so
  // 2^e_c is applied once, to the output row.
  //
  // Hidden unit u = 32 j + 4 i + q is element i of lane group q's A operand in
  // contraction step j, so the real units of the last step fill the lowest i;
  // W2 is staged as [j][t][hi, lo][q][n][i] (fp16): the B operand of tile t is
  // 16 contiguous bytes per lane.  W1 as [u][b] (b < 8).
  __shared__ __attribute__((aligned(16))) f16x8 w2s[kRadialMaxHidden / 32 * NT * 2 * 64];
  __shared__ __attribute__((aligned(16))) float w1s[kRadialMaxHidden * kRadialMaxBasis];
  __shared__ float hsc[kRadialMaxHidden];    // 2^-g_u
  __shared__ int hexp[kRadialMaxHidden];     // g_u
  __shared__ unsigned chmax[C];              // bits of max_{u,p} |W2[u, p C + c]| 2^g_u (non-negative floats order as integers)
  __shared__ float chsc[C];                  // 2^e_c
  // partial output rows of receivers shared between waves ([wave][slot][NO * C]),
  // which slots are used (bit 0: slot 0, bit 1: slot 1, bit 2: the receiver in
  // slot 0 also continues after the wave), the receiver in slot 1
  __shared__ float part[kRadialWaves * 2 * NO * C];
  __shared__ int part_flags[kRadialWaves];
  __shared__ int part_recv[kRadialWaves];

  constexpr int NPC = NP * C;
  const int H = prm.hidden, NB = prm.num_basis;
  const int S = (H + 31) >> 5;   // contraction steps of 32 hidden units
  const int tid = (int)threadIdx.x;
  // All weight loads are issued before any is used (clamped addresses and
  // selects instead of branches, which would wait for each load in turn).
  if (tid < S * 32) {
    float wv[kRadialMaxBasis];
    const int uc = tid < H ? tid : H - 1;
#pragma unroll
    for (int bb = 0; bb < kRadialMaxBasis; ++bb) wv[bb] = prm.w1[(bb < NB ? bb : NB - 1) * H + uc];
    float beta = 0.0f;
#pragma unroll
    for (int bb = 0; bb < kRadialMaxBasis; ++bb) {
      wv[bb] = bb < NB && tid < H ? wv[bb] : 0.0f;
      beta += fabsf(wv[bb]);
    }
    const int g = beta > 0.0f ? __builtin_amdgcn_frexp_expf(beta) - 14 : 0;
    hexp[tid] = g;
    hsc[tid] = __builtin_amdgcn_ldexpf(1.0f, -g);
#pragma unroll
    for (int bb = 0; bb < kRadialMaxBasis; ++bb) w1s[tid * kRadialMaxBasis + bb] = wv[bb];
  }
  if (tid < C) chmax[tid] = 0u;
  __syncthreads();
  {
    // thread: column c, steps 2 hf and 2 hf + 1 (64 rows); the loads are
    // coalesced across the lanes (consecutive columns)
    const int c = tid & 255, hf = tid >> 8;
    const int cc = c < NPC ? c : NPC - 1;
    float w[64];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int u = 32 * (2 * hf + jj) + 4 * i + q2;
          w[(jj * 4 + q2) * 8 + i] = prm.w2[(size_t)(u < H ? u : H - 1) * NPC + cc];
        }
    float m = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int u = 32 * (2 * hf + jj) + 4 * i + q2;
          float& v = w[(jj * 4 + q2) * 8 + i];
          v = c < NPC && u < H ? __builtin_amdgcn_ldexpf(v, hexp[u]) : 0.0f;
          m = fmaxf(m, fabsf(v));
        }
    if (c < NPC) atomicMax(&chmax[c % C], __float_as_uint(m));
    __syncthreads();
    const float cm = __uint_as_float(chmax[cc % C]);
    const int e = cm > 0.0f ? __builtin_amdgcn_frexp_expf(cm) - 14 : 0;
    if (hf == 0 && c < C) chsc[c] = __builtin_amdgcn_ldexpf(1.0f, e);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int j = 2 * hf + jj;
        if (j < S && c < NPC) {
          f16x8 hi, lo;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = __builtin_amdgcn_ldexpf(w[(jj * 4 + q2) * 8 + i], -e);
            hi[i] = (_Float16)v;
            lo[i] = (_Float16)(v - (float)hi[i]);
          }
          w2s[((j * NT + (c >> 4)) * 2 + 0) * 64 + q2 * 16 + (c & 15)] = hi;
          w2s[((j * NT + (c >> 4)) * 2 + 1) * 64 + q2 * 16 + (c & 15)] = lo;
        }
      }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, n = lane & 15;   // A-operand role (edge n, lane group q); output role (group q, column n)
  const float inv_sigma = 1.0f / prm.sigma;
  const float center_step = prm.r_max / (float)(NB - 1);
  const float half_turns = 0.5f / prm.r_max;   // cos(pi r / r_max) = cos(2 pi (r / (2 r_max)))

  // Work distribution.  The unit of work is a quad: up to four consecutive
  // edges of one receiver (a receiver of d edges has ceil(d / 4) quads), and a
  // tile is four consecutive quads, one per lane group, possibly of different
  // receivers.  Work-group ranges of receivers are cut at equal shares of
  // row_ptr[b] + 8 b in index order (edges plus a margin per receiver), at
  // equal receiver counts when a processing order is given.  Within a
  // work-group the tiles are split evenly over the 8 waves, so a receiver can
  // be shared by neighbouring waves: each wave writes the receivers it holds
  // entirely, keeps the partial rows of its first and last receiver in LDS
  // when they continue in another wave, and after a barrier the wave holding
  // the first part of such a receiver adds the others' parts and writes the
  // row.
  const int N = prm.num_nodes;
  const int nblk = (int)gridDim.x;
  const int blk = (int)(blockIdx.x & 7) * (nblk >> 3) + (int)(blockIdx.x >> 3);   // XCD-contiguous
  const int wid = (int)(threadIdx.x >> 6);
  int B0, B1;
  if (prm.order) {
    const int per = (N + nblk - 1) / nblk;
    B0 = blk * per < N ? blk * per : N;
    B1 = B0 + per < N ? B0 + per : N;
  } else {
    const long total = (long)prm.row_ptr[N] + 8L * N;
    B0 = radial_lower_bound(prm.row_ptr, N, total * blk / nblk, lane);
    B1 = blk == nblk - 1 ? N : radial_lower_bound(prm.row_ptr, N, total * (blk + 1) / nblk, lane);
  }

  // receiver at processing position i: node id and edge range (empty for padding receivers)
  auto recv = [&](int i, int& b, int& beg, int& end) {
    b = prm.order ? prm.order[i] : i;
    beg = prm.row_ptr[b];
    end = b < prm.num_real ? prm.row_ptr[b + 1] : beg;
  };
  auto wave_scan = [&](int v) {   // inclusive prefix sum over the wave's lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(v, d, 64);
      if (lane >= d) v += t;
    }
    return v;
  };
  // quads of the receivers at positions c0 + lane (< B1), their inclusive
  // prefix within the chunk, and the chunk's total
  auto chunk = [&](int c0, int& nu, int& incl) {
    nu = 0;
    if (c0 + lane < B1) {
      int bb, bg, en;
      recv(c0 + lane, bb, bg, en);
      nu = (en - bg + 3) >> 2;
    }
    incl = wave_scan(nu);
    return __builtin_amdgcn_readlane(incl, 63);
  };
  int nu0, incl0;
  int Q = chunk(B0, nu0, incl0);
  for (int c0 = B0 + 64; c0 < B1; c0 += 64) {
    int a, c;
    Q += chunk(c0, a, c);
  }
  // first position i with (quads up to and including i) >= v, for 1 <= v <= Q:
  // the receiver holding quad v - 1; also its inclusive prefix and quad count
  auto locate = [&](int v, int& at, int& a_incl, int& a_nu) {
    unsigned long long m = __ballot(B0 + lane < B1 && incl0 >= v);
    if (m) {
      const int k = (int)__builtin_ctzll(m);
      at = B0 + k;
      a_incl = __builtin_amdgcn_readlane(incl0, k);
      a_nu = __builtin_amdgcn_readlane(nu0, k);
      return;
    }
    int R = __builtin_amdgcn_readlane(incl0, 63);
    for (int c0 = B0 + 64; c0 < B1; c0 += 64) {
      int nu, incl;
      const int tot = chunk(c0, nu, incl);
      m = __ballot(c0 + lane < B1 && R + incl >= v);
      if (m) {
        const int k = (int)__builtin_ctzll(m);
        at = c0 + k;
        a_incl = R + __builtin_amdgcn_readlane(incl, k);
        a_nu = __builtin_amdgcn_readlane(nu, k);
        return;
      }
      R += tot;
    }
    at = B1;
    a_incl = R;
    a_nu = 0;
  };
  // this wave's tiles [ts, te) of the work-group's TT, i.e. quads [us, ue);
  // positions [p_lo, p_hi) it visits (with the receivers without quads that
  // lie between its quads and the previous wave's), P = quads before p_lo
  const int TT = (Q + 3) >> 2;
  const int ts = (int)((long)TT * wid / kRadialWaves), te = (int)((long)TT * (wid + 1) / kRadialWaves);
  const int us = 4 * ts, ue = 4 * te < Q ? 4 * te : Q;
  int p_lo = B0, P = 0;
  if (us > 0) {
    int at, ai, an;
    locate(us, at, ai, an);
    if (ai == us) {
      p_lo = at + 1;
      P = us;
    } else {
      p_lo = at;
      P = ai - an;
    }
  }
  int p_hi;
  if (wid == kRadialWaves - 1) {
    p_hi = B1;
  } else if (ue == us) {
    p_hi = p_lo;
  } else {
    int at, ai, an;
    locate(ue, at, ai, an);
    p_hi = at + 1;
  }

  // Partial rows are accumulated in this wave's two LDS slots: slot 0 for a
  // receiver that began in an earlier wave (only the wave's first can), slot
  // 1 for the others (cleared after each is written out; the last one is kept
  // there when it continues in a later wave).
  float* slot0 = part + (wid * 2) * (NO * C);
  float* slot1 = slot0 + NO * C;
  for (int idx = lane; idx < 2 * NO * C; idx += 64) slot0[idx] = 0.0f;
  if (lane == 0) part_flags[wid] = 0;

  // Window of up to 64 receivers in lanes: lane k holds position wstart + k
  // (< p_hi): node, edge range, quad count and inclusive quad prefix; WU =
  // quads before wstart.  Loading a window writes the zero rows of its
  // receivers without quads.
  int wstart = p_lo, WU = P;
  int w_b = 0, w_beg = 0, w_end = 0, w_incl = 0, w_tot = 0;
  auto load_window = [&]() {
    const int pos = wstart + lane;
    w_b = 0;
    w_beg = 0;
    w_end = 0;
    if (pos < p_hi) recv(pos, w_b, w_beg, w_end);
    w_incl = wave_scan((w_end - w_beg + 3) >> 2);
    w_tot = __builtin_amdgcn_readlane(w_incl, 63);
    unsigned long long zm = __ballot(pos < p_hi && w_end == w_beg);
    while (zm) {
      const int k = (int)__builtin_ctzll(zm);
      zm &= zm - 1;
      float* zrow = prm.out + (size_t)__builtin_amdgcn_readlane(w_b, k) * NO * C;
      for (int idx = lane; idx < NO * C; idx += 64) __builtin_nontemporal_store(0.0f, zrow + idx);
    }
  };
  if (p_lo < p_hi) load_window();

  // Quad U (us <= U < ue): its receiver's node, first edge and edge count, and
  // the receiver's first and last quads (absolute indices in the work-group).
  struct Quad {
    int b, es, c, first, last;
  };
  auto describe = [&](int U) {
    Quad d = {0, 0, 0, 0, 0};
    if (U >= ue) return d;
    unsigned long long m = __ballot(wstart + lane < p_hi && WU + w_incl > U);
    while (!m && wstart + 64 < p_hi) {   // past the window: the next one
      WU += w_tot;
      wstart += 64;
      load_window();
      m = __ballot(wstart + lane < p_hi && WU + w_incl > U);
    }
    if (!m) return d;   // not reached: every quad below ue lies before p_hi
    const int k = (int)__builtin_ctzll(m);
    const int beg = __builtin_amdgcn_readlane(w_beg, k), end = __builtin_amdgcn_readlane(w_end, k);
    const int nu = (end - beg + 3) >> 2;
    d.b = __builtin_amdgcn_readlane(w_b, k);
    d.first = WU + __builtin_amdgcn_readlane(w_incl, k) - nu;
    d.last = d.first + nu - 1;
    d.es = beg + 4 * (U - d.first);
    const int rem = end - d.es;
    d.c = rem < 4 ? rem : 4;
    return d;
  };

  // The edge length and sender index of a lane's A-operand edge (slot m & 3 of
  // the tile's quad m >> 2; the last edge of that quad for empty slots) are
  // fetched one tile ahead, so that neither the network nor the gathers wait
  // for them; the senders of a group's four edges are taken from lanes 4 q + i
  // of its row when needed.
  auto pick_es = [&](const Quad (&qd)[4], int g) {
    return g == 0 ? qd[0].es : g == 1 ? qd[1].es : g == 2 ? qd[2].es : qd[3].es;
  };
  auto pick_c = [&](const Quad (&qd)[4], int g) {
    return g == 0 ? qd[0].c : g == 1 ? qd[1].c : g == 2 ? qd[2].c : qd[3].c;
  };
  auto tile_ids = [&](const Quad (&qd)[4], float& rv, int& sv) {
    const int g = n >> 2, slot = n & 3;
    const int c = pick_c(qd, g);
    if (c > 0) {
      const int e = pick_es(qd, g) + (slot < c ? slot : c - 1);
      rv = prm.r[e];
      sv = prm.src[e];
    } else {
      rv = 0.0f;
      sv = 0;
    }
  };
  auto sender = [&](int sv, int i) { return __shfl(sv, (lane & 48) | (4 * q + i), 64); };

  // Writing out a receiver's partial row held in a slot: the whole row when
  // it lies entirely in this wave, else kept for the fixup after the barrier.
  auto finish = [&](const Quad& rq) {
    const bool open_start = rq.first < us, open_end = rq.last >= ue;
    if (open_start) {   // slot 0: began in an earlier wave
      if (lane == 0) part_flags[wid] |= open_end ? 5 : 1;
    } else if (open_end) {   // slot 1: continues in a later wave
      if (lane == 0) {
        part_flags[wid] |= 2;
        part_recv[wid] = rq.b;
      }
    } else {
      float* orow = prm.out + (size_t)rq.b * NO * C;
      for (int idx = lane; idx < NO * C; idx += 64) {
        __builtin_nontemporal_store(slot1[idx] * (prm.inv_avg * chsc[idx % C]), orow + idx);
        slot1[idx] = 0.0f;
      }
    }
  };

  Quad cur[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) cur[g] = describe(us + g);
  float r_cur = 0.0f;
  int s_cur = 0;
  if (us < ue) tile_ids(cur, r_cur, s_cur);
  Quad run = {-1, 0, 0, 0, 0};   // receiver whose partial row is accumulating
  float* run_slot = slot1;

  for (int t = ts; t < te; ++t) {
    Quad nxt[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) nxt[g] = describe(4 * (t + 1) + g);
    float r_next = 0.0f;
    int s_next = 0;
    if (t + 1 < te) tile_ids(nxt, r_next, s_next);

    // this group's quad: edges es_q .. es_q + c_q - 1
    const int es_q = pick_es(cur, q), c_q = pick_c(cur, q);
    // rows of this lane's first two edges, in flight during the network
    RadialRows<LY> ra, rb;
    const int a0 = sender(s_cur, 0), a1 = sender(s_cur, 1);
    // (unconditional, clamped like the loads of edges 2 and 3 below, and kept
    // ahead of the network by the scheduling barrier)
    radial_load<LY>(ra, prm, c_q > 0 ? es_q : 0, a0, n);
    radial_load<LY>(rb, prm, c_q > 0 ? es_q + (c_q > 1 ? 1 : 0) : 0, a1, n);
    __builtin_amdgcn_sched_barrier(0);

    float acc[NO][2];
#pragma unroll
    for (int o = 0; o < NO; ++o) acc[o][0] = acc[o][1] = 0.0f;


      // --- radial basis of this lane's edge (A-operand role)
      const float rr = r_cur;
      // the cutoff vanishes from r_max on
      const float cut = rr < prm.r_max ? 0.5f * (1.0f + __cosf(6.283185307179586f * (rr * half_turns))) : 0.0f;
      float f[kRadialMaxBasis];
#pragma unroll
      for (int bb = 0; bb < kRadialMaxBasis; ++bb) {
        const float d = (rr - center_step * (float)bb) * inv_sigma;
        f[bb] = bb < NB ? __expf(-d * d) * cut : 0.0f;
      }

      f32x4 D[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) D[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int j = 0; j < S; ++j) {
        // A operands: hidden units u = 32 j + 4 i + q of this lane's edge, scaled
        // and split; units beyond H (i >= imax, H a multiple of 4) are zero
        const int imax = (H - 32 * j) >> 2;
        f16x8 ah, al;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float h = 0.0f;
          if (i < imax) {
            const int u = 32 * j + 4 * i + q;
            const f32x4* w1u = reinterpret_cast<const f32x4*>(w1s + u * kRadialMaxBasis);
            const f32x4 wa = w1u[0], wb = w1u[1];
            float z = f[0] * wa.x;
            z = __builtin_fmaf(f[1], wa.y, z);
            z = __builtin_fmaf(f[2], wa.z, z);
            z = __builtin_fmaf(f[3], wa.w, z);
            z = __builtin_fmaf(f[4], wb.x, z);
            z = __builtin_fmaf(f[5], wb.y, z);
            z = __builtin_fmaf(f[6], wb.z, z);
            z = __builtin_fmaf(f[7], wb.w, z);
            h = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) * hsc[u];
          }
          ah[i] = (_Float16)h;
          al[i] = (_Float16)(h - (float)ah[i]);
        }
        // three products per tile, two tiles interleaved; the next pair's B
        // operands load while the current pair multiplies
        const f16x8* bj = w2s + j * NT * 2 * 64 + lane;
        f16x8 bv[4] = {bj[0], bj[64], bj[128], bj[192]};
        sfor<0, NT / 2>([&](auto pc) {
          constexpr int t = 2 * decltype(pc)::value;
          f16x8 nb[4];
          if constexpr (t + 2 < NT) {
#pragma unroll
            for (int k = 0; k < 4; ++k) nb[k] = bj[(2 * t + 4 + k) * 64];
          }
          __builtin_amdgcn_sched_barrier(0);   // the loads stay ahead of the products
          D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv[0], D[t], 0, 0, 0);
          D[t + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv[2], D[t + 1], 0, 0, 0);
          D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv[1], D[t], 0, 0, 0);
          D[t + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bv[3], D[t + 1], 0, 0, 0);
          D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv[0], D[t], 0, 0, 0);
          D[t + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bv[2], D[t + 1], 0, 0, 0);
          if constexpr (t + 2 < NT) {
#pragma unroll
            for (int k = 0; k < 4; ++k) bv[k] = nb[k];
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }

      // --- tensor product and mixing of the group's quad (edges es_q + r), channels n,
      // n + 16; the rows of edge r + 2 load while edge r is processed
      auto edge = [&](const RadialRows<LY>& R, int r) {
        float sv[NP][2];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          sv[p][0] = D[2 * p][r];
          sv[p][1] = D[2 * p + 1][r];
        }
        float yv[NY];
#pragma unroll
        for (int i = 0; i < NY / 4; ++i) {
          yv[4 * i] = R.y[i].x; yv[4 * i + 1] = R.y[i].y; yv[4 * i + 2] = R.y[i].z; yv[4 * i + 3] = R.y[i].w;
        }
        radial_edge<LY>(yv, R.x, sv, acc);
      };
      // Rows of edges 2 and 3, loaded unconditionally: past the quad's end
      // the index is clamped to its last edge (whose sender tile_ids also
      // repeats), and an empty quad reads edge 0 and node 0. A conditional
      // load here would make the compiler wait for every load in flight.
      const int e2 = c_q > 0 ? es_q + (c_q > 2 ? 2 : c_q - 1) : 0;
      const int e3 = c_q > 0 ? es_q + (c_q > 3 ? 3 : c_q - 1) : 0;
      if (c_q > 0) edge(ra, 0);
      radial_load<LY>(ra, prm, e2, sender(s_cur, 2), n);
      if (c_q > 1) edge(rb, 1);
      radial_load<LY>(rb, prm, e3, sender(s_cur, 3), n);
      if (c_q > 2) edge(ra, 2);
      if (c_q > 3) edge(rb, 3);

    // Combine the groups' partial sums per receiver: a segmented inclusive
    // scan over the four groups (quads of one receiver are contiguous), after
    // which the last group of each receiver's run in this tile holds the run's
    // sum; that group adds it to the receiver's row in LDS (lane (q, n): its
    // channels n and n + 16).  A receiver's row is written out when a quad of
    // another receiver follows it.
    {
      const int bq = q == 0 ? cur[0].b : q == 1 ? cur[1].b : q == 2 ? cur[2].b : cur[3].b;
      const bool s1 = q >= 1 && (q == 1 ? cur[0].b : q == 2 ? cur[1].b : cur[2].b) == bq;
      const bool s2 = q >= 2 && (q == 2 ? cur[0].b : cur[1].b) == bq;
#pragma unroll
      for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float t1 = __shfl_up(acc[o][c], 16, 64);
          acc[o][c] += s1 ? t1 : 0.0f;
          const float t2 = __shfl_up(acc[o][c], 32, 64);
          acc[o][c] += s2 ? t2 : 0.0f;
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (cur[g].c == 0) continue;
      if (cur[g].b != run.b) {
        if (run.b >= 0) finish(run);
        run = cur[g];
        run_slot = run.first < us ? slot0 : slot1;
      }
      const bool seg_end = g == 3 || cur[g + 1].c == 0 || cur[g + 1].b != cur[g].b;
      if (seg_end && q == g) {
#pragma unroll
        for (int o = 0; o < NO; ++o) {
          run_slot[o * C + n] += acc[o][0];
          run_slot[o * C + n + 16] += acc[o][1];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) cur[g] = nxt[g];
    r_cur = r_next;
    s_cur = s_next;
  }
  if (run.b >= 0) finish(run);
  // receivers without quads after this wave's last one (up to p_hi)
  while (wstart + 64 < p_hi) {
    WU += w_tot;
    wstart += 64;
    load_window();
  }


  // Receivers shared between waves: the wave holding the first part adds the
  // parts of the following waves (waves without tiles hold none) up to the one
  // in which the receiver ends.
  __syncthreads();
  if (part_flags[wid] & 2) {
    const int bb = part_recv[wid];
    for (int idx = lane; idx < NO * C; idx += 64) {
      float sum = part[(wid * 2 + 1) * (NO * C) + idx];
      for (int w2 = wid + 1; w2 < kRadialWaves; ++w2) {
        const int f = part_flags[w2];
        if (f == 0) continue;
        sum += part[(w2 * 2) * (NO * C) + idx];
        if (!(f & 4)) break;
      }
      __builtin_nontemporal_store(sum * (prm.inv_avg * chsc[idx % C]), prm.out + (size_t)bb * NO * C + idx);
    }
  }
}

template <class LY>
hipError_t launch_fwd_radial(const RadialParams& p, hipStream_t st) {
  if (p.num_nodes <= 0) return hipSuccess;
  if (p.num_basis < 2 || p.num_basis > kRadialMaxBasis || p.hidden < 4 || p.hidden > kRadialMaxHidden ||
      p.hidden % 4 != 0)
    return hipErrorInvalidValue;
  // one work-group per CU holds W2 and a contiguous range of receivers
  const long want = (p.num_nodes + kRadialWaves - 1) / kRadialWaves;
  long blocks = want < 256 ? want : 256;
  blocks = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_fwd_radial<LY>), dim3((unsigned)blocks), dim3(64 * kRadialWaves), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace e3c
