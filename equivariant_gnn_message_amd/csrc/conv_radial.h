// Convolution with the edge scalars computed in the kernel from the edge
// lengths (gate-points page: radial embedding of the edge length, then a
// fully connected network whose outputs weight the convolution's paths and
// channels), for layouts of 32 channels, fp32.
//
//   f_k(r) = exp(-((r - mu_k) / sigma)^2) (1 + cos(pi r / r_max)) / 2,
//   s[e]   = silu(f(r_e) W1) W2   -> (NP, C),
//   out[b] = (1/N) sum_{e=(a->b)} (x[a] (x) y[e]) (.) s[e].
//
// The scalars never reach memory: the (E, NP, C) tensor that would otherwise
// be written by the network and read back by the convolution is formed per
// receiver in registers.
//
// Per receiver, in tiles of 16 of its edges (one wave):
// * lane (m, q) = (lane % 16, lane / 16) evaluates the basis for edge m of the
//   tile and the hidden units k = 4 j + q (j = 0 .. hidden/4 - 1), which is
//   exactly the A operand of v_mfma_f32_16x16x4_f32 for contraction step j;
// * s (16 edges x NP*C) = h W2 is accumulated over hidden/4 steps in NP*C/16
//   accumulator tiles; W2 is staged once per work-group in LDS, permuted so
//   that a lane's B values of one step for all N tiles are contiguous;
// * the accumulator layout hands lane (g, n) = (lane / 16, lane % 16) the
//   scalars of edges 4g .. 4g+3 of the tile for channels n and n + 16 of every
//   path (column p*C + c lies in tile 2p + c/16), so each lane runs the tensor
//   product and mixing of its 4 edges for those two channels;
// * the partial sums of the 4 lane groups are combined per receiver with
//   cross-lane shuffles and each output row is written once.
#pragma once

#include "conv_kernels.h"

namespace e3c {
namespace {

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

// Wave index in processing order for 8-wave work-groups (XCD-contiguous
// ranges, as logical_wave() for 4-wave groups).
__device__ __forceinline__ int logical_wave8() {
  const int per_xcd = (int)(gridDim.x >> 3);
  const int bid = (int)blockIdx.x;
  const int lb = (bid & 7) * per_xcd + (bid >> 3);
  return __builtin_amdgcn_readfirstlane(lb * kRadialWaves + (int)(threadIdx.x >> 6));
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
  // W2 as [k][t/4][n][t%4] (k < hidden, n < 16, t < NT): the 16 lanes of a
  // quarter-wave read 16 consecutive 16-byte chunks (no bank conflicts);
  // W1 as [k][b] (b < 8)
  __shared__ __attribute__((aligned(16))) float w2s[kRadialMaxHidden * 16 * NT];
  __shared__ __attribute__((aligned(16))) float w1s[kRadialMaxHidden * kRadialMaxBasis];

  const int H = prm.hidden, NB = prm.num_basis;
  // Coalesced float4 reads of W2, eight in flight per thread, scattered into
  // the LDS layout (NP * C is a multiple of 64, so a float4 stays in one row
  // and one tile).
  {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(prm.w2);
    const int total4 = H * NP * C / 4;
    for (int base = threadIdx.x; base < total4; base += 8 * 64 * kRadialWaves) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i4 = base + u * 64 * kRadialWaves;
        v[u] = i4 < total4 ? g4[i4] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i4 = base + u * 64 * kRadialWaves;
        if (i4 < total4) {
          const int k = (4 * i4) / (NP * C), col = (4 * i4) % (NP * C);
          const int tt = col >> 4, n0 = col & 15;
          float* dst = w2s + ((k * (NT / 4) + (tt >> 2)) * 16 + n0) * 4 + (tt & 3);
          dst[0] = v[u].x;
          dst[4] = v[u].y;
          dst[8] = v[u].z;
          dst[12] = v[u].w;
        }
      }
    }
  }
  for (int i = threadIdx.x; i < H * kRadialMaxBasis; i += 64 * kRadialWaves) {
    const int k = i / kRadialMaxBasis, bb = i % kRadialMaxBasis;
    w1s[i] = bb < NB ? prm.w1[bb * H + k] : 0.0f;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, n = lane & 15;   // A-operand role (edge n, hidden units 4j + q); output role (group q, column n)
  const int steps = H / 4;
  const float inv_sigma = 1.0f / prm.sigma;
  const float center_step = prm.r_max / (float)(NB - 1);
  const float half_turns = 0.5f / prm.r_max;   // cos(pi r / r_max) = cos(2 pi (r / (2 r_max)))

  // Each wave owns a contiguous range of the processing order.  In index
  // order the ranges are cut at equal shares of the edges (receiver b goes to
  // the wave whose share holds row_ptr[b]), so waves get similar work; with a
  // permutation they are cut at equal numbers of receivers.
  const int waves = (int)gridDim.x * kRadialWaves;
  const int wave = logical_wave8();
  int b_first, b_last;
  if (prm.order) {
    const int per_wave = (prm.num_nodes + waves - 1) / waves;
    b_first = wave * per_wave < prm.num_nodes ? wave * per_wave : prm.num_nodes;
    b_last = b_first + per_wave < prm.num_nodes ? b_first + per_wave : prm.num_nodes;
  } else {
    auto first_at = [&](long v) {   // first b in [0, N] with row_ptr[b] >= v
      int lo = 0, hi = prm.num_nodes;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((long)prm.row_ptr[mid] < v) lo = mid + 1; else hi = mid;
      }
      return lo;
    };
    const long E = prm.row_ptr[prm.num_nodes];
    b_first = first_at(E * wave / waves);
    b_last = wave == waves - 1 ? prm.num_nodes : first_at(E * (wave + 1) / waves);
  }

  // The edge length and the four sender indices a lane needs for a tile are
  // fetched one tile ahead (across receiver boundaries), so that neither the
  // network nor the gathers of a tile wait for them.
  auto recv = [&](int bl, int& b, int& beg, int& end) {
    b = prm.order ? prm.order[bl] : bl;
    beg = prm.row_ptr[b];
    end = b < prm.num_real ? prm.row_ptr[b + 1] : beg;
  };
  auto tile_ids = [&](int e0, int end, float& rv, int (&sv)[4]) {
    rv = prm.r[e0 + n < end ? e0 + n : end - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = e0 + 4 * q + i < end ? prm.src[e0 + 4 * q + i] : 0;
  };
  int b = 0, beg = 0, end = 0;
  float r_cur = 0.0f;
  int s_cur[4] = {0, 0, 0, 0};
  if (b_first < b_last) {
    recv(b_first, b, beg, end);
    if (beg < end) tile_ids(beg, end, r_cur, s_cur);
  }

  for (int bl = b_first; bl < b_last; ++bl) {
    const bool more = bl + 1 < b_last;
    int bn = 0, begn = 0, endn = 0;
    if (more) recv(bl + 1, bn, begn, endn);

    float acc[NO][2];
#pragma unroll
    for (int o = 0; o < NO; ++o) acc[o][0] = acc[o][1] = 0.0f;

    for (int e0 = beg; e0 < end; e0 += 16) {
      float r_next = 0.0f;
      int s_next[4] = {0, 0, 0, 0};
      if (e0 + 16 < end) {
        tile_ids(e0 + 16, end, r_next, s_next);
      } else if (more && begn < endn) {
        tile_ids(begn, endn, r_next, s_next);
      }
      // rows of this lane's first two edges, in flight during the network
      const int eq = e0 + 4 * q;
      RadialRows<LY> ra, rb;
      if (eq < end) radial_load<LY>(ra, prm, eq, s_cur[0], n);
      if (eq + 1 < end) radial_load<LY>(rb, prm, eq + 1, s_cur[1], n);

      // --- hidden units of edge e0 + n (A operand: units 4j + q)
      const float rr = r_cur;
      const float cut = 0.5f * (1.0f + __cosf(6.283185307179586f * (rr * half_turns)));
      float f[kRadialMaxBasis];
#pragma unroll
      for (int bb = 0; bb < kRadialMaxBasis; ++bb) {
        const float d = (rr - center_step * (float)bb) * inv_sigma;
        f[bb] = bb < NB ? __expf(-d * d) * cut : 0.0f;
      }

      // silu(f . W1[:, k]) for this lane's edge
      auto hidden = [&](int k) {
        const f32x4* w1k = reinterpret_cast<const f32x4*>(w1s + k * kRadialMaxBasis);
        const f32x4 wa = w1k[0], wb = w1k[1];
        float z = f[0] * wa.x;
        z = __builtin_fmaf(f[1], wa.y, z);
        z = __builtin_fmaf(f[2], wa.z, z);
        z = __builtin_fmaf(f[3], wa.w, z);
        z = __builtin_fmaf(f[4], wb.x, z);
        z = __builtin_fmaf(f[5], wb.y, z);
        z = __builtin_fmaf(f[6], wb.z, z);
        z = __builtin_fmaf(f[7], wb.w, z);
        return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
      };
      // this lane's B values of hidden unit row k for all NT tiles
      auto bload = [&](int k, f32x4 (&bv)[NT / 4]) {
        const f32x4* bk = reinterpret_cast<const f32x4*>(w2s + k * 16 * NT) + n;
#pragma unroll
        for (int t4 = 0; t4 < NT / 4; ++t4) bv[t4] = bk[16 * t4];
      };
      f32x4 D[NT];
      auto step = [&](float h, const f32x4 (&bv)[NT / 4], bool first) {
#pragma unroll
        for (int t4 = 0; t4 < NT / 4; ++t4) {
          const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
          D[4 * t4 + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(h, bv[t4].x, first ? zero : D[4 * t4 + 0], 0, 0, 0);
          D[4 * t4 + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(h, bv[t4].y, first ? zero : D[4 * t4 + 1], 0, 0, 0);
          D[4 * t4 + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(h, bv[t4].z, first ? zero : D[4 * t4 + 2], 0, 0, 0);
          D[4 * t4 + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(h, bv[t4].w, first ? zero : D[4 * t4 + 3], 0, 0, 0);
        }
      };
      // Two operand buffers, each filled two steps before its MFMAs: a step's
      // hidden unit and B rows never wait for the instructions just before it.
      f32x4 b0[NT / 4], b1[NT / 4];
      bload(q, b0);
      float h0 = hidden(q), h1 = 0.0f;
      if (steps > 1) {
        bload(4 + q, b1);
        h1 = hidden(4 + q);
      }
      step(h0, b0, true);
      for (int j = 0; j < steps; j += 2) {
        if (j > 0) step(h0, b0, false);
        if (j + 2 < steps) {
          h0 = hidden(4 * (j + 2) + q);
          bload(4 * (j + 2) + q, b0);
        }
        if (j + 1 < steps) {
          step(h1, b1, false);
          if (j + 3 < steps) {
            h1 = hidden(4 * (j + 3) + q);
            bload(4 * (j + 3) + q, b1);
          }
        }
      }

      // --- tensor product and mixing of edges e0 + 4q + r, channels n, n + 16;
      // the rows of edge r + 2 load while edge r is processed
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
      if (eq < end) {
        edge(ra, 0);
        if (eq + 2 < end) radial_load<LY>(ra, prm, eq + 2, s_cur[2], n);
      }
      if (eq + 1 < end) {
        edge(rb, 1);
        if (eq + 3 < end) radial_load<LY>(rb, prm, eq + 3, s_cur[3], n);
      }
      if (eq + 2 < end) edge(ra, 2);
      if (eq + 3 < end) edge(rb, 3);
      r_cur = r_next;
#pragma unroll
      for (int i = 0; i < 4; ++i) s_cur[i] = s_next[i];
    }

    // the four lane groups hold partial sums of different edges
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        acc[o][c] += __shfl_xor(acc[o][c], 16, 64);
        acc[o][c] += __shfl_xor(acc[o][c], 32, 64);
      }
    float* orow = prm.out + (size_t)b * NO * C;
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      if ((o & 3) != q) continue;
      __builtin_nontemporal_store(acc[o][0] * prm.inv_avg, orow + o * C + n);
      __builtin_nontemporal_store(acc[o][1] * prm.inv_avg, orow + o * C + n + 16);
    }
    if (more) {
      // after a receiver without edges the next one's first tile was not fetched
      if (beg == end && begn < endn) tile_ids(begn, endn, r_cur, s_cur);
      b = bn;
      beg = begn;
      end = endn;
    }
  }
}

template <class LY>
hipError_t launch_fwd_radial(const RadialParams& p, hipStream_t st) {
  if (p.num_nodes <= 0) return hipSuccess;
  if (p.num_basis < 2 || p.num_basis > kRadialMaxBasis || p.hidden < 4 || p.hidden > kRadialMaxHidden ||
      p.hidden % 4 != 0)
    return hipErrorInvalidValue;
  // one work-group per CU holds W2; each wave owns a contiguous range of receivers
  const long want = (p.num_nodes + kRadialWaves - 1) / kRadialWaves;
  long blocks = want < 256 ? want : 256;
  blocks = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL((conv_fwd_radial<LY>), dim3((unsigned)blocks), dim3(64 * kRadialWaves), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace e3c
