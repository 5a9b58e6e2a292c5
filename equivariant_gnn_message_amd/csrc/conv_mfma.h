// Forward convolution on the matrix cores (bf16 operands, fp32 accumulation),
// gfx950, for layouts with 16 output components and 64 channels.
//
//   out[b] = (1/N) sum_{e=(a->b)} (x[a] (x) y[e]) (.) s[e]
// (e3j Convolution page: class formula.)
//
// Per receiver b, written as one matrix product summed over its edges:
//   out[b][o][c] = (1/N) sum_e sum_r K_e[o][r] u_e[r][c]
// with one row r per (path p, input component m1) (Σ_p (2 l1 + 1) rows):
//   K_e[o3 + m3][r] = sum_m2 C^p[m1, m2, m3] y_e[o2 + m2]   (edge-only)
//   u_e[r][c]       = s_e[p][c] x_a[o1 + m1][c]              (per channel)
// The weighting by s is a per-row, per-channel factor of the right operand,
// so the matrix product does both the tensor product and the mixing, and the
// vector ALU keeps one product per (row, channel) instead of the
// nnz(K) + (2 l3 + 1) products per path of the register form.
//
// Mapping (wave64, v_mfma_f32_16x16x32_bf16, M = 16 output components,
// N = 16 channels per tile, four tiles for 64 channels, K = 32):
// * The 32 contraction slots of one instruction are four edges x 8 rows: lane
//   group q = lane / 16 holds edge q of an edge quad, so every lane runs the
//   same rows and only its edge and channels differ.  A receiver's edges are
//   taken four at a time; lanes past its last edge get y = 0 (K = 0).
// * Right operand (u): lane (q, n) owns channels 4n .. 4n+3 (tile t holds
//   channel 4n + t), loads its edge's s rows and its sender's x row as 8-byte
//   bf16 slices, and forms u with one exact fp32 product of the decoded bf16
//   values (decoded once per path and per x component), rounded once to bf16
//   (round to nearest even).
// * Left operand (K): each edge's K has few nonzeros (215 CG terms for
//   64x(0e+1o+2e) x Y(<=3) -> 0e+1o+2e+3o), but a lane needs the entries of
//   its own output row.  The 16 lanes of a group build their edge's nonzero
//   entries from per-lane tables (CG value, y component, destination), take
//   the y values from the lanes that hold them (ds_bpermute), and write them
//   as bf16 into the group's LDS tile, which is read back in the operand
//   layout (16 bytes per lane per k-step).  Structural zeros of the tile are
//   written once per wave; the per-lane tables sit in LDS, read per quad.
// * Rounding beyond fp32: u and K are rounded once to bf16 (relative error
//   at most 2^-8 each; the products are exact and the sums fp32), so
//   |out - exact| <= ~2^-7 (1/N) sum |C| |y| |s| |x| element by element.
//   Measured max|err| / RMS(out) against the fp64 oracle: 1.5e-2 on the bf16
//   workload (100k nodes, 3.2M edges, degree ~32), 2.7e-2 on a graph of
//   degree 1 to 7 (fewer terms per output).  With LO, K is split into a bf16
//   high part and a bf16 remainder (one more matrix instruction per tile and
//   k-step, a second LDS tile, two waves per SIMD instead of three): 1.4e-2
//   on the workload, the rounding of u left.
// * The vector ALU still forms every u (one product, half a conversion and
//   the bf16 decoding per value), so the kernel is not far below the
//   register form's time; inline assembly for the bf16 products (a dot
//   product with one half zeroed) is avoided: the compiler cannot see its
//   hazards against the matrix instructions, and it gave wrong results.
// * A wave walks its receivers (every T-th of the processing order, T waves
//   in the persistent grid) as one stream of edge quads, with the next quad's
//   rows in flight while the current one is contracted and the sender indices
//   fetched two quads ahead.
#pragma once

#include "conv_kernels.h"

namespace e3c {
namespace {

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------- compile-time tables ------

template <class LY>
constexpr int mf_rows() {
  int r = 0;
  for (int p = 0; p < LY::T.num_paths; ++p) r += 2 * LY::T.path[p].l1 + 1;
  return r;
}

template <class LY>
constexpr int mf_row_base(int p) {
  int r = 0;
  for (int i = 0; i < p; ++i) r += 2 * LY::T.path[i].l1 + 1;
  return r;
}

// Path of row r.
template <class LY>
constexpr int mf_row_path(int r) {
  for (int p = 0; p < LY::T.num_paths; ++p)
    if (r < mf_row_base<LY>(p + 1)) return p;
  return -1;
}

// Number of K entries (p, m3, m1) with exactly `terms` CG terms.
template <class LY>
constexpr int mf_entries(int terms) {
  int n = 0;
  for (int p = 0; p < LY::T.num_paths; ++p) {
    const PathInfo P = LY::T.path[p];
    for (int m3 = 0; m3 < 2 * P.l3 + 1; ++m3)
      for (int m1 = 0; m1 < 2 * P.l1 + 1; ++m1) {
        int t = 0;
        for (int e = P.nnz_begin; e < P.nnz_end; ++e)
          t += (LY::T.entry[e].m3 == m3 && LY::T.entry[e].m1 == m1) ? 1 : 0;
        n += (t == terms) ? 1 : 0;
      }
  }
  return n;
}

template <class LY>
struct MfmaShape {
  static constexpr int NR = mf_rows<LY>();
  static constexpr int KS = (NR + 7) / 8;            // k-steps of 8 rows per edge
  static constexpr int TILE = KS * 16 * 16;           // bytes of one edge's K tile (bf16)
  static constexpr int TS = TILE + 16;                // tile stride: the tile, then a dummy slot
  static constexpr int S1 = (mf_entries<LY>(1) + 15) / 16;   // single-term entries per lane
  static constexpr int S2 = (mf_entries<LY>(2) + 15) / 16;   // two-term entries per lane
  static constexpr int NE = ((S1 + S2) + 1) / 2 * 2;         // entry slots per lane (even)
  static constexpr int NTERM = NE + S2;                      // term slots per lane
  static constexpr int HALF = 4 * TS;                        // four edge tiles
  // K-build table row of one lane position n: 16 coefficient words, then 16
  // words of (4 * y component of term k) | (destination of entry k) << 8; a
  // row stride of 36 words keeps the 16 rows' reads free of bank conflicts
  static constexpr int TROW = 36;
  static_assert(NTERM <= 16 && NE <= 16 && TS < (1 << 24), "K-build table row overflow");
};

// Per-lane K-build tables for the 16 lanes of a group.  Entry slot k < S1 of
// lane i is the single-term entry i + 16 k; slots S1 .. S1+S2-1 are two-term
// entries; the rest are padding (coefficient 0, written to the tile's dummy
// slot).  Term slot t < NE belongs to entry slot t; term slot NE + k is the
// second term of entry slot S1 + k.
template <class LY>
struct MfmaKTable {
  unsigned w[16][MfmaShape<LY>::TROW];
};

template <class LY>
constexpr MfmaKTable<LY> make_mfma_ktable() {
  using S = MfmaShape<LY>;
  MfmaKTable<LY> t{};
  for (int i = 0; i < 16; ++i)
    for (int k = 0; k < S::TROW; ++k) t.w[i][k] = (k >= 16 && k < 16 + S::NE) ? (unsigned)S::TILE << 8 : 0u;
  auto put = [&](int lane, int term, float c, int ycomp) {
    t.w[lane][term] = __builtin_bit_cast(unsigned, c);
    t.w[lane][16 + term] = (t.w[lane][16 + term] & ~0xffu) | (unsigned)(4 * ycomp);
  };
  auto put_dst = [&](int lane, int k, unsigned off) {
    t.w[lane][16 + k] = (t.w[lane][16 + k] & 0xffu) | off << 8;
  };
  int n1 = 0, n2 = 0;
  for (int p = 0; p < LY::T.num_paths; ++p) {
    const PathInfo P = LY::T.path[p];
    for (int m3 = 0; m3 < 2 * P.l3 + 1; ++m3)
      for (int m1 = 0; m1 < 2 * P.l1 + 1; ++m1) {
        int q[2] = {-1, -1}, nt = 0;
        for (int e = P.nnz_begin; e < P.nnz_end; ++e)
          if (LY::T.entry[e].m3 == m3 && LY::T.entry[e].m1 == m1) {
            if (nt < 2) q[nt] = e;
            ++nt;
          }
        if (nt == 0) continue;
        const int r = mf_row_base<LY>(p) + m1;
        const int o = P.o3 + m3;
        const unsigned off = (unsigned)((((r / 8) * 16 + o) * 8 + (r % 8)) * 2);
        if (nt == 1) {
          const int lane = n1 % 16, k = n1 / 16;
          put(lane, k, LY::CG.v[q[0]], P.o2 + LY::T.entry[q[0]].m2);
          put_dst(lane, k, off);
          ++n1;
        } else {
          const int lane = n2 % 16, k = n2 / 16;
          put(lane, S::S1 + k, LY::CG.v[q[0]], P.o2 + LY::T.entry[q[0]].m2);
          put(lane, S::NE + k, LY::CG.v[q[1]], P.o2 + LY::T.entry[q[1]].m2);
          put_dst(lane, S::S1 + k, off);
          ++n2;
        }
      }
  }
  return t;
}

template <class LY>
constexpr bool mfma_terms_ok() {
  int total = 0;
  for (int k = 1; k <= 2; ++k) total += k * mf_entries<LY>(k);
  return total == LY::NNZ;   // no entry has more than two terms
}

template <class LY>
__constant__ MfmaKTable<LY> kMfmaKTable = make_mfma_ktable<LY>();

// ------------------------------------------------------------ kernel --------

__device__ __forceinline__ unsigned mf_pack(float lo, float hi) {
  const f32x2 v = {lo, hi};
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf2));
}

template <class LY>
struct MfmaBuf {
  unsigned s[LY::NP][2];     // s[e][p][4n .. 4n+3]
  unsigned x[LY::NX][2];     // x[a][i][4n .. 4n+3]
  unsigned y;                // y[e][n] (bf16 in the low half)
  bool valid;                // the lane's edge belongs to the quad
};

// One edge quad of a receiver: edges e0 .. e0+3 (those < end), receiver bl of
// the processing order (b its node).  bl == bl_end marks the end of the stream.
struct MfmaQuad {
  int bl, b, e0, end;
};

// LO: K is split into a bf16 high part and a bf16 remainder (one more matrix
// instruction per tile and k-step, and a second set of LDS tiles); without
// it K is rounded once to bf16.
template <class LY, bool LO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LO ? 2 : 3)))
conv_fwd_mfma(FwdParams prm) {
  using S = MfmaShape<LY>;
  constexpr int C = LY::C, NX = LY::NX, NY = LY::NY, NP = LY::NP, NO = LY::NO;
  static_assert(C == 64 && NO == 16 && NY <= 16, "layout outside the matrix-core form");
  static_assert(mfma_terms_ok<LY>(), "a K entry with more than two CG terms");
  constexpr int KS = S::KS, TS = S::TS, HALF = S::HALF, NE = S::NE, S1 = S::S1, S2 = S::S2;
  constexpr int NTERM = S::NTERM, TROW = S::TROW;
  constexpr int WAVE_BYTES = LO ? 2 * HALF : HALF;
  constexpr int TAB = 4 * WAVE_BYTES;                 // table offset in the work-group's LDS
  static_assert(WAVE_BYTES % 16 == 0 && TAB % 16 == 0, "16-byte LDS rows");

  __shared__ __attribute__((aligned(16))) unsigned char lds[TAB + 16 * TROW * 4];

  const bf16_bits* __restrict__ x = static_cast<const bf16_bits*>(prm.x);
  const bf16_bits* __restrict__ y = static_cast<const bf16_bits*>(prm.y);
  const bf16_bits* __restrict__ s = static_cast<const bf16_bits*>(prm.s);
  const int* __restrict__ src = prm.src;
  const int* __restrict__ row_ptr = prm.row_ptr;

  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int n = lane & 15;
  const int wbase = (int)(threadIdx.x >> 6) * WAVE_BYTES;

  // the K-build table, and zeros in the wave's tiles (structural zeros are
  // never written again)
  {
    unsigned* tab = reinterpret_cast<unsigned*>(lds + TAB);
    const unsigned* g = &kMfmaKTable<LY>.w[0][0];
    for (int i = threadIdx.x; i < 16 * TROW; i += 256) tab[i] = g[i];
    for (int o = lane * 16; o < WAVE_BYTES; o += 64 * 16)
      *reinterpret_cast<u32x4*>(lds + wbase + o) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // Wave ws takes receivers ws, ws + T, ws + 2T, ... of the processing order
  // (T waves in the grid): the receivers in progress at a time form one
  // window of the order per XCD, whose shared senders' rows stay in its L2.
  const int ws = logical_wave();
  const int T = (int)gridDim.x * 4;
  const int bl_begin = ws;
  const int bl_end = prm.num_nodes;
  if (bl_begin >= bl_end) return;

  const int ka0 = 64 * q;                  // bpermute byte offset of the group's first lane
  const int kd0 = wbase + q * TS;          // the group's K tile
  const unsigned* trow = reinterpret_cast<const unsigned*>(lds + TAB) + n * TROW;

  // receiver bounds are wave-uniform: read through the scalar cache
  typedef const __attribute__((address_space(4))) int cint;
  cint* order_u = (cint*)(uintptr_t)prm.order;
  cint* row_ptr_u = (cint*)(uintptr_t)row_ptr;
  auto first = [&](int bl) -> MfmaQuad {
    if (bl >= bl_end) return MfmaQuad{bl_end, 0, 0, 0};   // end of the wave's stream
    const int b = prm.order ? order_u[bl] : bl;
    const int beg = row_ptr_u[b];
    const int end = b < prm.num_real ? row_ptr_u[b + 1] : beg;   // padding receivers: no messages
    return MfmaQuad{bl, b, beg, end};
  };
  auto advance = [&](const MfmaQuad& d) -> MfmaQuad {
    if (d.bl >= bl_end) return d;
    if (d.e0 + 4 < d.end) return MfmaQuad{d.bl, d.b, d.e0 + 4, d.end};
    return first(d.bl + T);
  };
  // the lane's edge, clamped to a real edge (num_edges >= 1)
  auto edge_of = [&](const MfmaQuad& d) -> int {
    const int e = d.e0 + q;
    return e < d.end ? e : (d.end > 0 ? d.end - 1 : 0);
  };
  auto load_edge = [&](MfmaBuf<LY>& buf, const MfmaQuad& d) {
    const int e = edge_of(d);
    buf.valid = d.e0 + q < d.end;
    const bf16_bits* srow = s + (size_t)e * NP * C + 4 * n;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const u32x2 v = ld<u32x2, true>(reinterpret_cast<const u32x2*>(srow + p * C));
      buf.s[p][0] = v.x;
      buf.s[p][1] = v.y;
    }
    buf.y = n < NY ? (unsigned)ld<bf16_bits, true>(y + (size_t)e * NY + n) : 0u;
  };
  auto load_sender = [&](MfmaBuf<LY>& buf, int a) {
    const bf16_bits* xrow = x + (size_t)a * NX * C + 4 * n;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const u32x2 v = ld<u32x2, false>(reinterpret_cast<const u32x2*>(xrow + i * C));
      buf.x[i][0] = v.x;
      buf.x[i][1] = v.y;
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // K entries of the lane's edge from the y values of its group, into its
  // group's LDS tile
  auto build_k = [&](const MfmaBuf<LY>& buf) {
    unsigned tw[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(trow + 4 * i);
      tw[4 * i] = v.x; tw[4 * i + 1] = v.y; tw[4 * i + 2] = v.z; tw[4 * i + 3] = v.w;
    }
    const int yi = buf.valid ? (int)(buf.y << 16) : 0;
    auto yv = [&](int term) {
      return __int_as_float(__builtin_amdgcn_ds_bpermute(ka0 + (int)(tw[16 + term] & 0xffu), yi));
    };
    float kv[NE];
#pragma unroll
    for (int k = 0; k < NE; ++k) kv[k] = __uint_as_float(tw[k]) * yv(k);
#pragma unroll
    for (int k = 0; k < S2; ++k) kv[S1 + k] = __builtin_fmaf(__uint_as_float(tw[NE + k]), yv(NE + k), kv[S1 + k]);
    wave_lds_sync();   // the previous quad's operand reads come first
#pragma unroll
    for (int k = 0; k < NE; k += 2) {
      const unsigned hi = mf_pack(kv[k], kv[k + 1]);
      bf16_bits* d0 = reinterpret_cast<bf16_bits*>(lds + kd0 + (int)(tw[16 + k] >> 8));
      bf16_bits* d1 = reinterpret_cast<bf16_bits*>(lds + kd0 + (int)(tw[17 + k] >> 8));
      *d0 = (bf16_bits)(hi & 0xffffu);
      *d1 = (bf16_bits)(hi >> 16);
      if constexpr (LO) {
        const unsigned lo = mf_pack(kv[k] - bf_lo(hi), kv[k + 1] - bf_hi(hi));
        *reinterpret_cast<bf16_bits*>(reinterpret_cast<unsigned char*>(d0) + HALF) = (bf16_bits)(lo & 0xffffu);
        *reinterpret_cast<bf16_bits*>(reinterpret_cast<unsigned char*>(d1) + HALF) = (bf16_bits)(lo >> 16);
      }
    }
    wave_lds_sync();
  };

  // the edge quad's products on the matrix cores
  auto contract = [&](const MfmaBuf<LY>& buf) {
    const unsigned char* arow = lds + kd0 + n * 16;
    sfor<0, KS>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      const u32x4 ah = *reinterpret_cast<const u32x4*>(arow + ks * 256);
      u32x4 al = {0u, 0u, 0u, 0u};
      if constexpr (LO) al = *reinterpret_cast<const u32x4*>(arow + HALF + ks * 256);
      unsigned bw[4][4];   // [tile][row pair]
      sfor<0, 4>([&](auto jpc) {
        constexpr int jp = decltype(jpc)::value;
        float u[2][4];
        sfor<0, 2>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          constexpr int r = 8 * ks + 2 * jp + h;
          if constexpr (r < S::NR) {
            constexpr int p = mf_row_path<LY>(r);
            constexpr int comp = LY::T.path[p].o1 + (r - mf_row_base<LY>(p));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const unsigned sw = buf.s[p][c >> 1], xw = buf.x[comp][c >> 1];
              u[h][c] = (c & 1) ? bf_hi(sw) * bf_hi(xw) : bf_lo(sw) * bf_lo(xw);   // exact
            }
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) u[h][c] = 0.0f;
          }
        });
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) bw[tt][jp] = mf_pack(u[0][tt], u[1][tt]);
      });
      mf_bf16x8 bb[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const u32x4 bv = {bw[tt][0], bw[tt][1], bw[tt][2], bw[tt][3]};
        bb[tt] = __builtin_bit_cast(mf_bf16x8, bv);
      }
      // the four tiles' products are independent: high parts, then remainders
      const mf_bf16x8 a_hi = __builtin_bit_cast(mf_bf16x8, ah);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bb[tt], acc[tt], 0, 0, 0);
      if constexpr (LO) {
        const mf_bf16x8 a_lo = __builtin_bit_cast(mf_bf16x8, al);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bb[tt], acc[tt], 0, 0, 0);
      }
    });
  };

  // row b of out from a wave-uniform base and a 32-bit lane offset (kept
  // opaque so that no 64-bit per-lane pointer lives across the loop)
  const unsigned lane_off = (unsigned)((4 * q * C + 4 * n) * 4);
  auto store = [&](int b) {
    char* orow = reinterpret_cast<char*>(prm.out + (size_t)__builtin_amdgcn_readfirstlane(b) * NO * C);
    unsigned off = lane_off;
    asm volatile("" : "+v"(off));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 v = {acc[0][r] * prm.inv_avg, acc[1][r] * prm.inv_avg, acc[2][r] * prm.inv_avg,
                       acc[3][r] * prm.inv_avg};
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(orow + off + r * C * 4));
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };

  MfmaQuad d0 = first(bl_begin);
  MfmaQuad d1 = advance(d0);
  MfmaQuad d2 = advance(d1);
  int a1 = src[edge_of(d1)];
  int a2 = src[edge_of(d2)];
  MfmaBuf<LY> b0, b1;
  load_edge(b0, d0);
  load_sender(b0, src[edge_of(d0)]);

  // One quad: the next one's edge rows go in flight, this one's K is built
  // and it is contracted, then the next one's sender rows (cache resident,
  // shorter latency) go in flight.
  // Past the end of the stream the loads are of edge 0 (unconditional loads
  // keep the wait for this quad's rows from covering the next quad's).
  auto step = [&](MfmaBuf<LY>& cur, MfmaBuf<LY>& nxt) -> bool {
    const bool more = d1.bl < bl_end;
    const MfmaQuad d3 = advance(d2);
    const int a3 = src[edge_of(d3)];
    load_edge(nxt, d1);
    __builtin_amdgcn_sched_barrier(0);
    build_k(cur);
    __builtin_amdgcn_sched_barrier(0);   // contract's operand decoding waits for cur's sender rows
    contract(cur);
    __builtin_amdgcn_sched_barrier(0);
    load_sender(nxt, a1);
    if (d1.bl != d0.bl) store(d0.b);
    d0 = d1;
    d1 = d2;
    d2 = d3;
    a1 = a2;
    a2 = a3;
    return more;
  };
  while (step(b0, b1) && step(b1, b0)) {
  }
}

// A persistent grid: as many work-groups as fit the chip at once (256 CUs,
// three or two work-groups of four waves per CU), each wave looping over its
// receivers.
template <class LY, bool LO = false>
hipError_t launch_fwd_mfma(const FwdParams& p, hipStream_t st) {
  if (p.num_nodes <= 0) return hipSuccess;
  if (p.num_edges <= 0)   // no messages: every row is zero
    return launch_fill_zero(p.out, (size_t)p.num_nodes * LY::NO * LY::C, st);
  const long resident = 256L * (LO ? 2 : 3);
  const long needed = ((p.num_nodes + 3) / 4 + 7) / 8 * 8;
  const long blocks = needed < resident ? needed : resident;
  hipLaunchKernelGGL((conv_fwd_mfma<LY, LO>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace e3c
