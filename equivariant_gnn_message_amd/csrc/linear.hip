// Output linear (channel mixing within each irrep block) on the matrix cores,
// fp32 products from three-part bf16 operands.
//
// cuEquivariance page, Flax NNX layers, IrrepsLinear: within each irrep block
// the channels are mixed, out[..., v, i] = scale / sqrt(mul_in) * sum_u w[u, v] in[..., u, i].
// With trailing channels the convolution output is (N, num_out, C): for each
// output component o (of block k) this is a plain GEMM over the node axis,
//     out[:, o, :] = alpha * in[:, o, :] @ W_k,   W_k (C, C_out),
// and its reverse is two more GEMMs:
//     grad_in[:, o, :] = alpha * grad_out[:, o, :] @ W_k^T,
//     grad_W_k        += alpha * in[:, o, :]^T @ grad_out[:, o, :]  (summed over o in block k).
// A tiled kernel serves all three through element strides (the row-streaming
// kernel further down takes out and grad_in when K, N <= 128): 128 x 128 output
// tiles per work-group of four waves (128 columns cover C_out <= 128 in one
// tile, so each input row is read from memory once; 128 rows share each read
// and split of B), 32-deep K chunks, each wave a 64 x 64 quadrant of 4 x 4
// accumulators of v_mfma_f32_16x16x32_bf16.
//
// fp32 products at fp32 accuracy on the bf16 matrix instruction: each operand
// element is split into three bf16 parts, v = v0 + v1 + v2 (v1 = bf16(v - v0),
// v2 = bf16(v - v0 - v1); 24 significand bits, fp32's exponent range), and the
// six partial products of total order <= 2 are accumulated in fp32
// (a0 b0 + a0 b1 + a1 b0 + a0 b2 + a1 b1 + a2 b0); the dropped ones are below
// 2^-24 of the product.  fp32 matrix instructions would take 2.7 times the
// matrix cycles and do not overlap vector work, which the split needs.
// The fp32 elements of the next K chunk are loaded into registers while the
// current chunk is multiplied, then split once and stored to LDS as three
// bf16 planes, rows of 32 k (+ 8 padding: conflict-free 16-byte reads).  The
// reduction over nodes for grad_W is split across work-groups and combined
// with fp32 atomics.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace e3c {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int TM = 128, TN = 128, TK = 32;
constexpr int MT = 4, NTW = 4;     // 16 x 16 MFMA tiles per wave (rows, columns)
constexpr int RU = TK / 8 + 1;     // 16-byte units per LDS row (4 used, 1 padding)

// Eight elements p[0], p[s], ..., p[7 s] (those with index < n; the others 0;
// with n == 0, p must still point at a valid element).
__device__ __forceinline__ void load8(const float* p, long s, int n, bool vec, float (&v)[8]) {
  if (vec) {   // s == 1, 16-byte aligned, n == 8
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = p[i < n ? (long)i * s : 0];   // clamped address, no branch
      v[i] = i < n ? x : 0.0f;
    }
  }
}

// v = v0 + v1 + v2 in bf16 (round to nearest at each step).
__device__ __forceinline__ void split3(const float (&v)[8], bf16x8& p0, bf16x8& p1, bf16x8& p2) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p0[i] = (__bf16)v[i];
    const float r1 = v[i] - (float)p0[i];
    p1[i] = (__bf16)r1;
    p2[i] = (__bf16)(r1 - (float)p1[i]);
  }
}

__global__ void __launch_bounds__(256) linear_gemm(LinearGemm g) {
  __shared__ __attribute__((aligned(16))) bf16x8 As[3][TM][RU];
  __shared__ __attribute__((aligned(16))) bf16x8 Bs[3][TN][RU];   // B transposed: [column][k]

  const int o = blockIdx.z % g.num_comp;           // output component of this slice
  const int split = blockIdx.z / g.num_comp;       // K split (reduction over nodes)
  const int blk = g.comp_block[o];
  const float* A = g.A + (long)o * g.a_comp;
  const float* B = g.B + (long)o * g.b_comp + (long)blk * g.b_block;
  float* C = g.C + (long)o * g.c_comp + (long)blk * g.c_block;

  const int i0 = blockIdx.x * TM, j0 = blockIdx.y * TN;
  const int kbeg = split * g.k_chunk;
  const int kend = kbeg + g.k_chunk < g.K ? kbeg + g.k_chunk : g.K;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wr = (w >> 1) * 64, wc = (w & 1) * 64;
  const int lr = lane & 15, lk = lane >> 4;

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging units: eight consecutive k of one row of A or of one column of B
  // (512 units each, two per thread).  Consecutive threads walk the operand's
  // contiguous axis: the k runs when it is k (then read as two 16-byte loads
  // where aligned), else the rows/columns.
  const bool a_kc = g.a_k == 1, b_kc = g.b_k == 1;
  int ua_i[2], ua_c[2];
  bool ua_ok[2];
  const float* pa[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = t + 256 * r;
    ua_i[r] = a_kc ? u >> 2 : u & 127;
    ua_c[r] = a_kc ? u & 3 : u >> 7;
    ua_ok[r] = i0 + ua_i[r] < g.M;
    pa[r] = A + (ua_ok[r] ? (long)(i0 + ua_i[r]) * g.a_i : 0) + (long)(8 * ua_c[r]) * g.a_k;
  }
  const bool a_vec = a_kc && (g.a_i & 3) == 0 && ((reinterpret_cast<unsigned long>(A) & 15) == 0);
  int ub_j[2], ub_c[2];
  bool ub_ok[2];
  const float* pb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = t + 256 * r;
    ub_j[r] = b_kc ? u >> 2 : u & 127;
    ub_c[r] = b_kc ? u & 3 : u >> 7;
    ub_ok[r] = j0 + ub_j[r] < g.N;
    pb[r] = B + (ub_ok[r] ? (long)(j0 + ub_j[r]) * g.b_j : 0) + (long)(8 * ub_c[r]) * g.b_k;
  }
  const bool b_vec = b_kc && (g.b_j & 3) == 0 && ((reinterpret_cast<unsigned long>(B) & 15) == 0);

  // Full tiles whose operands are contiguous across rows/columns and strided
  // along k (grad_W: A = in^T, B = grad_out over the node axis): threads
  // 0..127 read A, 128..255 read B, each eight 16-byte rows (four rows or
  // columns at eight consecutive k), which are four staging units.
  const bool kt = g.a_i == 1 && g.b_j == 1 && (g.a_k & 3) == 0 && (g.b_k & 3) == 0 &&
                  (reinterpret_cast<unsigned long>(A) & 15) == 0 && (reinterpret_cast<unsigned long>(B) & 15) == 0 &&
                  i0 + TM <= g.M && j0 + TN <= g.N;
  const int kt_c4 = t & 31, kt_r = (t >> 5) & 3;   // 4 rows/columns from 4 kt_c4, k run kt_r
  const float* kt_p = t < 128 ? A + (long)(i0 + 4 * kt_c4) : B + (long)(j0 + 4 * kt_c4);
  const long kt_s = t < 128 ? g.a_k : g.b_k;
  f32x4 kraw[8];
  int kt_n = 0;
  auto fetch_kt = [&](int k0) {
    int n = kend - (k0 + 8 * kt_r);
    kt_n = n < 8 ? (n > 0 ? n : 0) : 8;
    const float* p = kt_p + (long)(k0 + 8 * kt_r) * kt_s;
#pragma unroll
    for (int i = 0; i < 8; ++i) kraw[i] = *reinterpret_cast<const f32x4*>(i < kt_n ? p + i * kt_s : kt_p);
  };
  auto stage_kt = [&]() {
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < kt_n ? kraw[i][c4] : 0.0f;
      bf16x8 p0, p1, p2;
      split3(v, p0, p1, p2);
      const int row = 4 * kt_c4 + c4;
      if (t < 128) {
        As[0][row][kt_r] = p0;
        As[1][row][kt_r] = p1;
        As[2][row][kt_r] = p2;
      } else {
        Bs[0][row][kt_r] = p0;
        Bs[1][row][kt_r] = p1;
        Bs[2][row][kt_r] = p2;
      }
    }
  };

  float ra[2][8], rb[2][8];
  auto fetch = [&](int k0) {
    const bool full = k0 + TK <= kend;
    // slots past M, N or the chunk's end read element 0 of the operand and are zeroed
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int na = ua_ok[r] ? kend - (k0 + 8 * ua_c[r]) : 0;
      na = na < 8 ? (na > 0 ? na : 0) : 8;
      load8(na > 0 ? pa[r] + (long)k0 * g.a_k : A, g.a_k, na, a_vec && full && ua_ok[r], ra[r]);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      int nb = ub_ok[r] ? kend - (k0 + 8 * ub_c[r]) : 0;
      nb = nb < 8 ? (nb > 0 ? nb : 0) : 8;
      load8(nb > 0 ? pb[r] + (long)k0 * g.b_k : B, g.b_k, nb, b_vec && full && ub_ok[r], rb[r]);
    }
  };
  auto stage = [&]() {
    bf16x8 p0, p1, p2;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      split3(ra[r], p0, p1, p2);
      As[0][ua_i[r]][ua_c[r]] = p0;
      As[1][ua_i[r]][ua_c[r]] = p1;
      As[2][ua_i[r]][ua_c[r]] = p2;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      split3(rb[r], p0, p1, p2);
      Bs[0][ub_j[r]][ub_c[r]] = p0;
      Bs[1][ub_j[r]][ub_c[r]] = p1;
      Bs[2][ub_j[r]][ub_c[r]] = p2;
    }
  };
  if (kbeg < kend) {
    if (kt) fetch_kt(kbeg);
    else fetch(kbeg);
  }
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    if (kt) stage_kt();
    else stage();
    __syncthreads();
    if (k0 + TK < kend) {
      if (kt) fetch_kt(k0 + TK);
      else fetch(k0 + TK);
    }
    // A[m][8 q + i] and B[8 q + i][n] of lane (q, m or n) = (lk, lr)
    bf16x8 av[3][MT], bv[3][NTW];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
      for (int a = 0; a < MT; ++a) av[p][a] = As[p][wr + a * 16 + lr][lk];
#pragma unroll
      for (int b = 0; b < NTW; ++b) bv[p][b] = Bs[p][wc + b * 16 + lr][lk];
    }
    constexpr int PA[6] = {0, 0, 1, 0, 1, 2}, PB[6] = {0, 1, 0, 2, 1, 0};
#pragma unroll
    for (int pr = 0; pr < 6; ++pr)
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[PA[pr]][a], bv[PB[pr]][b], acc[a][b], 0, 0, 0);
    __syncthreads();
  }

  // D[4*(lane/16) + r][lane % 16] of each 16 x 16 accumulator
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = i0 + wr + a * 16 + 4 * lk + r;
        const int gj = j0 + wc + b * 16 + lr;
        if (gi < g.M && gj < g.N) {
          float* dst = C + (long)gi * g.c_i + (long)gj * g.c_j;
          const float v = g.alpha * acc[a][b][r];
          if (g.atomic) {
            unsafeAtomicAdd(dst, v);
          } else {
            *dst = v;
          }
        }
      }
}

// Row-streaming variant for the GEMMs whose B is one weight block shared by all
// components of an irrep block (out = in W_k and grad_in = grad_out W_k^T: A
// contiguous along k, K <= 128, N <= 128).  A work-group splits W_k once into
// LDS (three bf16 planes, 96 KiB at 128 x 128, laid out so that a B operand
// is 16 contiguous bytes per lane) and its waves stream 16-row tiles of A
// straight from memory into the A operands (lane (m, q) reads A[m][32 s + 8 q
// .. + 7], splitting it in registers), the next tile's rows in flight during
// the current tile's products.  Row tiles are numbered component-major, so a
// work-group's contiguous range spans few irrep blocks (W_k is restaged at
// each change).
constexpr int RW = 8;                     // waves per work-group
constexpr int RKS = 4, RNT = 8;           // at most 4 K steps of 32, 8 column tiles of 16

// KSC, NTC > 0: K = 32 KSC, N = 16 NTC and A rows 16-byte aligned (checked by
// the launcher): static loops, one row pointer per tile, rows past M read row
// M - 1 and are not stored (an output row depends on its own input row only).
// KSC = NTC = 0: any K, N <= 128 with masked loads and stores.
template <int KSC, int NTC>
__global__ void __launch_bounds__(64 * RW) linear_rows(LinearGemm g, int tiles_total, int tiles_per_block,
                                                         int node_tiles) {
  __shared__ __attribute__((aligned(16))) bf16x8 Ws[3 * RKS * RNT * 64];   // [plane][s][t][q][n]
  constexpr bool FIX = KSC > 0;
  constexpr int PS = RKS * RNT * 64;   // plane size (16-byte units)

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int KS = FIX ? KSC : (g.K + 31) >> 5, NT = FIX ? NTC : (g.N + 15) >> 4;
  const int t0 = blockIdx.x * tiles_per_block;
  const int t1 = t0 + tiles_per_block < tiles_total ? t0 + tiles_per_block : tiles_total;
  const bool a_vec = (g.a_i & 3) == 0 && (g.a_comp & 3) == 0 && (g.K & 7) == 0 &&
                     (reinterpret_cast<unsigned long>(g.A) & 15) == 0;
  const bool b_vec = g.b_k == 1 && (g.b_j & 3) == 0 && (g.K & 7) == 0 &&
                     (reinterpret_cast<unsigned long>(g.B) & 15) == 0 && (g.b_block & 3) == 0;

  // raw rows of a tile: k = 32 s + 8 q + i of row n0 + m
  auto fetch = [&](int tau, float (&raw)[RKS][8]) {
    const int o = tau / node_tiles, row = (tau % node_tiles) * 16 + m;
    const float* Ao = g.A + (long)o * g.a_comp;
    if constexpr (FIX) {
      const f32x4* rp = reinterpret_cast<const f32x4*>(Ao + (long)(row < g.M ? row : g.M - 1) * g.a_i + 8 * q);
#pragma unroll
      for (int st = 0; st < KSC; ++st) {
        const f32x4 lo = rp[8 * st], hi = rp[8 * st + 1];
        raw[st][0] = lo.x; raw[st][1] = lo.y; raw[st][2] = lo.z; raw[st][3] = lo.w;
        raw[st][4] = hi.x; raw[st][5] = hi.y; raw[st][6] = hi.z; raw[st][7] = hi.w;
      }
    } else {
#pragma unroll
      for (int st = 0; st < RKS; ++st) {
        int n = row < g.M ? g.K - (32 * st + 8 * q) : 0;
        n = n < 8 ? (n > 0 ? n : 0) : 8;
        load8(n > 0 ? Ao + (long)row * g.a_i + 32 * st + 8 * q : g.A, 1, n, a_vec && n == 8, raw[st]);
      }
    }
  };

  for (int base = t0; base < t1;) {
    const int blk = g.comp_block[base / node_tiles];
    int o_end = base / node_tiles;
    while (o_end < g.num_comp && g.comp_block[o_end] == blk) ++o_end;
    const int te = o_end * node_tiles < t1 ? o_end * node_tiles : t1;

    // W_k, split into three planes: unit (s, q, t, n) holds B[32 s + 8 q + i][16 t + n], i < 8
    __syncthreads();   // the previous block's W is no longer read
    const float* Bk = g.B + (long)blk * g.b_block;
    for (int u = threadIdx.x; u < RKS * 4 * RNT * 16; u += 64 * RW) {
      const int n = u & 15, tt = (u >> 4) & 7, qq = (u >> 7) & 3, st = u >> 9;
      const int j = 16 * tt + n, k0 = 32 * st + 8 * qq;
      int cnt = j < g.N ? g.K - k0 : 0;
      cnt = cnt < 8 ? (cnt > 0 ? cnt : 0) : 8;
      float v[8];
      load8(cnt > 0 ? Bk + (long)k0 * g.b_k + (long)j * g.b_j : g.B, g.b_k, cnt, b_vec && cnt == 8, v);
      bf16x8 p0, p1, p2;
      split3(v, p0, p1, p2);
      const int idx = (st * RNT + tt) * 64 + qq * 16 + n;
      Ws[idx] = p0;
      Ws[PS + idx] = p1;
      Ws[2 * PS + idx] = p2;
    }
    __syncthreads();

    float raw[RKS][8];
    int tau = base + wid;
    if (tau < te) fetch(tau, raw);
    for (; tau < te; tau += RW) {
      bf16x8 a0[RKS], a1[RKS], a2[RKS];
#pragma unroll
      for (int st = 0; st < RKS; ++st)
        if (!FIX || st < KSC) split3(raw[st], a0[st], a1[st], a2[st]);
      if (tau + RW < te) fetch(tau + RW, raw);   // next tile's rows in flight

      f32x4 acc[RNT];
#pragma unroll
      for (int tt = 0; tt < RNT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int o = tau / node_tiles, n0 = (tau % node_tiles) * 16;
      float* Co = g.C + (long)o * g.c_comp + (long)blk * g.c_block;
      if constexpr (FIX) {
        // groups of up to four column tiles: four independent products between dependent ones
        constexpr int GT = NTC < 4 ? NTC : 4;
#pragma unroll
        for (int st = 0; st < KSC; ++st)
#pragma unroll
          for (int t0g = 0; t0g < NTC; t0g += GT) {
            bf16x8 b0[GT], b1[GT], b2[GT];
#pragma unroll
            for (int u = 0; u < GT; ++u) {
              const int idx = (st * RNT + t0g + u) * 64 + lane;
              b0[u] = Ws[idx];
              b1[u] = Ws[PS + idx];
              b2[u] = Ws[2 * PS + idx];
            }
#pragma unroll
            for (int u = 0; u < GT; ++u) acc[t0g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[st], b0[u], acc[t0g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < GT; ++u) acc[t0g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[st], b1[u], acc[t0g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < GT; ++u) acc[t0g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[st], b0[u], acc[t0g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < GT; ++u) acc[t0g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[st], b2[u], acc[t0g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < GT; ++u) acc[t0g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[st], b1[u], acc[t0g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < GT; ++u) acc[t0g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[st], b0[u], acc[t0g + u], 0, 0, 0);
            // one group's operands at a time (hoisting every group's LDS reads exceeds the registers)
            __builtin_amdgcn_sched_barrier(0);
          }
        // D[4 q + r][n] of column tile tt: row n0 + 4 q + r, column 16 tt + m
        float* cp = Co + (long)(n0 + 4 * q) * g.c_i + m;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n0 + 4 * q + r < g.M) {
#pragma unroll
            for (int tt = 0; tt < NTC; ++tt) __builtin_nontemporal_store(g.alpha * acc[tt][r], cp + 16 * tt);
          }
          cp += g.c_i;
        }
      } else {
#pragma unroll
        for (int st = 0; st < RKS; ++st) {
          if (st >= KS) break;
#pragma unroll
          for (int tt = 0; tt < RNT; ++tt) {
            if (tt >= NT) break;
            const int idx = (st * RNT + tt) * 64 + lane;
            const bf16x8 b0 = Ws[idx], b1 = Ws[PS + idx], b2 = Ws[2 * PS + idx];
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[st], b0, acc[tt], 0, 0, 0);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[st], b1, acc[tt], 0, 0, 0);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[st], b0, acc[tt], 0, 0, 0);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[st], b2, acc[tt], 0, 0, 0);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[st], b1, acc[tt], 0, 0, 0);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[st], b0, acc[tt], 0, 0, 0);
          }
        }
#pragma unroll
        for (int tt = 0; tt < RNT; ++tt) {
          const int j = 16 * tt + m;
          if (tt >= NT || j >= g.N) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = n0 + 4 * q + r;
            if (row < g.M) __builtin_nontemporal_store(g.alpha * acc[tt][r], Co + (long)row * g.c_i + j);
          }
        }
      }
    }
    base = te;
  }
}

// Zeroes p[0, n): 16-byte stores from the first 16-byte boundary on, single
// floats for the head before it and the tail after the last whole vector.
__global__ void fill_zero(float* __restrict__ p, size_t n) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t lead = ((16 - (reinterpret_cast<size_t>(p) & 15)) & 15) / sizeof(float);
  const size_t head = lead < n ? lead : n;
  if (tid < head) p[tid] = 0.0f;
  f32x4* q = reinterpret_cast<f32x4*>(p + head);
  const size_t nq = (n - head) / 4;
  for (size_t i = tid; i < nq; i += stride) q[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const size_t t0 = head + nq * 4;
  if (tid < n - t0) p[t0 + tid] = 0.0f;
}

}  // namespace

hipError_t launch_linear_gemm(const LinearGemm& g, int k_splits, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.num_comp <= 0) return hipSuccess;
  const long gx = (g.M + TM - 1) / TM, gy = (g.N + TN - 1) / TN, gz = (long)g.num_comp * k_splits;
  if (gx > 0x7fffffffL || gy > 65535 || gz > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_gemm, dim3((unsigned)gx, (unsigned)gy, (unsigned)gz), dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_linear_rows(const LinearGemm& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.num_comp <= 0) return hipSuccess;
  if (g.K > 32 * RKS || g.N > 16 * RNT || g.a_k != 1 || g.c_j != 1 || g.b_comp != 0 || g.atomic)
    return hipErrorInvalidValue;
  const long node_tiles = (g.M + 15) / 16, total = node_tiles * g.num_comp;
  if (total > 0x7fffffffL) return hipErrorInvalidValue;
  // one work-group per CU holds a W block; ranges of at least a tile per wave
  long blocks = (total + RW - 1) / RW;
  if (blocks > 256) blocks = 256;
  const long per = (total + blocks - 1) / blocks;
  blocks = (total + per - 1) / per;
  const bool rows_aligned = (g.a_i & 3) == 0 && (g.a_comp & 3) == 0 &&
                            (reinterpret_cast<unsigned long>(g.A) & 15) == 0;
  auto kernel = linear_rows<0, 0>;
  if (rows_aligned && g.K == 128 && g.N == 128) kernel = linear_rows<4, 8>;
  else if (rows_aligned && g.K == 64 && g.N == 64) kernel = linear_rows<2, 4>;
  else if (rows_aligned && g.K == 32 && g.N == 32) kernel = linear_rows<1, 2>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * RW), 0, stream, g, (int)total, (int)per,
                     (int)node_tiles);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t vecs = (n + 3) / 4;
  const size_t blocks = (vecs + 255) / 256 < 8192 ? (vecs + 255) / 256 : 8192;
  hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace e3c
