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
// One tiled kernel serves all three through element strides: 128 x 128 output
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
  if (kbeg < kend) fetch(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    stage();
    __syncthreads();
    if (k0 + TK < kend) fetch(k0 + TK);
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

__global__ void linear_fill_zero(float* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_linear_gemm(const LinearGemm& g, int k_splits, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.num_comp <= 0) return hipSuccess;
  const long gx = (g.M + TM - 1) / TM, gy = (g.N + TN - 1) / TN, gz = (long)g.num_comp * k_splits;
  if (gx > 0x7fffffffL || gy > 65535 || gz > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_gemm, dim3((unsigned)gx, (unsigned)gy, (unsigned)gz), dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  hipLaunchKernelGGL(linear_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace e3c
