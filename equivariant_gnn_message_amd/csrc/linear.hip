// Output linear (channel mixing within each irrep block) on fp32 MFMA.
//
// cuEquivariance page, Flax NNX layers, IrrepsLinear: matching irreps mix
// their channels, out[..., v, i] = scale / sqrt(mul_in) * sum_u w[u, v] in[..., u, i].
// With trailing channels the convolution output is (N, num_out, C): for each
// output component o (of block k) this is a plain GEMM over the node axis,
//     out[:, o, :] = alpha * in[:, o, :] @ W_k,   W_k (C, C_out),
// and its reverse is two more GEMMs:
//     grad_in[:, o, :] = alpha * grad_out[:, o, :] @ W_k^T,
//     grad_W_k        += alpha * in[:, o, :]^T @ grad_out[:, o, :]  (summed over o in block k).
// One tiled kernel serves all three through element strides: 64 x 64 output
// tiles per work-group of four waves, 32-deep K chunks staged in LDS, each
// wave a 32 x 32 sub-tile of 2 x 2 v_mfma_f32_16x16x4_f32 accumulators
// (fp32 products and sums, as the scalar reference computes them).  The
// reduction over nodes for grad_W is split across work-groups and combined
// with fp32 atomics.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace e3c {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64, TN = 64, TK = 32;

__global__ void __launch_bounds__(256) linear_gemm(LinearGemm g) {
  __shared__ float As[TM][TK + 1];
  __shared__ float Bs[TK][TN + 1];

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
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
  const int lr = lane & 15, lk = lane >> 4;

  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    // Stage A (TM x TK) and B (TK x TN); consecutive threads walk the
    // operand's contiguous axis.
#pragma unroll
    for (int r = 0; r < TM * TK / 256; ++r) {
      const int idx = t + 256 * r;
      int i, k;
      if (g.a_k == 1) { i = idx / TK; k = idx % TK; } else { k = idx / TM; i = idx % TM; }
      const int gi = i0 + i, gk = k0 + k;
      As[i][k] = (gi < g.M && gk < kend) ? A[(long)gi * g.a_i + (long)gk * g.a_k] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < TK * TN / 256; ++r) {
      const int idx = t + 256 * r;
      int k, j;
      if (g.b_j == 1) { k = idx / TN; j = idx % TN; } else { j = idx / TK; k = idx % TK; }
      const int gk = k0 + k, gj = j0 + j;
      Bs[k][j] = (gk < kend && gj < g.N) ? B[(long)gk * g.b_k + (long)gj * g.b_j] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; kk += 4) {
      float av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = As[wr + a * 16 + lr][kk + lk];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = Bs[kk + lk][wc + b * 16 + lr];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }

  // D[4*(lane/16) + r][lane % 16] of each 16 x 16 accumulator
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
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
