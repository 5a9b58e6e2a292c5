// Output linear (channel mixing within each irrep block) on fp32 MFMA.
//
// cuEquivariance page, Flax NNX layers, IrrepsLinear: within each irrep block
// the channels are mixed, out[..., v, i] = scale / sqrt(mul_in) * sum_u w[u, v] in[..., u, i].
// With trailing channels the convolution output is (N, num_out, C): for each
// output component o (of block k) this is a plain GEMM over the node axis,
//     out[:, o, :] = alpha * in[:, o, :] @ W_k,   W_k (C, C_out),
// and its reverse is two more GEMMs:
//     grad_in[:, o, :] = alpha * grad_out[:, o, :] @ W_k^T,
//     grad_W_k        += alpha * in[:, o, :]^T @ grad_out[:, o, :]  (summed over o in block k).
// One tiled kernel serves all three through element strides: 64 x 128 output
// tiles per work-group of four waves (128 columns cover C_out <= 128 in one
// tile, so each input row is read from memory once), 32-deep K chunks staged
// in LDS, each wave a 64 x 32 slab of 4 x 2 v_mfma_f32_16x16x4_f32
// accumulators (fp32 products and sums, as the scalar reference computes them).  The
// reduction over nodes for grad_W is split across work-groups and combined
// with fp32 atomics.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace e3c {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64, TN = 128, TK = 32;
constexpr int MT = TM / 16;   // 16-row MFMA tiles per wave

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
  const int wc = w * 32;
  const int lr = lane & 15, lk = lane >> 4;

  f32x4 acc[MT][2];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging map: thread t always loads the same (row, column) slots of the
  // A and B tiles, so their element offsets (32-bit: the tensors hold fewer
  // than 2^31 elements) are computed once; each K chunk only adds k0 * stride.
  // Consecutive threads walk the operand's contiguous axis.
  constexpr int RA = TM * TK / 256, RB = TK * TN / 256;
  const bool a_rows = g.a_k == 1;      // A contiguous along k: thread keeps k, walks rows
  const bool b_cols = g.b_j == 1;      // B contiguous along j: thread keeps j, walks k
  int a_off[RA], a_i[RA], a_k[RA];
  bool a_ok[RA];
#pragma unroll
  for (int r = 0; r < RA; ++r) {
    const int idx = t + 256 * r;
    a_i[r] = a_rows ? idx / TK : idx % TM;
    a_k[r] = a_rows ? idx % TK : idx / TM;
    a_ok[r] = i0 + a_i[r] < g.M;
    a_off[r] = a_ok[r] ? (int)((long)(i0 + a_i[r]) * g.a_i + (long)a_k[r] * g.a_k) : 0;
  }
  int b_off[RB], b_k[RB], b_j[RB];
  bool b_ok[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int idx = t + 256 * r;
    b_k[r] = b_cols ? idx / TN : idx % TK;
    b_j[r] = b_cols ? idx % TN : idx / TK;
    b_ok[r] = j0 + b_j[r] < g.N;
    b_off[r] = b_ok[r] ? (int)((long)b_k[r] * g.b_k + (long)(j0 + b_j[r]) * g.b_j) : 0;
  }

  // Out-of-range slots load a valid element (offset 0 of the chunk: row or
  // column k0 exists) and are then replaced by zero, so the loads need no
  // branches.  The next chunk's elements are loaded into registers while the
  // current chunk is multiplied.
  float ra[RA], rb[RB];
  auto fetch = [&](int k0) {
    const float* Ak = A + (long)k0 * g.a_k;
    const float* Bk = B + (long)k0 * g.b_k;
#pragma unroll
    for (int r = 0; r < RA; ++r) {
      const bool ok = a_ok[r] && k0 + a_k[r] < kend;
      const float v = Ak[ok ? a_off[r] : 0];
      ra[r] = ok ? v : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const bool ok = b_ok[r] && k0 + b_k[r] < kend;
      const float v = Bk[ok ? b_off[r] : 0];
      rb[r] = ok ? v : 0.0f;
    }
  };
  if (kbeg < kend) fetch(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
#pragma unroll
    for (int r = 0; r < RA; ++r) As[a_i[r]][a_k[r]] = ra[r];
#pragma unroll
    for (int r = 0; r < RB; ++r) Bs[b_k[r]][b_j[r]] = rb[r];
    __syncthreads();
    if (k0 + TK < kend) fetch(k0 + TK);
#pragma unroll
    for (int kk = 0; kk < TK; kk += 4) {
      float av[MT], bv[2];
#pragma unroll
      for (int a = 0; a < MT; ++a) av[a] = As[a * 16 + lr][kk + lk];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = Bs[kk + lk][wc + b * 16 + lr];
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }

  // D[4*(lane/16) + r][lane % 16] of each 16 x 16 accumulator
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = i0 + a * 16 + 4 * lk + r;
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
