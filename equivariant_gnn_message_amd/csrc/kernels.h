// Device-kernel registry: one set of fused kernels per compiled irrep layout.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <string>

#include "e3conv.h"
#include "layout.h"

namespace e3c {

struct FwdParams {
  const void* x;        // (N, NX, C) f32 or bf16 bits
  const void* y;        // (E, NY)
  const void* s;        // (E, NP, C)
  const int* src;       // (E)
  const int* row_ptr;   // (N+1)
  const int* order;     // (N) receiver processing order, or nullptr for 0..N-1
  float* out;           // (N, NO, C)
  int num_nodes;
  int num_edges;
  float inv_avg;
  int num_real;         // receivers b >= num_real are padding: zero rows, no messages
  const float* lin_w;   // fused output linear: (blocks, C, C) weights, or unused
  float lin_alpha;      // its factor scale / sqrt(C) / N
  const int* emap;      // pair-stored rows: (E) pair of each edge, ~pair when reversed; or unused
};

struct BwdParams {
  const float* x;
  const float* y;
  const float* s;
  const int* src;
  const int* row_ptr;
  const int* order;     // (N) or nullptr
  const float* g;       // (N, NO, C) cotangent of out
  float* gx;            // (N, NX, C), zeroed by the launcher then accumulated
  float* gy;            // (E, NY)
  float* gs;            // (E, NP, C)
  int num_nodes;
  int num_edges;
  float inv_avg;
  int num_real;         // edges into receivers b >= num_real get zero grad_y / grad_s
  int flags;            // kAccumulate*: add into the output instead of overwriting it
  int tiles;            // edge ranges of the edge-tiled kernel (set by its launcher)
  const int* dst;       // pair-stored pass: (E) receiver of each stored edge, else unused
};

// BwdParams::flags.  Only the general reverse launchers honour them and
// nullptr outputs (an output that is not computed).
constexpr int kAccumulateX = 1, kAccumulateY = 2, kAccumulateS = 4;

struct JvpParams {
  const void* x;        // primal operands, as in FwdParams
  const void* y;
  const void* s;
  const void* dx;       // tangents, same shapes and dtype as x, y, s
  const void* dy;
  const void* ds;
  const int* src;
  const int* row_ptr;
  const int* order;
  float* out;           // (N, NO, C) primal output, or nullptr
  float* out_dot;       // (N, NO, C) tangent output
  int num_nodes;
  int num_edges;
  float inv_avg;
  int num_real;
};

// Convolution with the edge scalars computed per edge from its length:
// s[e] = silu(f(r[e]) W1) W2, f the Gaussian radial basis times the cosine
// cutoff (centers k r_max / (num_basis - 1), width sigma).
struct RadialParams {
  const float* x;       // (N, NX, C)
  const float* y;       // (E, NY)
  const float* r;       // (E) edge lengths
  const float* w1;      // (num_basis, hidden) row-major
  const float* w2;      // (hidden, NP * C) row-major; column p * C + c is s[., p, c]
  const int* src;
  const int* row_ptr;
  const int* order;     // (N) or nullptr
  float* out;           // (N, NO, C)
  int num_nodes;
  int num_edges;
  float inv_avg;
  int num_real;
  int num_basis;        // <= 8
  int hidden;           // multiple of 4, <= 128
  float r_max;
  float sigma;
};

using FwdLauncher = hipError_t (*)(const FwdParams&, hipStream_t);
using RadialLauncher = hipError_t (*)(const RadialParams&, hipStream_t);
using BwdLauncher = hipError_t (*)(const BwdParams&, hipStream_t);
using JvpLauncher = hipError_t (*)(const JvpParams&, hipStream_t);

// Kernels of one graph ordering: RECEIVER (edges grouped by receiver, x
// gathered at the sender) or SENDER (edges grouped by sender, x gathered at
// the receiver, odd-l edge-feature blocks negated: the reverse edge's
// features under the graded symmetry y_ab = (-1)^l y_ba).
struct OrderingKernels {
  const FwdLauncher* fwd_f32;   // variant lists, [0] is the default
  int n_fwd_f32;
  const FwdLauncher* fwd_bf16;
  int n_fwd_bf16;
  const BwdLauncher* bwd_f32;
  int n_bwd_f32;
  BwdLauncher bwd_f32_general;  // optional outputs and accumulation
  JvpLauncher jvp_f32;
  JvpLauncher jvp_bf16;
  RadialLauncher radial_f32;    // nullptr: no radial-scalar kernel for this layout
  BwdLauncher bwd_pairs_f32;    // pair-stored reverse pass, or nullptr
  FwdLauncher fwd_lin_f32;      // forward with the output linear fused, or nullptr
  FwdLauncher fwd_lin_bf16;
  FwdLauncher fwd_pairs_f32;    // forward reading pair-stored y and s, or nullptr
};

struct KernelSet {
  int channels;
  uint32_t xcode;
  int lmax;
  uint32_t ocode;
  const LayoutTables* tables;   // path / pattern enumeration the kernels use
  const float* cg_values;       // compile-time CG values, one per pattern entry
  OrderingKernels receiver;
  OrderingKernels sender;
};

// Returns nullptr if no kernels are compiled for the layout.
const KernelSet* find_kernels(int channels, uint32_t xcode, int lmax, uint32_t ocode);

// One per compiled layout (defined in the layout_*.hip files).
const KernelSet* kernels_tiny();
const KernelSet* kernels_gate();
const KernelSet* kernels_mace();
const KernelSet* kernels_big();

// One strided GEMM per output component o (blockIdx.z), optionally split
// along K: C_o(i, j) (+)= alpha * sum_k A_o(i, k) B_o(k, j), with
// A_o(i, k) = A[o*a_comp + i*a_i + k*a_k], B_o(k, j) = B[o*b_comp + blk(o)*b_block +
// k*b_k + j*b_j], C_o(i, j) = C[o*c_comp + blk(o)*c_block + i*c_i + j*c_j].
constexpr int kMaxLinearComponents = 128;
struct LinearGemm {
  const float* A;
  long a_i, a_k, a_comp;
  const float* B;
  long b_k, b_j, b_comp, b_block;
  float* C;
  long c_i, c_j, c_comp, c_block;
  int M, N, K;
  int k_chunk;          // K range of one split (a multiple of 32 when split)
  int num_comp;
  int atomic;           // 1: atomic add (K split), 0: store
  float alpha;
  int comp_block[kMaxLinearComponents];
};

hipError_t launch_linear_gemm(const LinearGemm& g, int k_splits, hipStream_t stream);
// Rows variant for B shared by the components of an irrep block (b_comp == 0),
// A contiguous along k, K <= 128, N <= 128, stores (no K split).
hipError_t launch_linear_rows(const LinearGemm& g, hipStream_t stream);
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t stream);

// Streaming reference kernels (copy when dst != nullptr, else read only).
hipError_t launch_stream(const void* src, void* dst, size_t bytes, hipStream_t stream);

hipError_t launch_csr_from_receivers(const int* dst, int num_edges, int num_nodes, int* row_ptr,
                                     hipStream_t stream);

// Ints of a graph-check result: violation count, first bad row_ptr index,
// first edge with an out-of-range sender, reserved.
constexpr int kValidateResultInts = 4;

// Status reporting of the C ABI (the thread's last-error detail), shared by
// the source files that implement entry points.
e3conv_status api_fail(e3conv_status st, const std::string& msg);
e3conv_status api_ok();
e3conv_status api_hip_fail(hipError_t err, const char* what);

}  // namespace e3c
