// Receiver CSR, streaming references and the layout registry.
#include "conv_kernels.h"

namespace e3c {
namespace {

// ------------------------------------------------------- graph utilities ----

__global__ void csr_kernel(const int* __restrict__ dst, int num_edges, int num_nodes,
                           int* __restrict__ row_ptr) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > num_nodes) return;
  int lo = 0, hi = num_edges;
  while (lo < hi) {
    const int mid = (int)(((unsigned)lo + (unsigned)hi) >> 1);
    if (dst[mid] < b) lo = mid + 1; else hi = mid;
  }
  row_ptr[b] = lo;
}

// Streaming references.  Each work-group moves one contiguous chunk and exits,
// so the resident work-groups cover a narrow, steadily advancing address
// window; on MI355X this runs well ahead of grid-stride loops over the whole
// buffer (measured 7.0 vs 6.2 TB/s read-only, 5.9 vs 5.1 TB/s copy).
constexpr int kStreamPerBlock = 1024;   // 16-byte elements per work-group (16 KiB)

__global__ void __launch_bounds__(256) stream_copy_kernel(const f32x4* __restrict__ src,
                                                         f32x4* __restrict__ dst, size_t n4) {
  const size_t beg = (size_t)blockIdx.x * kStreamPerBlock;
  const size_t end = beg + kStreamPerBlock < n4 ? beg + kStreamPerBlock : n4;
  f32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t i = beg + threadIdx.x + u * 256;
    if (i < end) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t i = beg + threadIdx.x + u * 256;
    if (i < end) __builtin_nontemporal_store(v[u], dst + i);
  }
}

// Written only if a lane's sum equals 1234.5678f (never for the calibration
// data): keeps the read-only pass's loads alive without touching its input.
__device__ float stream_sink;

__global__ void __launch_bounds__(256) stream_read_kernel(const f32x4* __restrict__ src, size_t n4) {
  const size_t beg = (size_t)blockIdx.x * (2 * kStreamPerBlock);
  const size_t end = beg + 2 * kStreamPerBlock < n4 ? beg + 2 * kStreamPerBlock : n4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = beg + threadIdx.x; i < end; i += 4 * 256) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t k = i + u * 256;
      if (k < end) acc += __builtin_nontemporal_load(src + k);
    }
  }
  const float v = acc.x + acc.y + acc.z + acc.w;
  if (v == 1234.5678f) stream_sink = v;
}

}  // namespace

hipError_t launch_stream(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const size_t n4 = bytes / 16;
  if (n4 == 0) return hipSuccess;
  const size_t per = dst ? kStreamPerBlock : 2 * kStreamPerBlock;
  const size_t blocks = (n4 + per - 1) / per;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  if (dst) {
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n4);
  } else {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const f32x4*>(src), n4);
  }
  return hipGetLastError();
}

const KernelSet* find_kernels(int channels, uint32_t xcode, int lmax, uint32_t ocode) {
  const KernelSet* const kSets[] = {kernels_tiny(), kernels_gate(), kernels_mace(), kernels_big()};
  for (const KernelSet* k : kSets)
    if (k->channels == channels && k->xcode == xcode && k->lmax == lmax && k->ocode == ocode) return k;
  return nullptr;
}

hipError_t launch_csr_from_receivers(const int* dst, int num_edges, int num_nodes, int* row_ptr,
                                     hipStream_t stream) {
  const unsigned blocks = (unsigned)((num_nodes + 1 + 255) / 256);
  hipLaunchKernelGGL(csr_kernel, dim3(blocks), dim3(256), 0, stream, dst, num_edges, num_nodes,
                     row_ptr);
  return hipGetLastError();
}

}  // namespace e3c
