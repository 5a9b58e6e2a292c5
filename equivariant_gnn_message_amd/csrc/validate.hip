// Graph checks (e3j Convolution page, __call__: sender and receiver indices lie
// in [0, num_nodes), and the fused kernels need the edges sorted by receiver,
// i.e. a valid receiver CSR).  Host check, and three device forms:
//   e3conv_validate_graph(on_device = 1)   synchronous, allocates its result;
//   e3conv_validate_graph_async            caller-owned result, asynchronous;
//   e3conv_validate_graph_noalloc          synchronous, result in a static
//                                          device array (allocates nothing).
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <string>
#include <vector>

#include "e3conv.h"
#include "kernels.h"

namespace e3c {
namespace {

// result[0]: number of violations; result[1]: first index i with row_ptr[i]
// outside [0, num_edges] (or != 0 at i = 0, != num_edges at i = num_nodes) or
// row_ptr[i + 1] < row_ptr[i] (INT_MAX if none); result[2]: first edge whose
// sender is out of range (INT_MAX if none); result[3]: 0.
__global__ void validate_init(int* __restrict__ r) {
  const int t = (int)threadIdx.x;
  if (t < kValidateResultInts) r[t] = (t == 1 || t == 2) ? INT_MAX : 0;
}

__global__ void validate_kernel(const int* __restrict__ src, const int* __restrict__ row_ptr,
                                int num_nodes, int num_edges, int* __restrict__ r) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i <= num_nodes) {
    const int v = row_ptr[i];
    bool ok = v >= 0 && v <= num_edges;
    if (i == 0) ok = ok && v == 0;
    if (i == num_nodes) ok = ok && v == num_edges;
    if (i < num_nodes) ok = ok && row_ptr[i + 1] >= v;
    if (!ok) {
      atomicAdd(r, 1);
      atomicMin(r + 1, (int)i);
    }
  }
  if (i < num_edges) {
    const int a = src[i];
    if (a < 0 || a >= num_nodes) {
      atomicAdd(r, 1);
      atomicMin(r + 2, (int)i);
    }
  }
}

// Result array of e3conv_validate_graph_noalloc.  One copy per device, held
// until the process ends.  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) int scratch[kValidateResultInts];

std::mutex g_scratch_mu;
std::vector<int*> g_scratch_ptr;   // per device id; nullptr until looked up

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
hipError_t scratch_address(int** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<int*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_validate(const int* src, const int* row_ptr, int num_nodes, int num_edges, int* r,
                           hipStream_t stream) {
  hipLaunchKernelGGL(validate_init, dim3(1), dim3(64), 0, stream, r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long n = (num_nodes + 1L > num_edges ? num_nodes + 1L : (long)num_edges);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(256), 0, stream, src, row_ptr, num_nodes,
                     num_edges, r);
  return hipGetLastError();
}

e3conv_status check_args(const int32_t* src, const int32_t* row_ptr, int64_t N, int64_t E) {
  if (N < 0 || E < 0) return api_fail(E3CONV_ERR_INVALID_ARGUMENT, "negative size");
  if (E >= (int64_t)1 << 31 || N >= ((int64_t)1 << 31) - 1)
    return api_fail(E3CONV_ERR_INVALID_ARGUMENT, "sizes must fit int32 indices");
  if (!row_ptr || (E > 0 && !src)) return api_fail(E3CONV_ERR_INVALID_ARGUMENT, "NULL pointer");
  return E3CONV_OK;
}

// Status and detail from a result read back to the host.
e3conv_status report(const int (&r)[kValidateResultInts]) {
  if (r[0] == 0) return api_ok();
  std::string msg = std::to_string(r[0]) + " violations in the graph";
  if (r[1] != INT_MAX) msg += "; first at row_ptr index " + std::to_string(r[1]);
  if (r[2] != INT_MAX) msg += "; first out-of-range sender at edge " + std::to_string(r[2]);
  return api_fail(E3CONV_ERR_GRAPH, msg);
}

}  // namespace
}  // namespace e3c

extern "C" {

e3conv_status e3conv_validate_graph(const int32_t* src, const int32_t* row_ptr, int64_t N,
                                    int64_t E, int on_device) {
  e3conv_status st = e3c::check_args(src, row_ptr, N, E);
  if (st != E3CONV_OK) return st;
  if (!on_device) {
    // the device check's definition, first offending index of each kind
    int r[e3c::kValidateResultInts] = {0, INT_MAX, INT_MAX, 0};
    for (int64_t i = 0; i <= N; ++i) {
      const int64_t v = row_ptr[i];
      bool ok = v >= 0 && v <= E;
      if (i == 0) ok = ok && v == 0;
      if (i == N) ok = ok && v == E;
      if (i < N) ok = ok && row_ptr[i + 1] >= v;
      if (!ok) {
        ++r[0];
        if (r[1] == INT_MAX) r[1] = (int)i;
      }
    }
    for (int64_t e = 0; e < E; ++e)
      if (src[e] < 0 || src[e] >= N) {
        ++r[0];
        if (r[2] == INT_MAX) r[2] = (int)e;
      }
    return e3c::report(r);
  }
  int* r = nullptr;
  hipError_t err = hipMalloc(&r, sizeof(int) * e3c::kValidateResultInts);
  if (err != hipSuccess) return e3c::api_hip_fail(err, "hipMalloc");
  int host[e3c::kValidateResultInts] = {};
  err = e3c::launch_validate(src, row_ptr, (int)N, (int)E, r, nullptr);
  if (err == hipSuccess) err = hipMemcpy(host, r, sizeof(host), hipMemcpyDeviceToHost);
  const hipError_t ferr = hipFree(r);
  if (err == hipSuccess) err = ferr;
  if (err != hipSuccess) return e3c::api_hip_fail(err, "validate");
  return e3c::report(host);
}

e3conv_status e3conv_validate_graph_async(const int32_t* src, const int32_t* row_ptr, int64_t N,
                                          int64_t E, int32_t* result, void* stream) {
  e3conv_status st = e3c::check_args(src, row_ptr, N, E);
  if (st != E3CONV_OK) return st;
  if (!result) return e3c::api_fail(E3CONV_ERR_INVALID_ARGUMENT, "result is NULL");
  const hipError_t err =
      e3c::launch_validate(src, row_ptr, (int)N, (int)E, result, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return e3c::api_hip_fail(err, "validate launch");
  return e3c::api_ok();
}

e3conv_status e3conv_validate_graph_noalloc(const int32_t* src, const int32_t* row_ptr, int64_t N,
                                            int64_t E, void* stream) {
  e3conv_status st = e3c::check_args(src, row_ptr, N, E);
  if (st != E3CONV_OK) return st;
  int* r = nullptr;
  hipError_t err = e3c::scratch_address(&r);
  if (err != hipSuccess) return e3c::api_hip_fail(err, "scratch address");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int host[e3c::kValidateResultInts] = {};
  // the first kernel of launch_validate resets the array before the check writes it
  err = e3c::launch_validate(src, row_ptr, (int)N, (int)E, r, s);
  if (err == hipSuccess) err = hipMemcpyAsync(host, r, sizeof(host), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return e3c::api_hip_fail(err, "validate");
  return e3c::report(host);
}

}  // extern "C"
