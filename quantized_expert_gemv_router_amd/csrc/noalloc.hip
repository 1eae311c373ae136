// moe_expert_stack_decode without caller-provided workspace and without any
// allocation: the workspace lives in a file-scope device array, one copy per
// GPU, whose address is taken once per device with hipGetSymbolAddress.
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
#include <hip/hip_runtime.h>

#include <mutex>

#include "moeq.h"
#include "moeq_internal.hpp"

namespace moeq {
namespace {

constexpr int64_t kNoAllocBytes = MOEQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The scratch workspace.  In host code this name is only a stand-in for the
// symbol: kernels are given the device address held in g_scratch[device].
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];

__global__ void zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Hands the status word to the caller (if asked) and clears it for the next call.
__global__ void take_status_kernel(int32_t* word, int32_t* out) {
  if (threadIdx.x == 0) {
    const int32_t v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (out) *out = v;
    __hip_atomic_store(word, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// This device's scratch address; on the first call for the device, with it
// current, the symbol's address is taken and the array cleared on `stream`.
int device_scratch(hipStream_t stream, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOEQ_E_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(p), kNoAllocBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
    g_scratch[dev] = p;
  }
  *out = static_cast<char*>(g_scratch[dev]);
  return MOEQ_OK;
}

}  // namespace
}  // namespace moeq

using namespace moeq;

extern "C" int moe_expert_stack_decode_noalloc(const moeq_shape* s, const moeq_experts* ex,
                                               const uint16_t* const* w_router, int layer0, int L, int T, int k,
                                               uint32_t flags, float* h, int32_t* topk_trace, float* h_trace,
                                               int32_t* status_out, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (T < 0 || k < 0) return fail(MOEQ_E_INVALID, "T=%d k=%d must be non-negative", T, k);
  if (T > MOEQ_MAX_DECODE_TOKENS || k > MOEQ_MAX_TOPK || k > s->n_experts)
    return fail(MOEQ_E_UNSUPPORTED, "T=%d k=%d outside the decode limits", T, k);
  const int64_t need = workspace_layout(*s, T, k).total;
  if (need > kNoAllocBytes)
    return fail(MOEQ_E_UNSUPPORTED,
                "workspace for hidden=%d inter=%d n_experts=%d T=%d k=%d is %lld bytes, above the "
                "%lld-byte static scratch of the allocation-free entry point",
                s->hidden, s->inter, s->n_experts, T, k, (long long)need, (long long)kNoAllocBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = nullptr;
  if (int rc = device_scratch(st, &ws)) return rc;
  int rc = moe_expert_stack_decode(s, ex, w_router, layer0, L, T, k, flags, h, topk_trace, h_trace, ws, stream);
  if (rc != MOEQ_OK) return rc;
  int32_t* status = reinterpret_cast<int32_t*>(ws + workspace_layout(*s, T, k).counters) + kCounterStatus;
  hipLaunchKernelGGL(take_status_kernel, dim3(1), dim3(64), 0, st, status, status_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "status hand-off launch");
  return ok();
}
