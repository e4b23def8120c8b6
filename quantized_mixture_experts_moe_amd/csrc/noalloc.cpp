// The whole layer for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// moe_layer_forward with its workspace in a fixed device array of the
// library instead of a caller's buffer.
#include <mutex>

#include "moe_internal.h"

namespace {

// The scratch array: large enough for a 128-token prefill chunk of the
// Gemma-4-26B-A4B-shaped layer (moe_workspace_bytes = 40.1 MiB).  Every GPU
// the library runs on holds its own copy until the process ends.
constexpr size_t kScratchBytes = size_t(48) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device
bool g_cleared[kMaxDevices];    // zero-fill enqueued once on that device

__global__ void zero_fill(uint4 *p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch array's address on the current device, and its first use's
// zero-fill: a kernel on the caller's stream, so it comes before the call's
// own kernels in stream order (and into a graph, if the first call is
// captured: then each replay starts from a cleared array, which the
// workspace's protocol allows).
moe_status scratch_for_call(hipStream_t s, void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_E_HIP;
    g_scratch[dev] = p;
  }
  if (!g_cleared[dev]) {
    zero_fill<<<1024, 256, 0, s>>>((uint4 *)g_scratch[dev], kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return MOE_E_HIP;
    g_cleared[dev] = true;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const void *x, int32_t x_dtype, int32_t T,
                                                const moe_qmat *router, const float *logit_bias,
                                                int32_t k, const moe_bank *routed,
                                                const moe_bank *shared, void *out,
                                                int32_t out_dtype, int32_t *ids_out,
                                                float *gates_out, void *stream) {
  moe::Dims d;
  moe_status st = moe::layer_forward_args(x, x_dtype, T, router, k, routed, shared, nullptr, 0,
                                          out, out_dtype, &d);
  if (st) return st;
  if (moe::workspace_bytes(d) > kScratchBytes) return MOE_E_WORKSPACE;
  void *ws = nullptr;
  st = scratch_for_call((hipStream_t)stream, &ws);
  if (st) return st;
  st = moe_layer_forward(x, x_dtype, T, router, logit_bias, k, routed, shared, nullptr, 0, out,
                         out_dtype, ids_out, gates_out, ws, kScratchBytes, stream);
  if (st == MOE_E_HIP) {
    // a launch failed part way: the next call clears the array again
    int dev = -1;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
      std::lock_guard<std::mutex> lock(g_mu);
      g_cleared[dev] = false;
    }
  }
  return st;
}
