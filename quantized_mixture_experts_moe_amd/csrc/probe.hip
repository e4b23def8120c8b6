// Streaming read probe: a measurement helper, not a step of the method.  It
// reads a device buffer once with 16-byte loads, eight in flight per thread,
// and writes one word per block, so that its duration gives the rate at which
// this chip streams reads from HBM; the benchmark reports the layer kernels'
// achieved bytes per second against that measured rate as well as against
// the 8 TB/s datasheet figure.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  const gptr<u32x4> g = as_global(src);
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = g[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = g[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per block (the xor of the block's words), so the loads are used
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t s[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                                     int32_t blocks, void *stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15u) || bytes % 16 || blocks < 1 || blocks > 65536)
    return MOE_E_INVALID;
  hipLaunchKernelGGL(moe::read_probe_kernel, dim3(blocks), dim3(moe::kProbeThreads), 0,
                     (hipStream_t)stream, (const moe::u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}
