// The residual block around the MoE layer: a pre-norm RMSNorm of the
// residual stream feeds the layer, and the layer's output is normalised by a
// post-norm RMSNorm and added back to the residual stream (a Gemma-style
// sandwich; the pages name the normalisation and residual work of a block
// as what a production engine fuses around the experts but do not define it:
// es.news.hada.io, "Alcance de implementacion y registro experimental").
//   u   = round16(x / sqrt(mean(x^2) + eps) * (1 + w_pre))   (the layer's input)
//   out = x + y / sqrt(mean(y^2) + eps) * (1 + w_post)        (y: the layer's output)
// One block per token row.  The sums of squares run in a fixed order (each
// thread over its columns in order, a DPP wave sum, the waves in order), so
// results are bitwise reproducible.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNT = 256;  // threads per row
constexpr int kMaxPer = kBlockMaxD / kNT;

template <bool F16X>
__device__ __forceinline__ float x_val(uint16_t v) {
  return F16X ? f16_to_f32(v) : bf16_to_f32(v);
}

// Sum over the block of one value per thread (fixed order).
__device__ __forceinline__ float block_sum(float v, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

template <bool F16X>
__global__ __launch_bounds__(kNT) void block_pre_kernel(const uint16_t *x, const float *w,
                                                        float eps, int D, uint16_t *u) {
  __shared__ float red[kNT / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint16_t *xr = x + (size_t)t * D;
  float v[kMaxPer];
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = tid + i * kNT;
    v[i] = c < D ? x_val<F16X>(xr[c]) : 0.0f;
    sq = fmaf(v[i], v[i], sq);
  }
  const float inv = 1.0f / sqrtf(block_sum(sq, red) / (float)D + eps);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = tid + i * kNT;
    if (c < D) {
      const float r = v[i] * inv * (1.0f + w[c]);
      u[(size_t)t * D + c] = (uint16_t)(F16X ? f32_to_f16(r) : f32_to_bf16(r));
    }
  }
}

template <bool F16X>
__global__ __launch_bounds__(kNT) void block_post_kernel(const float *y, const uint16_t *x,
                                                         const float *w, float eps, int D,
                                                         void *out, int out_dtype) {
  __shared__ float red[kNT / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float *yr = y + (size_t)t * D;
  float v[kMaxPer];
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = tid + i * kNT;
    v[i] = c < D ? yr[c] : 0.0f;
    sq = fmaf(v[i], v[i], sq);
  }
  const float inv = 1.0f / sqrtf(block_sum(sq, red) / (float)D + eps);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = tid + i * kNT;
    if (c < D) {
      const size_t o = (size_t)t * D + c;
      const float r = x_val<F16X>(x[o]) + v[i] * inv * (1.0f + w[c]);
      if (out_dtype == MOE_F32)
        ((float *)out)[o] = r;
      else if (out_dtype == MOE_BF16)
        ((uint16_t *)out)[o] = (uint16_t)f32_to_bf16(r);
      else
        ((uint16_t *)out)[o] = (uint16_t)f32_to_f16(r);
    }
  }
}

}  // namespace

hipError_t launch_block_pre(const void *x, int f16x, int T, int D, const float *w, float eps,
                            uint16_t *u, hipStream_t s) {
  if (D > kMaxPer * kNT) return hipErrorInvalidValue;
  if (f16x)
    hipLaunchKernelGGL(block_pre_kernel<true>, dim3(T), dim3(kNT), 0, s, (const uint16_t *)x, w,
                       eps, D, u);
  else
    hipLaunchKernelGGL(block_pre_kernel<false>, dim3(T), dim3(kNT), 0, s, (const uint16_t *)x, w,
                       eps, D, u);
  return hipGetLastError();
}

hipError_t launch_block_post(const float *y, const void *x, int f16x, int T, int D,
                             const float *w, float eps, void *out, int out_dtype, hipStream_t s) {
  if (D > kMaxPer * kNT) return hipErrorInvalidValue;
  if (f16x)
    hipLaunchKernelGGL(block_post_kernel<true>, dim3(T), dim3(kNT), 0, s, y, (const uint16_t *)x, w,
                       eps, D, out, out_dtype);
  else
    hipLaunchKernelGGL(block_post_kernel<false>, dim3(T), dim3(kNT), 0, s, y, (const uint16_t *)x,
                       w, eps, D, out, out_dtype);
  return hipGetLastError();
}

}  // namespace moe
