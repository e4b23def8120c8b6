// The residual block around the MoE layer: a pre-norm RMSNorm of the
// residual stream feeds the layer, and the layer's output is normalised by a
// post-norm RMSNorm and added back to the residual stream (a Gemma-style
// sandwich; the pages name the normalisation and residual work of a block
// as what a production engine fuses around the experts but do not define it:
// es.news.hada.io, "Alcance de implementacion y registro experimental").
//   u   = round16(x / sqrt(mean(x^2) + eps) * (1 + w_pre))   (the layer's input)
//   out = x + y / sqrt(mean(y^2) + eps) * (1 + w_post)        (y: the layer's output)
// These kernels serve the calls whose layer runs in several launches; the
// one-launch decode layer does both norms itself.  One wave per row, the
// sums of squares in the fixed order of device_common.h, so both give the
// same bits.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row

template <bool F16X>
__global__ __launch_bounds__(64 * kRowsPerBlock) void block_pre_kernel(const uint16_t *x,
                                                                      const float *w, float eps,
                                                                      int T, int D, uint16_t *u) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const int nch = D / 8;
  const u32x4 *xr = (const u32x4 *)(x + (size_t)t * D);
  const float sq = row_sumsq_wave(nch, [&](int c, float (&v)[8]) { unpack8<F16X>(xr[c], v); });
  const float inv = norm_inv(sq, D, eps);
  u32x4 *ur = (u32x4 *)(u + (size_t)t * D);
  const float4 *w4 = (const float4 *)w;
  for (int c = lane; c < nch; c += 64) ur[c] = norm_chunk<F16X>(xr[c], inv, w4[2 * c], w4[2 * c + 1]);
}

template <bool F16X>
__global__ __launch_bounds__(64 * kRowsPerBlock) void block_post_kernel(
    const float *y, const uint16_t *x, const float *w, float eps, int T, int D, void *out,
    int out_dtype) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const int nch = D / 8;
  const float4 *yr = (const float4 *)(y + (size_t)t * D);
  const float sq = row_sumsq_wave(nch, [&](int c, float (&v)[8]) {
    const float4 a = yr[2 * c], b = yr[2 * c + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  });
  const float inv = norm_inv(sq, D, eps);
  const u32x4 *xr = (const u32x4 *)(x + (size_t)t * D);
  const float4 *w4 = (const float4 *)w;
  for (int c = lane; c < nch; c += 64) {
    const float4 a = yr[2 * c], b = yr[2 * c + 1], wa = w4[2 * c], wb = w4[2 * c + 1];
    const float yv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
    float xv[8], r[8];
    unpack8<F16X>(xr[c], xv);
#pragma unroll
    for (int m = 0; m < 8; ++m) r[m] = xv[m] + norm_scale(yv[m], inv, wv[m]);
    const size_t o = (size_t)t * D + 8 * c;
    if (out_dtype == MOE_F32) {
      ((float4 *)((float *)out + o))[0] = float4{r[0], r[1], r[2], r[3]};
      ((float4 *)((float *)out + o))[1] = float4{r[4], r[5], r[6], r[7]};
    } else {
      uint32_t h[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) h[m] = out_dtype == MOE_BF16 ? f32_to_bf16(r[m]) : f32_to_f16(r[m]);
      *(u32x4 *)((uint16_t *)out + o) =
          u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
  }
}

}  // namespace

hipError_t launch_block_pre(const void *x, int f16x, int T, int D, const float *w, float eps,
                            uint16_t *u, hipStream_t s) {
  if (D > kBlockMaxD || D % 8) return hipErrorInvalidValue;
  const dim3 grid((T + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  if (f16x)
    hipLaunchKernelGGL(block_pre_kernel<true>, grid, block, 0, s, (const uint16_t *)x, w, eps, T,
                       D, u);
  else
    hipLaunchKernelGGL(block_pre_kernel<false>, grid, block, 0, s, (const uint16_t *)x, w, eps, T,
                       D, u);
  return hipGetLastError();
}

hipError_t launch_block_post(const float *y, const void *x, int f16x, int T, int D,
                             const float *w, float eps, void *out, int out_dtype, hipStream_t s) {
  if (D > kBlockMaxD || D % 8) return hipErrorInvalidValue;
  const dim3 grid((T + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  if (f16x)
    hipLaunchKernelGGL(block_post_kernel<true>, grid, block, 0, s, y, (const uint16_t *)x, w, eps,
                       T, D, out, out_dtype);
  else
    hipLaunchKernelGGL(block_post_kernel<false>, grid, block, 0, s, y, (const uint16_t *)x, w,
                       eps, T, D, out, out_dtype);
  return hipGetLastError();
}

}  // namespace moe
