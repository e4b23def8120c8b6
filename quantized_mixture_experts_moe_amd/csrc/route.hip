// Router GEMV (8-bit affine, group 64), top-k selection and softmax gates.
//
// The router scores every expert of the layer from the resident 8-bit router
// weights and the top 8 expert IDs drive the rest of the layer
// (es.news.hada.io, "Proceso de generacion de tokens"; imasters.com.br,
// "O truque").  One kernel: blocks of ROWS experts x TT tokens compute the
// logits; the last block of a token group to finish (a counter in the
// workspace) selects the top k and computes the gates, so decode needs a
// single launch for routing.  Block (0, *) also writes the activations in the
// pair layout the 4-bit expert kernels read (dot2 pairs and 64-column sums).
#include <float.h>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <bool F16X>
__device__ __forceinline__ float x_to_f32(uint16_t v) {
  return F16X ? f16_to_f32(v) : bf16_to_f32(v);
}

// Top-k over logits[0..E) of one token by one wave (see topk_regs); writes
// ids, gates and optionally the blob address of every selected expert.
template <int NV>
__device__ void topk_wave_t(const float *lg, int E, int k, int32_t *ids, float *gates,
                            const void *const *table, const void **slot_blob, uint2 *xch) {
  const int lane = threadIdx.x & 63;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int idx = lane + 64 * j;
    v[j] = idx < E ? ld_dev(lg + idx) : -INFINITY;
  }
  int32_t id;
  float gate;
  topk_regs(v, k, xch, &id, &gate);
  if (lane < k) {
    ids[lane] = id;
    gates[lane] = gate;
    if (slot_blob) slot_blob[lane] = table[id];
  }
}
__device__ void topk_wave(const float *lg, int E, int k, int32_t *ids, float *gates,
                          const void *const *table, const void **slot_blob, uint2 *xch) {
  if (E <= 128)
    topk_wave_t<2>(lg, E, k, ids, gates, table, slot_blob, xch);
  else if (E <= 256)
    topk_wave_t<4>(lg, E, k, ids, gates, table, slot_blob, xch);
  else if (E <= 512)
    topk_wave_t<8>(lg, E, k, ids, gates, table, slot_blob, xch);
  else
    topk_wave_t<16>(lg, E, k, ids, gates, table, slot_blob, xch);
}

// Activations [nt][D] of fp16/bf16 bits into LDS as fp32: every thread issues
// its 16-byte loads first (clamped in range), then converts.
template <bool F16X, int NV>
__device__ __forceinline__ void stage_x(const uint16_t *x, int n_elems, float *sx) {
  const int nv = n_elems / 8;
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = min((int)threadIdx.x + i * kThreads, nv - 1);
    v[i] = *(const u32x4 *)(x + (size_t)idx * 8);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    if (idx < nv) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        sx[idx * 8 + 2 * m] = x_to_f32<F16X>(w[m] & 0xFFFFu);
        sx[idx * 8 + 2 * m + 1] = x_to_f32<F16X>(w[m] >> 16);
      }
    }
  }
}

template <bool F16X, int ROWS, int TT, int MAXC>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteLaunch a) {
  constexpr int KL = kThreads / ROWS;  // lanes splitting the reduction
  extern __shared__ float smem[];
  const int D = a.D, E = a.E;
  const int nch = D / 16;  // 16 eight-bit codes per chunk
  float *sx = smem;                  // [TT][D]
  float *sxs = sx + TT * D;          // [TT][D/16] chunk sums
  float *red = sxs + TT * nch;       // [KL][ROWS*TT]
  __shared__ int s_last;
  __shared__ uint2 s_xch[TT][128];  // top-k exchange, one area per selecting wave

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.y * TT;
  // clear the counters of the kernel that follows (visible to it at the launch
  // boundary)
  if (a.zero && blockIdx.y == 0) {
    for (int i = blockIdx.x * kThreads + tid; i < a.zero_words; i += gridDim.x * kThreads)
      a.zero[i] = 0u;
    for (int i = blockIdx.x * kThreads + tid; i < a.zero2_count; i += gridDim.x * kThreads)
      a.zero2[(size_t)i * a.zero2_stride] = 0u;
  }
  const int nt = min(TT, a.T - t0);
  const uint16_t *x = (const uint16_t *)a.x + (size_t)t0 * D;

  // router codes of this thread: chunks kl, kl + KL, ... (loads issued first)
  const int r = tid % ROWS, kl = tid / ROWS;
  const int e = min(blockIdx.x * ROWS + r, E - 1);
  u32x4 q[MAXC];
  uint32_t mw[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = min(kl + i * KL, nch - 1);
    q[i] = as_global((const u32x4 *)a.codes)[(size_t)c * E + e];
    mw[i] = as_global(a.meta)[(size_t)(c >> 2) * E + e];
  }
  stage_x<F16X, (TT * 8192 / 8 + kThreads - 1) / kThreads>(x, nt * D, sx);
  for (int i = nt * D + tid; i < TT * D; i += kThreads) sx[i] = 0.0f;
  __syncthreads();
  for (int i = tid; i < TT * nch; i += kThreads) {
    const float *p = sx + (size_t)i * 16;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += p[j];
    sxs[i] = s;
  }
  {
    // activations for the 4-bit expert kernels (dot2 pairs and 64-column
    // sums), split over the router blocks; the fp32 copy in LDS converts back
    // to the original 16-bit pattern exactly
    const int words = D / 8, groups = D / 64;
    const int w0 = blockIdx.x * words / gridDim.x, w1 = (blockIdx.x + 1) * words / gridDim.x;
    for (int i = tid; i < nt * (w1 - w0); i += kThreads) {
      const int tt = i / (w1 - w0), w = w0 + i - tt * (w1 - w0);
      const float *xv = sx + (size_t)tt * D + 8 * w;
      uint32_t *o = a.xp + (size_t)(t0 + tt) * (D / 2) + 4 * w;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = F16X ? f32_to_f16(xv[m]) : (__float_as_uint(xv[m]) >> 16);
        const uint32_t hi = F16X ? f32_to_f16(xv[m + 4]) : (__float_as_uint(xv[m + 4]) >> 16);
        o[m] = lo | (hi << 16);
      }
    }
    // 64-column sums: 8 threads per group, 8 columns each (sum8_lanes order)
    const int q0 = blockIdx.x * groups / gridDim.x, q1 = (blockIdx.x + 1) * groups / gridDim.x;
    for (int i = tid; i < nt * (q1 - q0) * 8; i += kThreads) {
      const int gi = i / 8, c = i - gi * 8;
      const int tt = gi / (q1 - q0), g = q0 + gi - tt * (q1 - q0);
      const float *xv = sx + (size_t)tt * D + 64 * g + 8 * c;
      float s8 = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s8 += xv[j];
      const float s = sum8_lanes(s8);
      if (c == 0) a.xs[(size_t)(t0 + tt) * (D / 64) + g] = s;
    }
  }
  __syncthreads();

  float acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = kl + i * KL;
    if (c >= nch) break;
    const float sc = f16_to_f32(mw[i]), bi = f16_to_f32(mw[i] >> 16);
    const uint32_t w[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
    float qf[16];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b) qf[u * 4 + b] = (float)((w[u] >> (8 * b)) & 0xFFu);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float *xv = sx + tt * D + c * 16;
      float d = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) d = fmaf(xv[jj], qf[jj], d);
      acc[tt] = fmaf(sc, d, acc[tt]);
      acc[tt] = fmaf(bi, sxs[tt * nch + c], acc[tt]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) red[kl * (ROWS * TT) + tt * ROWS + r] = acc[tt];
  __syncthreads();

  if (wave == 0) {
    if (lane < ROWS * TT) {
      const int tt = lane / ROWS, rr = lane - tt * ROWS;
      const int ee = blockIdx.x * ROWS + rr;
      float s = 0.0f;
      for (int jj = 0; jj < KL; ++jj) s += red[jj * (ROWS * TT) + lane];
      if (ee < E && tt < nt) {
        if (a.logit_bias) s += a.logit_bias[ee];
        st_dev(a.logits + (size_t)(t0 + tt) * E + ee, s);
      }
    }
    wait_all_memory();
    uint32_t old = 0;
    if (lane == 0) old = add_dev(&a.counters[blockIdx.y], 1u);
    old = __shfl(old, 0, 64);
    if (lane == 0) s_last = (old == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (wave < nt) {
    const int t = t0 + wave;
    topk_wave(a.logits + (size_t)t * E, E, a.k, a.ids + (size_t)t * a.k,
              a.gates + (size_t)t * a.k, a.table,
              a.slot_blob ? a.slot_blob + (size_t)t * a.k : nullptr, s_xch[wave]);
  }
  if (tid == 0) st_dev(&a.counters[blockIdx.y], 0u);
}

template <bool F16X, int ROWS, int TT, int MAXC>
hipError_t launch_route_t(const RouteLaunch &a, hipStream_t s) {
  const int nch = a.D / 16;
  if ((nch + kThreads / ROWS - 1) / (kThreads / ROWS) > MAXC || a.D > 8192 || a.D % 64)
    return hipErrorInvalidValue;
  const size_t smem = sizeof(float) * ((size_t)TT * a.D + (size_t)TT * nch +
                                       (size_t)(kThreads / ROWS) * ROWS * TT);
  dim3 grid((a.E + ROWS - 1) / ROWS, (a.T + TT - 1) / TT);
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void *)route_kernel<F16X, ROWS, TT, MAXC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((route_kernel<F16X, ROWS, TT, MAXC>), grid, dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

template <bool F16X>
__global__ __launch_bounds__(256) void prep_x_kernel(const uint16_t *__restrict__ x, int T, int D,
                                                     uint32_t *__restrict__ xp,
                                                     float *__restrict__ xs) {
  // one thread per 64-column group: 8 words of pairs and the group sum
  const int G = D / 64;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * G) return;
  const int t = i / G, g = i - t * G;
  const uint16_t *xg = x + (size_t)t * D + 64 * g;
  uint32_t *o = xp + (size_t)t * (D / 2) + 32 * g;
  // same order as sum8_lanes: eight in-order sums of 8, combined pairwise
  float c8[8];
  for (int c = 0; c < 8; ++c) {
    float v = 0.0f;
    for (int j = 0; j < 8; ++j) v += x_to_f32<F16X>(xg[8 * c + j]);
    c8[c] = v;
  }
  const float s = ((c8[0] + c8[1]) + (c8[2] + c8[3])) + ((c8[4] + c8[5]) + (c8[6] + c8[7]));
  for (int w = 0; w < 8; ++w)
    for (int m = 0; m < 4; ++m)
      o[4 * w + m] = (uint32_t)xg[8 * w + m] | ((uint32_t)xg[8 * w + m + 4] << 16);
  xs[(size_t)t * G + g] = s;
}

}  // namespace

hipError_t launch_prep_x(const void *x, int f16x, int T, int D, uint32_t *xp, float *xs,
                         hipStream_t s) {
  const int n = T * (D / 64);
  dim3 grid((n + 255) / 256);
  if (f16x)
    hipLaunchKernelGGL(prep_x_kernel<true>, grid, dim3(256), 0, s, (const uint16_t *)x, T, D, xp,
                       xs);
  else
    hipLaunchKernelGGL(prep_x_kernel<false>, grid, dim3(256), 0, s, (const uint16_t *)x, T, D, xp,
                       xs);
  return hipGetLastError();
}

hipError_t launch_route(const RouteLaunch &a, hipStream_t s) {
  // one token per block for decode; four tokens share each router load in
  // prefill.  MAXC: 16-column chunks per thread (64 threads split a row, the
  // same split and order as the one-launch decode layer's router).
  const bool small_d = a.D <= 3072;
  if (a.T >= 16) {
    if (small_d)
      return a.f16x ? launch_route_t<true, 4, 4, 3>(a, s) : launch_route_t<false, 4, 4, 3>(a, s);
    return a.f16x ? launch_route_t<true, 4, 4, 8>(a, s) : launch_route_t<false, 4, 4, 8>(a, s);
  }
  if (small_d)
    return a.f16x ? launch_route_t<true, 4, 1, 3>(a, s) : launch_route_t<false, 4, 1, 3>(a, s);
  return a.f16x ? launch_route_t<true, 4, 1, 8>(a, s) : launch_route_t<false, 4, 1, 8>(a, s);
}

}  // namespace moe
