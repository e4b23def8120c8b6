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

#include <algorithm>

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
                            const void *const *table, const void **slot_blob, uint2 *xch,
                            int32_t *host_ids) {
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
    if (host_ids) host_ids[lane] = id;
  }
}
__device__ void topk_wave(const float *lg, int E, int k, int32_t *ids, float *gates,
                          const void *const *table, const void **slot_blob, uint2 *xch,
                          int32_t *host_ids = nullptr) {
  if (E <= 128)
    topk_wave_t<2>(lg, E, k, ids, gates, table, slot_blob, xch, host_ids);
  else if (E <= 256)
    topk_wave_t<4>(lg, E, k, ids, gates, table, slot_blob, xch, host_ids);
  else if (E <= 512)
    topk_wave_t<8>(lg, E, k, ids, gates, table, slot_blob, xch, host_ids);
  else
    topk_wave_t<16>(lg, E, k, ids, gates, table, slot_blob, xch, host_ids);
}

// Top-k of token t's logits published as tagged words (value, epoch) by the
// token group's blocks: one wave polls the E words (NV per lane) until each
// carries `tag` (bounded, then the error word), then selects as topk_wave;
// the blob addresses come from the table staged in LDS.
template <int NV>
__device__ void topk_tagged_t(const uint64_t *lg, int E, int k, uint32_t tag, int32_t *ids,
                              float *gates, const void *const *s_tab, const void **slot_blob,
                              uint2 *xch, int32_t *host_ids, uint32_t *err) {
  const int lane = threadIdx.x & 63;
  uint64_t w[NV];
  for (long s = 0;; ++s) {
#pragma unroll
    for (int j = 0; j < NV; ++j) w[j] = ld_dev(lg + min(lane + 64 * j, E - 1));
    bool ok = true;
#pragma unroll
    for (int j = 0; j < NV; ++j) ok = ok && (lane + 64 * j >= E || (uint32_t)(w[j] >> 32) == tag);
    if (__all(ok)) break;
    if (s > (1L << 20)) {
      if (lane == 0) add_dev(err, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j)
    v[j] = lane + 64 * j < E ? __uint_as_float((uint32_t)w[j]) : -INFINITY;
  int32_t id;
  float gate;
  topk_regs(v, k, xch, &id, &gate);
  if (lane < k) {
    ids[lane] = id;
    gates[lane] = gate;
    if (slot_blob) slot_blob[lane] = s_tab[id];
    if (host_ids) host_ids[lane] = id;
  }
}
__device__ void topk_tagged(const uint64_t *lg, int E, int k, uint32_t tag, int32_t *ids,
                            float *gates, const void *const *s_tab, const void **slot_blob,
                            uint2 *xch, int32_t *host_ids, uint32_t *err) {
  if (E <= 128)
    topk_tagged_t<2>(lg, E, k, tag, ids, gates, s_tab, slot_blob, xch, host_ids, err);
  else if (E <= 256)
    topk_tagged_t<4>(lg, E, k, tag, ids, gates, s_tab, slot_blob, xch, host_ids, err);
  else if (E <= 512)
    topk_tagged_t<8>(lg, E, k, tag, ids, gates, s_tab, slot_blob, xch, host_ids, err);
  else
    topk_tagged_t<16>(lg, E, k, tag, ids, gates, s_tab, slot_blob, xch, host_ids, err);
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
  __shared__ const void *s_tab[kMaxE];  // the blob table (tagged selection)

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
  // the logit bias of the row that wave 0's lane finishes (lane % ROWS)
  const float lbias =
      a.logit_bias ? a.logit_bias[min((int)blockIdx.x * ROWS + lane % ROWS, E - 1)] : 0.0f;
  // Calls of at most kRowTagTokens tokens publish their logits as tagged
  // words (value, call epoch) and block 0 of each token group selects as
  // soon as all of them carry the epoch: no wait for the stores, no counter,
  // no reload after the last block.  Each block keeps its own copy of the
  // epoch and every block advances the copies b, b + grid, ... so that all
  // copies agree whatever the next call's grid.
  const bool tagged = a.rowtag && a.T <= kRowTagTokens && TT == 1;
  const int bid = blockIdx.y * gridDim.x + blockIdx.x, nblk = gridDim.x * gridDim.y;
  uint32_t tag = 0;
  const bool selector = tagged && blockIdx.x == 0;
  if (tagged) {
    tag = __hip_atomic_load(a.rowep + bid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    // the selecting block stages the blob table while the logits are made
    if (selector && a.slot_blob)
      for (int i = tid; i < E; i += kThreads) s_tab[i] = a.table[i];
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
        if (a.logit_bias) s += lbias;
        st_dev(a.logits + (size_t)(t0 + tt) * E + ee, s);
        if (tagged)
          st_dev(a.rowtag + (size_t)(t0 + tt) * E + ee,
                 (uint64_t)__float_as_uint(s) | ((uint64_t)tag << 32));
      }
    }
  }
  if (tagged) {
    if (selector) {
      __syncthreads();  // the staged table
      if (wave < nt) {
        const int t = t0 + wave;
        topk_tagged(a.rowtag + (size_t)t * E, E, a.k, tag, a.ids + (size_t)t * a.k,
                    a.gates + (size_t)t * a.k, s_tab,
                    a.slot_blob ? a.slot_blob + (size_t)t * a.k : nullptr, s_xch[wave],
                    a.host_ids ? a.host_ids + (size_t)t * a.k : nullptr, a.err);
      }
      if (a.host_ids) {
        __threadfence_system();
        __syncthreads();
        if (tid < nt)
          __hip_atomic_store(a.host_flag + t0 + tid, a.host_epoch, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    if (tid == 0)
      for (int j = bid; j < kRowEpochs; j += nblk) st_dev(a.rowep + j, tag);
    return;
  }
  if (wave == 0) {
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
              a.slot_blob ? a.slot_blob + (size_t)t * a.k : nullptr, s_xch[wave],
              a.host_ids ? a.host_ids + (size_t)t * a.k : nullptr);
  }
  if (a.host_ids) {
    // the ids in host memory, then the tokens' flags (release at system
    // scope: the host reads the ids once it sees its epoch)
    __threadfence_system();
    __syncthreads();
    if (tid < nt)
      __hip_atomic_store(a.host_flag + t0 + tid, a.host_epoch, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_SYSTEM);
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

// ---------------------------------------------------------------------------
// Router of a prefill chunk on the matrix cores.  The logits of 16 tokens
// against 16 experts are a 16 x 16 product of the tokens' activations with
// the router weights, accumulated per 64-column group (the affine scale and
// bias are per group): logit[t][e] = sum_g s[g][e] P[t][e][g] + b[g][e] X[t][g],
// P = sum over the group of x q, X = sum over the group of x (the same
// algebra as the row-by-row router; pages: hndistilled.com, "Enfoque
// tecnico", 8-bit router).  P comes from v_mfma_f32_16x16x32 with the codes
// as exact 16-bit integers (bf16 for bf16 activations: q < 256 has 8
// significant bits; fp16 for fp16 activations) and fp32 accumulation, so its
// only rounding is the fp32 summation.
//
// Grid: (parts of the groups, 16-token tiles).  Block (part, tile) stages
// only its part of the tokens' activations and sums, over that part, the
// logits of every expert (one 16-expert tile per wave).  It publishes them
// as tagged words (value, epoch of the token tile); then each block selects
// 16 / parts of the tile's tokens: a wave polls the parts' words of its
// token, adds them in part order and runs the top k.  No block waits for
// another's stores to drain and no counter is taken.
constexpr int kRTok = 16;               // tokens per block (matrix rows)
constexpr int kRWaves = 8;
constexpr int kRThr = kRWaves * 64;
constexpr int kRMaxWords = 16;          // 8-column words of x per thread and part (D <= 4096)
constexpr long kRSpin = 1L << 20;       // bounded waits, then the tokens are marked

// The 16 codes of one chunk (columns 16 c + 0..15 of an expert) as the B
// operands of two products (values 0..7 and 8..15), each register holding
// two consecutive values.
template <bool F16>
__device__ __forceinline__ void codes_b(u32x4 q, u32x4 &b0, u32x4 &b1) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t wd = w[i / 2], sh = 16 * (i % 2);
    if constexpr (F16) {
      // fp16 bits 0x6400 | q = 1024 + q exactly; minus 1024 is exact
      const uint32_t m = __builtin_amdgcn_perm(0x64646464u, wd >> sh, 0x04010400u);
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 v = __builtin_bit_cast(h2, m) - h2{(_Float16)1024.0f, (_Float16)1024.0f};
      r[i] = __builtin_bit_cast(uint32_t, v);
    } else {
      // fp32 of a byte is exact and its upper half is the bf16 value
      const float f0 = (float)((wd >> sh) & 0xFFu), f1 = (float)((wd >> (sh + 8)) & 0xFFu);
      r[i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    }
  }
  b0 = u32x4{r[0], r[1], r[2], r[3]};
  b1 = u32x4{r[4], r[5], r[6], r[7]};
}

// One group of one expert tile: the two products and the affine fold.
template <bool F16X>
__device__ __forceinline__ void group_fold(u32x4 q, uint32_t mw, const uint16_t *xa,
                                           const float *sX, int g, int g4, float (&acc)[4]) {
  u32x4 b0, b1;
  codes_b<F16X>(q, b0, b1);
  const u32x4 a0 = *(const u32x4 *)(xa + 64 * g);
  const u32x4 a1 = *(const u32x4 *)(xa + 64 * g + 8);
  f32x4 P = {0.0f, 0.0f, 0.0f, 0.0f};
  P = mma16<F16X>(a0, b0, P);
  P = mma16<F16X>(a1, b1, P);
  const float sc = f16_to_f32(mw & 0xFFFFu), bi = f16_to_f32(mw >> 16);
  const f32x4 X = *(const f32x4 *)(sX + g * kRTok + 4 * g4);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(bi, X[i], fmaf(sc, P[i], acc[i]));
}

// Groups g0 .. g0 + ng - 1 of one expert tile (xa and sX hold those groups
// only) through a ring of R groups of loads in flight: slot j holds groups
// g0 + j, g0 + j + R, ... and is refilled right after its use, so every wait
// covers exactly the group it needs (ng is a multiple of R).  A group's
// address is a scalar base plus the lane's 32-bit offset.
template <int R>
__device__ __forceinline__ void tile_issue(const RouteLaunch &a, int g0, int e, int g4,
                                           u32x4 (&q)[R], uint32_t (&mw)[R]) {
  const int E = a.E;
  const uint8_t *cb = (const uint8_t *)a.codes, *mb = (const uint8_t *)a.meta;
  const uint32_t vq = (uint32_t)(g4 * E + e) * 16u, vm = (uint32_t)e * 4u;
  const size_t cs = (size_t)E * 64, ms = (size_t)E * 4;  // bytes per group
#pragma unroll
  for (int j = 0; j < R; ++j) {
    q[j] = *(const u32x4 *)(cb + (g0 + j) * cs + vq);
    mw[j] = *(const uint32_t *)(mb + (g0 + j) * ms + vm);
    __builtin_amdgcn_sched_barrier(0);  // issued in slot order
  }
}
// The ring's first R groups already issued (tile_issue); ng a multiple of R.
template <bool F16X, int R>
__device__ __forceinline__ void tile_run(const RouteLaunch &a, int g0, int ng, int e, int g4,
                                         const uint16_t *xa, const float *sX, float (&acc)[4],
                                         u32x4 (&q)[R], uint32_t (&mw)[R]) {
  const int E = a.E, gl = g0 + ng - 1;
  const uint8_t *cb = (const uint8_t *)a.codes, *mb = (const uint8_t *)a.meta;
  const uint32_t vq = (uint32_t)(g4 * E + e) * 16u, vm = (uint32_t)e * 4u;
  const size_t cs = (size_t)E * 64, ms = (size_t)E * 4;  // bytes per group
  if (ng == R) {  // the whole part in the ring: no refill
#pragma unroll
    for (int j = 0; j < R; ++j) group_fold<F16X>(q[j], mw[j], xa, sX, j, g4, acc);
    return;
  }
  for (int gb = g0; gb <= gl; gb += R) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      group_fold<F16X>(q[j], mw[j], xa, sX, gb + j - g0, g4, acc);  // LDS holds g0 ..
      const int gn = min(gb + R + j, gl);  // past the end: the last group again
      q[j] = *(const u32x4 *)(cb + gn * cs + vq);
      mw[j] = *(const uint32_t *)(mb + gn * ms + vm);
      __builtin_amdgcn_sched_barrier(0);  // the refill stays right after its use
    }
  }
}
template <bool F16X, int R>
__device__ __forceinline__ void tile_logits(const RouteLaunch &a, int g0, int ng, int e, int g4,
                                            const uint16_t *xa, const float *sX,
                                            float (&acc)[4]) {
  u32x4 q[R];
  uint32_t mw[R];
  tile_issue<R>(a, g0, e, g4, q, mw);
  tile_run<F16X, R>(a, g0, ng, e, g4, xa, sX, acc, q, mw);
}

size_t route_mfma_smem(int D, int kp) {
  const int P = D / 64 / kp;
  return (size_t)kRTok * (P * 64 + 8) * 2 + (size_t)P * kRTok * 4 + (size_t)kRWaves * 128 * 8;
}

template <bool F16X, int NV, int R>
__global__ __launch_bounds__(kRThr) void route_mfma_kernel(RouteLaunch a, int kp) {
  extern __shared__ __align__(16) uint8_t rsm[];
  const int D = a.D, E = a.E, G = D / 64, W8 = D / 8;
  const int part = blockIdx.x, tt = blockIdx.y;
  const int P = G / kp, g0 = part * P, ldx = P * 64 + 8, PW = P * 8;
  uint16_t *sx = (uint16_t *)rsm;                       // [16][ldx] this part's activation bits
  float *sX = (float *)(rsm + (size_t)kRTok * ldx * 2);  // [P][16] 64-column sums
  uint2 *xch = (uint2 *)(sX + P * kRTok);               // [waves][128] top-k exchange
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = tt * kRTok, nt = min(kRTok, a.T - t0);
  // the token tile's epoch, read with a vector load: nothing waits for it
  // before the logits are published
  const uint32_t tag =
      __hip_atomic_load(a.rep + tt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // clear the counters of the kernel that follows
  if (a.zero) {
    const int bl = tt * gridDim.x + part, nbl = gridDim.x * gridDim.y;
    for (int i = bl * kRThr + tid; i < a.zero_words; i += nbl * kRThr) a.zero[i] = 0u;
    for (int i = bl * kRThr + tid; i < a.zero2_count; i += nbl * kRThr)
      a.zero2[(size_t)i * a.zero2_stride] = 0u;
  }

  // this part's activations: 8-column words into LDS as they are, 64-column
  // sums (sum8_lanes order, as the row router).  No global store in this
  // loop: a store would make each later wait for a load also wait for it.
  const uint16_t *x = (const uint16_t *)a.x;
  u32x4 xv[kRMaxWords];
#pragma unroll
  for (int r = 0; r < kRMaxWords; ++r) {
    const int i = min(tid + r * kRThr, kRTok * PW - 1);
    const int tk = min(i / PW, nt - 1), w = i % PW;
    xv[r] = *(const u32x4 *)(x + (size_t)(t0 + tk) * D + 64 * g0 + 8 * w);
  }
  // the router codes of this wave's first expert tile, in flight while the
  // activations are staged (lane l: expert 16 tile + l % 16, chunk l / 16)
  const int NT = (E + 15) / 16, g4 = lane >> 4, col = lane & 15;
  u32x4 q0[R];
  uint32_t m0[R];
  tile_issue<R>(a, g0, min(wave * 16 + col, E - 1), g4, q0, m0);
#pragma unroll
  for (int r = 0; r < kRMaxWords; ++r) {
    const int i = tid + r * kRThr;
    if (r * kRThr >= kRTok * PW) break;  // uniform over the block
    const bool in = i < kRTok * PW;
    const int tk = i / PW, w = i - tk * PW;
    const bool tok = in && tk < nt;
    const uint32_t wd[4] = {xv[r].x, xv[r].y, xv[r].z, xv[r].w};
    if (in) *(u32x4 *)(sx + (size_t)tk * ldx + 8 * w) = tok ? xv[r] : u32x4{0u, 0u, 0u, 0u};
    float s8 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s8 += x_to_f32<F16X>((wd[j / 2] >> (16 * (j % 2))) & 0xFFFFu);
    const float gs = sum8_lanes(tok ? s8 : 0.0f);
    if (in && (w & 7) == 0) sX[(w >> 3) * kRTok + tk] = tok ? gs : 0.0f;
  }
  __syncthreads();

  // this part's sums of the logits: wave w takes expert tiles w, w + 8, ...;
  // lane l supplies expert 16 tile + l % 16 and the 16-column chunk l / 16
  uint64_t *mine = a.rtag + (size_t)part * a.T * E;
  for (int et = wave; et < NT; et += kRWaves) {
    const int e = min(et * 16 + col, E - 1);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (et == wave)  // the first tile: its codes were issued above
      tile_run<F16X, R>(a, g0, P, e, g4, sx + (size_t)col * ldx + 16 * g4, sX, acc, q0, m0);
    else
      tile_logits<F16X, R>(a, g0, P, e, g4, sx + (size_t)col * ldx + 16 * g4, sX, acc);
    const int ee = et * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g4 + i;
      if (ee < E && row < nt)
        st_dev(mine + (size_t)(t0 + row) * E + ee,
               (uint64_t)__float_as_uint(acc[i]) | ((uint64_t)tag << 32));
    }
  }

  // selection: this block's share of the tile's tokens, one per wave
  const int per = (kRTok + kp - 1) / kp;
  for (int j = wave; j < per; j += kRWaves) {
    const int row = part * per + j;
    if (row >= nt) break;  // uniform over the wave
    const int t = t0 + row;
    // the logit bias before the wait (no load after it but the polls)
    float bias[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q)
      bias[q] = a.logit_bias ? a.logit_bias[min(lane + 64 * q, E - 1)] : 0.0f;
    // every part's words of the token in one round trip per try
    uint64_t w[kRouteParts][NV];
    for (long sp = 0;; ++sp) {
      bool ok = true;
#pragma unroll
      for (int pp = 0; pp < kRouteParts; ++pp) {
        const uint64_t *src = a.rtag + ((size_t)min(pp, kp - 1) * a.T + t) * E;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
          w[pp][q] = ld_dev(src + min(lane + 64 * q, E - 1));
          ok = ok && (pp >= kp || (uint32_t)(w[pp][q] >> 32) == tag);
        }
      }
      if (__all(ok) || sp > kRSpin) break;
      __builtin_amdgcn_s_sleep(1);
    }
    float v[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      v[q] = 0.0f;
#pragma unroll
      for (int pp = 0; pp < kRouteParts; ++pp)  // part order
        if (pp < kp) v[q] += __uint_as_float((uint32_t)w[pp][q]);
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        if (a.logit_bias) v[q] += bias[q];
        a.logits[(size_t)t * E + e] = v[q];
      } else {
        v[q] = -INFINITY;
      }
    }
    int32_t id;
    float gate;
    topk_regs(v, a.k, xch + wave * 128, &id, &gate);
    const size_t o = (size_t)t * a.k + lane;
    if (lane < a.k) {
      a.ids[o] = id;
      a.gates[o] = gate;
      if (a.slot_blob) a.slot_blob[o] = a.table[id];
    }
  }
  // the pairs and sums the 4-bit expert kernels read, for this part's groups
  // (after the waits: a store ahead of a load would make its wait longer)
  for (int i = tid; i < nt * PW; i += kRThr) {
    const int tk = i / PW, w = i - tk * PW;
    const u32x4 v = *(const u32x4 *)(sx + (size_t)tk * ldx + 8 * w);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      o[m] = ((wd[m / 2] >> (16 * (m % 2))) & 0xFFFFu) |
             (((wd[2 + m / 2] >> (16 * (m % 2))) & 0xFFFFu) << 16);
    *(u32x4 *)(a.xp + (size_t)(t0 + tk) * (D / 2) + 32 * g0 + 4 * w) = u32x4{o[0], o[1], o[2], o[3]};
    if ((w & 7) == 0) a.xs[(size_t)(t0 + tk) * G + g0 + (w >> 3)] = sX[(w >> 3) * kRTok + tk];
  }
  // every block of the tile has read its epoch (their logits are in), so
  // part 0 can advance it, and the copies tt + j ntt with it, once its own
  // selection is done: all copies move in step whatever the next call's T
  __syncthreads();
  const int ntt = gridDim.y;
  if (part == 0)
    for (int j = tt + tid * ntt; j < kMaxRouteTiles; j += kRThr * ntt)
      __hip_atomic_store(a.rep + j, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool F16X, int NV, int R>
hipError_t launch_route_mfma_r(const RouteLaunch &a, int kp, hipStream_t s) {
  const size_t smem = route_mfma_smem(a.D, kp);
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void *)route_mfma_kernel<F16X, NV, R>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  const dim3 grid(kp, (a.T + kRTok - 1) / kRTok);
  hipLaunchKernelGGL((route_mfma_kernel<F16X, NV, R>), grid, dim3(kRThr), smem, s, a, kp);
  return hipGetLastError();
}
// kp parts of the groups (4 when they divide), and the deepest ring that
// divides a part
template <bool F16X, int NV>
hipError_t launch_route_mfma_t(const RouteLaunch &a, hipStream_t s) {
  const int G = a.D / 64;
  const int kp = G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1, P = G / kp;
  if (P % 11 == 0) return launch_route_mfma_r<F16X, NV, 11>(a, kp, s);
  if (P % 8 == 0) return launch_route_mfma_r<F16X, NV, 8>(a, kp, s);
  if (P % 4 == 0) return launch_route_mfma_r<F16X, NV, 4>(a, kp, s);
  if (P % 2 == 0) return launch_route_mfma_r<F16X, NV, 2>(a, kp, s);
  return launch_route_mfma_r<F16X, NV, 1>(a, kp, s);
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
  if (a.T >= 16 && a.host_ids) return hipErrorInvalidValue;  // ids to the host: row router only
  if (a.T >= 16 && tuning().route_mfma && a.E <= 256 && a.D <= 4096 && a.rtag && a.rep) {
    // windows of as many tokens as the tagged area holds (whole 16-token tiles)
    const int win = (int)(kRouteTagBytes / (sizeof(uint64_t) * kRouteParts * a.E)) / kRTok * kRTok;
    for (int t0 = 0; t0 < a.T; t0 += win) {
      RouteLaunch b = a;
      const int n = std::min(win, a.T - t0);
      b.T = n;
      b.x = (const uint16_t *)a.x + (size_t)t0 * a.D;
      b.logits = a.logits + (size_t)t0 * a.E;
      b.ids = a.ids + (size_t)t0 * a.k;
      b.gates = a.gates + (size_t)t0 * a.k;
      if (a.slot_blob) b.slot_blob = a.slot_blob + (size_t)t0 * a.k;
      b.xp = a.xp + (size_t)t0 * (a.D / 2);
      b.xs = a.xs + (size_t)t0 * (a.D / 64);
      if (t0 > 0) b.zero = nullptr, b.zero_words = 0, b.zero2 = nullptr, b.zero2_count = 0;
      hipError_t e;
      if (a.E <= 128)
        e = a.f16x ? launch_route_mfma_t<true, 2>(b, s) : launch_route_mfma_t<false, 2>(b, s);
      else
        e = a.f16x ? launch_route_mfma_t<true, 4>(b, s) : launch_route_mfma_t<false, 4>(b, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
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
