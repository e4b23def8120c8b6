// 4-bit affine expert FFN kernels for few tokens per expert (decode).
//
// The selected experts are GLU blocks stored as MLX-affine 4-bit weights with
// one fp16 scale and bias per 64 columns (es.news.hada.io, "Estructura de
// ejecucion para reducir memoria"); the weights are consumed in their stored
// layout with no conversion pass (stork.ai blog, "El arma secreta de Apple:
// memoria unificada").  Decode is a matrix-vector product bound by HBM
// bandwidth, so the kernels run on the vector ALUs:
//
//  * lane = weight row; the chunk-major layout makes the 64 lanes of a wave
//    read one contiguous 1 KiB span per 16-byte load;
//  * codes become bf16 (fp16) 128 + q by an OR into the mantissa and meet the
//    activation pairs in v_dot2c_f32_bf16; per 64-column group the affine terms
//    fold as  sum x (s q + b) = s * sum x (128 + q) + (b - 128 s) * sum x;
//  * activations are wave-uniform, so the compiler keeps them in scalar
//    registers (no LDS traffic);
//  * the reduction is split over the waves of a block and over KS blocks; the
//    last block of a row tile (a workspace counter) adds the partials in a
//    fixed order, so results are bitwise reproducible.
//
// glu_kernel:  h[slot, j] = gelu_tanh(x . Wg[j]) * (x . Wu[j]), written as bf16
//              hi/lo pairs plus 64-unit sums for the down projection.
// down_kernel: y[slot, n] = h . Wd[n]  (per slot), or
//              out[t, n] = sum_j gate[t,j] y[(t,j), n] + y_shared[t, n]
//              with the combine fused (decode layer forward).
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNW = 4;    // waves per block
constexpr int kMaxG = 4;  // 64-column groups per wave (GLU)
constexpr int kMaxU = 4;  // (slot, group) units per wave (down)

// Map a GLU block index to its slot, expert blob and hidden-row tile.
struct SlotInfo {
  const uint8_t *blob;  // null: skip (invalid expert id)
  int slot, t, F, rb;
  size_t hoff;  // first hidden unit of the slot in h
};

__device__ __forceinline__ SlotInfo glu_slot(const ExpertLaunch &a, int bid) {
  SlotInfo si;
  const int nr = a.T * a.k;
  const int rbr = a.F / 64;
  if (bid < nr * rbr) {
    si.slot = bid / rbr;
    si.rb = bid - si.slot * rbr;
    si.t = si.slot / a.k;
    si.F = a.F;
    if (a.slot_blob) {
      si.blob = (const uint8_t *)a.slot_blob[si.slot];
    } else {
      const int e = a.ids ? a.ids[si.slot] : 0;
      si.blob = (e >= 0 && e < a.E) ? (const uint8_t *)a.rblobs[e] : nullptr;
    }
    si.hoff = (size_t)si.slot * a.F;
  } else {
    const int rbs = a.Fs / 64;
    const int b2 = bid - nr * rbr;
    si.t = b2 / rbs;
    si.rb = b2 - si.t * rbs;
    si.slot = nr + si.t;
    si.F = a.Fs;
    si.blob = (const uint8_t *)a.sblobs[0];
    si.hoff = (size_t)nr * a.F + (size_t)si.t * a.Fs;
  }
  return si;
}

// Split-reduction handoff: every block of a tile stores its partial, the last
// one to arrive (workspace counter) adds all partials in split order.
// Returns false in the blocks that are not last.  Wave 0 only.
template <int W>
__device__ __forceinline__ bool split_reduce(float (&v)[W], float *part, uint32_t *counter, int KS,
                                             int ks) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < W; ++i) st_dev(part + (ks * W + i) * 64 + lane, v[i]);
  wait_all_memory();
  uint32_t old = 0;
  if (lane == 0) old = add_dev(counter, 1u);
  old = __shfl(old, 0, 64);
  if (old != (uint32_t)(KS - 1)) return false;
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = 0.0f;
  // eight splits' partials in flight at a time, added in split order
  for (int p0 = 0; p0 < KS; p0 += 8) {
    float q[8][W];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < W; ++i)
        q[j][i] = p0 + j < KS ? ld_dev(part + ((p0 + j) * W + i) * 64 + lane) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j < KS)
#pragma unroll
        for (int i = 0; i < W; ++i) v[i] += q[j][i];
  }
  if (lane == 0) st_dev(counter, 0u);
  return true;
}

template <bool F16X>
__global__ __launch_bounds__(kNW * 64) void glu_kernel(ExpertLaunch a, int KS) {
  __shared__ float red[kNW][2][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int bid = a.glu_first + blockIdx.x, ks = blockIdx.y;
  const SlotInfo si = glu_slot(a, bid);
  const int D = a.D, F = si.F, G = D / 64;
  const int j = si.rb * 64 + lane;
  const int g0 = ks * G / KS, g1 = (ks + 1) * G / KS;

  float accg = 0.0f, accu = 0.0f;
  if (si.blob) {
    const BlobLayout L = blob_layout(D, F);
    const gptr<u32x4> gc = as_global((const u32x4 *)(si.blob + L.gate_codes) + j);
    const gptr<u32x4> uc = as_global((const u32x4 *)(si.blob + L.up_codes) + j);
    const gptr<uint32_t> gm = as_global((const uint32_t *)(si.blob + L.gate_meta) + j);
    const gptr<uint32_t> um = as_global((const uint32_t *)(si.blob + L.up_meta) + j);
    const uint32_t *xp = a.xp + (size_t)si.t * (D / 2);
    const float *xs = a.xs + (size_t)si.t * G;
    const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);
    // every load of a batch first (the tail clamps to a valid group), then the
    // arithmetic: one memory latency per batch (decode: a single batch)
    for (int base = g0; base < g1; base += kNW * kMaxG) {
      u32x4 qg0[kMaxG], qg1[kMaxG], qu0[kMaxG], qu1[kMaxG];
      uint32_t mg[kMaxG], mu[kMaxG];
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        const int g = min(base + wave + i * kNW, g1 - 1);
        const size_t c0 = (size_t)(2 * g) * F;
        qg0[i] = gc[c0];
        qg1[i] = gc[c0 + F];
        qu0[i] = uc[c0];
        qu1[i] = uc[c0 + F];
        mg[i] = gm[(size_t)g * F];
        mu[i] = um[(size_t)g * F];
      }
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        const int g = base + wave + i * kNW;
        if (g >= g1) break;
        uint32_t xg[32];
        load_uniform(xp + g * 32, xg);
        float dg = dot_chunk<F16X>(qg0[i], xg, 0.0f, magic);
        dg = dot_chunk<F16X>(qg1[i], xg + 16, dg, magic);
        float du = dot_chunk<F16X>(qu0[i], xg, 0.0f, magic);
        du = dot_chunk<F16X>(qu1[i], xg + 16, du, magic);
        const float xsg = as_const(xs)[g];
        const float sg = f16_to_f32(mg[i]), bg = f16_to_f32(mg[i] >> 16);
        const float su = f16_to_f32(mu[i]), bu = f16_to_f32(mu[i] >> 16);
        accg = fmaf(sg, dg, accg);
        accg = fmaf(fmaf(-Magic<F16X>::offset, sg, bg), xsg, accg);
        accu = fmaf(su, du, accu);
        accu = fmaf(fmaf(-Magic<F16X>::offset, su, bu), xsg, accu);
      }
    }
  }
  red[wave][0][lane] = accg;
  red[wave][1][lane] = accu;
  __syncthreads();
  if (wave != 0) return;

  float v[2] = {0.0f, 0.0f};
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    v[0] += red[w][0][lane];
    v[1] += red[w][1][lane];
  }
  if (KS > 1 &&
      !split_reduce(v, a.part + (size_t)blockIdx.x * KS * 128, a.counters + blockIdx.x, KS, ks))
    return;
  const float h = si.blob ? gelu_tanh(v[0]) * v[1] : 0.0f;
  const size_t unit = si.hoff + (size_t)si.rb * 64;
  a.h[unit + lane] = h;
  const float hsum = wave_sum(h);
  if (lane == 0) a.hs[unit / 64] = hsum;
}

// Down projection; COMBINE fuses the gate-weighted sum over a token's slots
// and the shared expert.  h is fp32 and the codes are converted exactly, so
// no large offset enters the accumulation (the hidden activations have a
// large mean).
template <bool COMBINE>
__global__ __launch_bounds__(kNW * 64) void down_kernel(ExpertLaunch a, int KS) {
  __shared__ float red[kNW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int D = a.D, NB = D / 64;
  const int bid = blockIdx.x, ks = blockIdx.y;
  const int o = bid / NB, nb = bid - o * NB;  // o: token (COMBINE) or slot
  const int n = nb * 64 + lane;
  const int Gf = a.F / 64;
  const int Gs = (COMBINE && a.sblobs) ? a.Fs / 64 : 0;
  const int U = COMBINE ? a.k * Gf + Gs : Gf;
  const int u0 = ks * U / KS, u1 = (ks + 1) * U / KS;

  float acc = 0.0f;
  for (int base = u0; base < u1; base += kNW * kMaxU) {
    u32x4 q0[kMaxU], q1[kMaxU];
    uint32_t mw[kMaxU];
    size_t hoff[kMaxU];
    int gg[kMaxU];
    float gate[kMaxU];
    bool use[kMaxU];
#pragma unroll
    for (int i = 0; i < kMaxU; ++i) {
      const int u = min(base + wave + i * kNW, u1 - 1);
      int g, Fb;
      const uint8_t *blob;
      gate[i] = 1.0f;
      use[i] = base + wave + i * kNW < u1;
      if (!COMBINE || u < a.k * Gf) {
        const int jj = COMBINE ? u / Gf : 0;
        g = COMBINE ? u - jj * Gf : u;
        const int slot = COMBINE ? o * a.k + jj : o;
        if (a.slot_blob) {
          blob = (const uint8_t *)a.slot_blob[slot];
        } else {
          const int e = a.ids ? a.ids[slot] : 0;
          const bool ok = e >= 0 && e < a.E;
          use[i] = use[i] && ok;
          blob = (const uint8_t *)a.rblobs[ok ? e : 0];
        }
        if (COMBINE) gate[i] = a.gates[slot];
        Fb = a.F;
        hoff[i] = (size_t)slot * a.F;
      } else {
        g = u - a.k * Gf;
        blob = (const uint8_t *)a.sblobs[0];
        Fb = a.Fs;
        hoff[i] = (size_t)a.T * a.k * a.F + (size_t)o * a.Fs;
      }
      gg[i] = g;
      const BlobLayout L = blob_layout(D, Fb);
      const gptr<u32x4> dc = as_global((const u32x4 *)(blob + L.down_codes) + n);
      q0[i] = dc[(size_t)(2 * g) * D];
      q1[i] = dc[(size_t)(2 * g + 1) * D];
      mw[i] = as_global((const uint32_t *)(blob + L.down_meta))[(size_t)g * D + n];
    }
#pragma unroll
    for (int i = 0; i < kMaxU; ++i) {
      if (!use[i]) continue;
      float hv[64];
      load_uniform_f(a.h + hoff[i] + (size_t)gg[i] * 64, hv);
      const float d = dot_group_f32(q0[i], q1[i], hv);
      const float hsg = as_const(a.hs)[hoff[i] / 64 + gg[i]];
      const float v = fmaf(f16_to_f32(mw[i]), d, f16_to_f32(mw[i] >> 16) * hsg);
      acc = fmaf(gate[i], v, acc);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float sum[1] = {0.0f};
#pragma unroll
  for (int w = 0; w < kNW; ++w) sum[0] += red[w][lane];
  if (KS > 1 &&
      !split_reduce(sum, a.part + (size_t)bid * KS * 64, a.counters + bid, KS, ks))
    return;
  if (COMBINE) {
    const size_t idx = (size_t)o * D + n;
    if (a.out_dtype == MOE_F32)
      ((float *)a.out)[idx] = sum[0];
    else if (a.out_dtype == MOE_BF16)
      ((uint16_t *)a.out)[idx] = (uint16_t)f32_to_bf16(sum[0]);
    else
      ((uint16_t *)a.out)[idx] = (uint16_t)f32_to_f16(sum[0]);
  } else {
    a.y[(size_t)o * D + n] = sum[0];
  }
}

__global__ void combine_kernel(const float *__restrict__ y, const float *__restrict__ gates,
                               const float *__restrict__ ys, int T, int k, int D, void *out,
                               int out_dtype) {
  const size_t total = (size_t)T * D;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / D, n = i - t * D;
    // in double, rounded once (exact products; outputs of large magnitude)
    double acc = ys ? (double)ys[i] : 0.0;
    for (int j = 0; j < k; ++j)
      acc = fma((double)gates[t * k + j], (double)y[(t * k + j) * D + n], acc);
    const float s = (float)acc;
    if (out_dtype == MOE_F32)
      ((float *)out)[i] = s;
    else if (out_dtype == MOE_BF16)
      ((uint16_t *)out)[i] = (uint16_t)f32_to_bf16(s);
    else
      ((uint16_t *)out)[i] = (uint16_t)f32_to_f16(s);
  }
}

}  // namespace

// Split of a reduction over blocks: about two resident blocks per compute
// unit (256 CUs), at most kMaxKS, and never more than kMaxSplitBlocks blocks
// in a split launch (the workspace holds that many partial tiles).
int pick_ks(int blocks, int reduce_len, int min_ks, int override_ks) {
  int ks = override_ks > 0 ? override_ks : (512 + blocks - 1) / blocks;
  if (ks < min_ks) ks = min_ks;
  if (ks > reduce_len) ks = reduce_len;
  if (ks > kMaxKS) ks = kMaxKS;
  if (ks > 1 && (long)blocks * ks > kMaxSplitBlocks) ks = kMaxSplitBlocks / blocks;
  return ks < 1 ? 1 : ks;
}

int glu_blocks(const ExpertLaunch &a) {
  return a.T * a.k * (a.F / 64) + (a.sblobs ? a.T * (a.Fs / 64) : 0);
}

int glu_min_ks(int D) { return (D / 64 + kNW * kMaxG - 1) / (kNW * kMaxG); }

hipError_t launch_glu(const ExpertLaunch &a, hipStream_t s) {
  const int blocks = a.glu_count;
  if (blocks <= 0) return hipSuccess;
  const int KS = a.glu_ks > 0 ? a.glu_ks
                              : pick_ks(blocks, a.D / 64, glu_min_ks(a.D), tuning().glu_ks);
  if (KS > 1 && (long)blocks * KS > kMaxSplitBlocks) return hipErrorInvalidValue;
  dim3 grid(blocks, KS);
  if (a.f16x)
    hipLaunchKernelGGL((glu_kernel<true>), grid, dim3(kNW * 64), 0, s, a, KS);
  else
    hipLaunchKernelGGL((glu_kernel<false>), grid, dim3(kNW * 64), 0, s, a, KS);
  return hipGetLastError();
}

hipError_t launch_down(const ExpertLaunch &a, bool combine, hipStream_t s) {
  const int NB = a.D / 64;
  const int outs = combine ? a.T : a.T * a.k;
  const int U = combine ? a.k * (a.F / 64) + (a.sblobs ? a.Fs / 64 : 0) : a.F / 64;
  const int min_ks = (U + kNW * kMaxU - 1) / (kNW * kMaxU);
  const int KS = pick_ks(outs * NB, U, min_ks, tuning().down_ks);
  if (KS > 1 && (long)outs * NB * KS > kMaxSplitBlocks) return hipErrorInvalidValue;
  dim3 grid(outs * NB, KS);
  if (combine)
    hipLaunchKernelGGL((down_kernel<true>), grid, dim3(kNW * 64), 0, s, a, KS);
  else
    hipLaunchKernelGGL((down_kernel<false>), grid, dim3(kNW * 64), 0, s, a, KS);
  return hipGetLastError();
}

hipError_t launch_combine(const float *y, const float *gates, const float *ys, int T, int k,
                          int D, void *out, int out_dtype, hipStream_t s) {
  const size_t total = (size_t)T * D;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, y, gates, ys, T, k, D, out,
                     out_dtype);
  return hipGetLastError();
}

}  // namespace moe
