// One-launch expert phase of a decode step: gate/up GLU of every selected
// expert and the shared expert, down projection and combine.
//
// Per token the pages run the selected routed experts and the resident shared
// expert, then combine the two outputs (es.news.hada.io, "Proceso de
// generacion de tokens").  After routing, every byte this phase reads is
// known, so each block issues all of its loads at once -- its gate/up tile and
// the down-projection codes of its output tile -- and only then waits: the
// gate/up tile needs nothing from other blocks, the down tile needs the hidden
// activations of the slots it sums over.  Those arrive through per-slot
// counters in the workspace (device-scope stores, loads and atomics; no
// full-cache fences).  Every block of the grid must be resident at once (the
// host checks the occupancy before choosing this kernel), every wait is
// bounded, and the last block to finish returns the counters to zero.
//
// Work split (decode, T = 1, k = 8, D = 2816, F = 704, F_s = 2112):
//   gate/up: 121 tiles of 64 hidden rows (88 routed + 33 shared) x KSg
//            reduction splits over the 44 column groups;
//   down:    44 tiles of 64 output rows x (KSdr splits of the 88 routed
//            (slot, group) units + KSds splits of the 33 shared units), the
//            splits of the one-launch layer kernel, so both agree bit for bit.
// Block b owns gate/up item b and down item b.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNW = 4;
constexpr long kSpinLimit = 1L << 24;  // bounded waits (~seconds), then an error flag

struct GluTile {
  const uint8_t *blob;
  int slot, t, F, rb;
  size_t hoff;
};

__device__ __forceinline__ GluTile fused_tile(const FusedLaunch &f, int tile) {
  const ExpertLaunch &a = f.a;
  GluTile gt;
  const int nr = a.T * a.k, rbr = a.F / 64;
  if (tile < nr * rbr) {
    gt.slot = tile / rbr;
    gt.rb = tile - gt.slot * rbr;
    gt.t = gt.slot / a.k;
    gt.F = a.F;
    gt.blob = (const uint8_t *)a.slot_blob[gt.slot];
    gt.hoff = (size_t)gt.slot * a.F;
  } else {
    const int rbs = a.Fs / 64, b2 = tile - nr * rbr;
    gt.t = b2 / rbs;
    gt.rb = b2 - gt.t * rbs;
    gt.slot = nr + gt.t;
    gt.F = a.Fs;
    gt.blob = (const uint8_t *)a.sblobs[0];
    gt.hoff = (size_t)nr * a.F + (size_t)gt.t * a.Fs;
  }
  return gt;
}

template <bool F16X, int kMaxG, int kMaxU>
__global__ __launch_bounds__(kNW * 64) void experts_fused_kernel(FusedLaunch f) {
  __shared__ float red[kNW][2][64];
  __shared__ float hbuf[kNW][kMaxU][64];
  const ExpertLaunch &a = f.a;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int D = a.D, G = D / 64, NB = D / 64;
  const bool has_g = b < (f.tile_end - f.tile_begin) * f.KSg;
  const bool has_d = f.do_down && b < a.T * NB * f.KSd;

  // ---------------- issue the gate/up loads of this block's tile split
  GluTile gt{};
  int g0 = 0, g1 = 0;
  u32x4 qg0[kMaxG], qg1[kMaxG], qu0[kMaxG], qu1[kMaxG];
  uint32_t mg[kMaxG], mu[kMaxG];
  if (has_g) {
    const int tile = f.tile_begin + b / f.KSg, ks = b % f.KSg;
    gt = fused_tile(f, tile);
    g0 = ks * G / f.KSg;
    g1 = (ks + 1) * G / f.KSg;
    const int F = gt.F, j = gt.rb * 64 + lane;
    const BlobLayout L = blob_layout(D, F);
    const gptr<u32x4> gc = as_global((const u32x4 *)(gt.blob + L.gate_codes) + j);
    const gptr<u32x4> uc = as_global((const u32x4 *)(gt.blob + L.up_codes) + j);
    const gptr<uint32_t> gm = as_global((const uint32_t *)(gt.blob + L.gate_meta) + j);
    const gptr<uint32_t> um = as_global((const uint32_t *)(gt.blob + L.up_meta) + j);
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) {
      const int g = min(g0 + wave + i * kNW, g1 - 1);
      const size_t c0 = (size_t)(2 * g) * F;
      qg0[i] = gc[c0];
      qg1[i] = gc[c0 + F];
      qu0[i] = uc[c0];
      qu1[i] = uc[c0 + F];
      mg[i] = gm[(size_t)g * F];
      mu[i] = um[(size_t)g * F];
    }
  }

  // ---------------- issue the down-projection loads of this block's output split
  const int Gf = a.F / 64, Gs = a.sblobs ? a.Fs / 64 : 0;
  const int Ur = a.k * Gf;  // units: routed (slot by slot), then shared
  int t_out = 0, n = 0, ksd = 0, u0 = 0, u1 = 0;
  u32x4 dq0[kMaxU], dq1[kMaxU];
  uint32_t dmw[kMaxU];
  size_t hoff[kMaxU];
  int gg[kMaxU];
  float gate[kMaxU];
  bool use[kMaxU];
  if (has_d) {
    const int ot = b / f.KSd;
    ksd = b - ot * f.KSd;
    t_out = ot / NB;
    n = (ot - t_out * NB) * 64 + lane;
    if (ksd < f.KSdr) {  // a split of the routed units, else of the shared units
      u0 = ksd * Ur / f.KSdr;
      u1 = (ksd + 1) * Ur / f.KSdr;
    } else {
      u0 = Ur + (ksd - f.KSdr) * Gs / f.KSds;
      u1 = Ur + (ksd - f.KSdr + 1) * Gs / f.KSds;
    }
#pragma unroll
    for (int i = 0; i < kMaxU; ++i) {
      const int u = min(u0 + wave + i * kNW, u1 - 1);
      use[i] = u0 + wave + i * kNW < u1;
      const uint8_t *blob;
      int g, Fb;
      if (u < a.k * Gf) {
        const int jj = u / Gf;
        g = u - jj * Gf;
        const int slot = t_out * a.k + jj;
        blob = (const uint8_t *)a.slot_blob[slot];
        gate[i] = a.gates[slot];
        Fb = a.F;
        hoff[i] = (size_t)slot * a.F;
      } else {
        g = u - a.k * Gf;
        blob = (const uint8_t *)a.sblobs[0];
        gate[i] = 1.0f;
        Fb = a.Fs;
        hoff[i] = (size_t)a.T * a.k * a.F + (size_t)t_out * a.Fs;
      }
      gg[i] = g;
      const BlobLayout L = blob_layout(D, Fb);
      const gptr<u32x4> dc = as_global((const u32x4 *)(blob + L.down_codes) + n);
      dq0[i] = dc[(size_t)(2 * g) * D];
      dq1[i] = dc[(size_t)(2 * g + 1) * D];
      dmw[i] = as_global((const uint32_t *)(blob + L.down_meta))[(size_t)g * D + n];
    }
  }

  // ---------------- gate/up arithmetic, split reduction, hidden activations
  if (has_g) {
    const uint32_t *xp = a.xp + (size_t)gt.t * (D / 2);
    const float *xs = a.xs + (size_t)gt.t * G;
    const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);
    float accg = 0.0f, accu = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) {
      const int g = g0 + wave + i * kNW;
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
    red[wave][0][lane] = accg;
    red[wave][1][lane] = accu;
    __syncthreads();
    if (wave == 0) {
      float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        v0 += red[w][0][lane];
        v1 += red[w][1][lane];
      }
      const int tile = f.tile_begin + b / f.KSg;
      bool last = true;
      if (f.KSg > 1) {
        const float pv[2] = {v0, v1};
        float sv[2];
        last = split_reduce_fixed<2>(f.gacc + (size_t)tile * 128, f.gcnt + (size_t)tile * kCntStride,
                                     f.KSg, pv, sv, f.err);
        v0 = sv[0];
        v1 = sv[1];
      }
      if (last) {
        const float h = gelu_tanh(v0) * v1;
        st_dev(a.h + gt.hoff + (size_t)gt.rb * 64 + lane, h);
        wait_all_memory();
        uint32_t old = 0;
        if (lane == 0) old = add_dev(f.slot_cnt + gt.slot, 1u);
        old = __shfl(old, 0, 64);
        if (old == (uint32_t)(gt.F / 64 - 1) && lane < kFlagCopies)  // the slot is complete
          st_dev(f.slot_flag + ((size_t)gt.slot * kFlagCopies + lane) * 32, 1u);
      }
    }
  }

  // ---------------- down projection and combine
  if (has_d) {
    // one thread waits for the ready flags of the slots this split sums over
    // (each slot's flag is replicated so that the polls spread over lines)
    if (threadIdx.x == 0) {
      const int s_lo = u0 / Gf < a.k ? u0 / Gf : a.k;
      const int s_hi = (u1 - 1) / Gf < a.k ? (u1 - 1) / Gf : a.k;  // a.k: the shared expert
      bool ok = true;
      for (int sj = s_lo; sj <= s_hi; ++sj) {
        const int slot = sj < a.k ? t_out * a.k + sj : a.T * a.k + t_out;
        const uint32_t *flag = f.slot_flag + ((size_t)slot * kFlagCopies + b % kFlagCopies) * 32;
        long spins = 0;
        while (ld_dev(flag) == 0u) {
          if (++spins > kSpinLimit) {
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
      }
      if (!ok) add_dev(f.err, 1u);
    }
    __syncthreads();
    float hsum[kMaxU];
#pragma unroll
    for (int i = 0; i < kMaxU; ++i) {
      const float hv = use[i] ? ld_dev(a.h + hoff[i] + (size_t)gg[i] * 64 + lane) : 0.0f;
      hbuf[wave][i][lane] = hv;
      hsum[i] = wave_sum(hv);
    }
    __builtin_amdgcn_wave_barrier();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxU; ++i) {
      if (!use[i]) continue;
      float hv[64];
#pragma unroll
      for (int j = 0; j < 64; j += 4) {
        const float4 v4 = *(const float4 *)&hbuf[wave][i][j];
        hv[j] = v4.x;
        hv[j + 1] = v4.y;
        hv[j + 2] = v4.z;
        hv[j + 3] = v4.w;
      }
      const float d = dot_group_f32(dq0[i], dq1[i], hv);
      const float v = fmaf(f16_to_f32(dmw[i]), d, f16_to_f32(dmw[i] >> 16) * hsum[i]);
      acc = fmaf(gate[i], v, acc);
    }
    __syncthreads();  // red[] is reused
    red[wave][0][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) s += red[w][0][lane];
      const int ot = b / f.KSd;
      bool last = true;
      if (f.KSd > 1) {
        const float pv[1] = {s};
        float sv[1];
        last = split_reduce_fixed<1>(f.dacc + (size_t)ot * 64, f.dcnt + (size_t)ot * kCntStride,
                                     f.KSd, pv, sv, f.err);
        s = sv[0];
      }
      if (last) {
        const size_t idx = (size_t)t_out * D + n;
        if (a.out_dtype == MOE_F32)
          ((float *)a.out)[idx] = s;
        else if (a.out_dtype == MOE_BF16)
          ((uint16_t *)a.out)[idx] = (uint16_t)f32_to_bf16(s);
        else
          ((uint16_t *)a.out)[idx] = (uint16_t)f32_to_f16(s);
      }
    }
  }

}



int g_capacity[4096];  // co-resident blocks per (device, dtype, kernel shape)

}  // namespace

int fused_grid(const FusedLaunch &f) {
  const int g = (f.tile_end - f.tile_begin) * f.KSg;
  const int d = f.do_down ? f.a.T * (f.a.D / 64) * f.KSd : 0;
  return g > d ? g : d;
}

namespace {
using KernelFn = void (*)(FusedLaunch);
template <bool F16X>
KernelFn pick_kernel(int mg, int mu) {
#define MOE_FUSED_CASE(G, U) \
  if (mg == G && mu == U) return experts_fused_kernel<F16X, G, U>;
  MOE_FUSED_CASE(2, 2) MOE_FUSED_CASE(2, 3) MOE_FUSED_CASE(2, 4)
  MOE_FUSED_CASE(3, 2) MOE_FUSED_CASE(3, 3) MOE_FUSED_CASE(3, 4)
  MOE_FUSED_CASE(4, 2) MOE_FUSED_CASE(4, 3) MOE_FUSED_CASE(4, 4)
#undef MOE_FUSED_CASE
  return nullptr;
}
int ceil_div(int a, int b) { return (a + b - 1) / b; }
}  // namespace

// groups per wave and units per wave of a split (at least 2: one kernel shape
// serves the smallest splits too)
int fused_max_g(const FusedLaunch &f) {
  const int m = ceil_div(ceil_div(f.a.D / 64, f.KSg), kNW);
  return m < 2 ? 2 : m;
}
int fused_max_u(const FusedLaunch &f) {
  int m = ceil_div(ceil_div(f.a.k * (f.a.F / 64), f.KSdr), kNW);
  if (f.KSds > 0) {
    const int ms = ceil_div(ceil_div(f.a.Fs / 64, f.KSds), kNW);
    m = m > ms ? m : ms;
  }
  return m < 2 ? 2 : m;
}

hipError_t fused_capacity(const FusedLaunch &f, int *cap) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int mg = fused_max_g(f), mu = fused_max_u(f);
  KernelFn k = f.a.f16x ? pick_kernel<true>(mg, mu) : pick_kernel<false>(mg, mu);
  if (!k) {
    *cap = 0;
    return hipSuccess;
  }
  const int key = (dev * 2 + (f.a.f16x ? 1 : 0)) * 16 + (mg - 2) * 3 + (mu - 2);
  if (key < 0 || key >= 4096) return hipErrorInvalidDevice;
  if (!g_capacity[key]) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k, kNW * 64, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_capacity[key] = per_cu * cus;
  }
  *cap = g_capacity[key];
  return hipSuccess;
}

hipError_t launch_fused(const FusedLaunch &f, hipStream_t s) {
  const int grid = fused_grid(f);
  if (grid <= 0) return hipSuccess;
  const int mg = fused_max_g(f), mu = fused_max_u(f);
  KernelFn k = f.a.f16x ? pick_kernel<true>(mg, mu) : pick_kernel<false>(mg, mu);
  if (!k) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, dim3(grid), dim3(kNW * 64), 0, s, f);
  return hipGetLastError();
}

}  // namespace moe
