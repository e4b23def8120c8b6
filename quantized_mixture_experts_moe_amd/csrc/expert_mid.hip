// Expert phase of a batched decode step (a few tokens per call): every
// distinct selected expert is read once and applied to every token that
// chose it, and the shared expert is read once for all tokens.
//
// The pages fetch an expert once and let it serve every row routed to it
// (es.news.hada.io, "Proceso de generacion de tokens"); with a handful of
// tokens most experts are chosen by one token, so the saving is the
// repeated experts and, above all, the shared expert, which the per-token
// kernels read once per token.  The arithmetic per (token, weight) is that
// of the few-token kernels (4-bit codes into 128 + q via the mantissa, dot2
// against activation pairs for gate/up; exact codes and fp32 h for down),
// with the tokens of an expert in a loop over the weights held in registers.
//
// mid_glu_kernel:  grid (routed tiles T k F/64 + shared tiles F_s/64, KSg).
//   A routed tile belongs to slot l = (t, j); its block runs only if l is the
//   first slot (in token-major order) that selected its expert, and then
//   computes the tile for every slot of that expert.  The splits add their
//   partials as 64-bit fixed-point integers (units of 2^-32) with
//   device-scope atomics, so the sums do not depend on the arrival order; the
//   last split of a tile (counter) writes h = gelu(gate) * up and its 64-unit
//   sums per slot.
// mid_down_kernel: grid (D/64 output tiles, KSd splits of the units).  A unit
//   is 64 hidden rows of one distinct expert (or of the shared expert); the
//   block reads its down codes once and adds gate[t, j] * (W_d h[t, j]) for
//   every token of the expert (gate 1 for the shared expert).  Splits add
//   into fixed-point accumulators as above; the last split of an output
//   tile writes out.
// Accumulators and counters are zero between calls (the last arriver puts
// them back); a partial large enough to wrap a sum (|sum| < 2^31) counts in
// the workspace's error word.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNW = 4;    // waves per block
constexpr int kMaxG = 4;  // 64-column groups per wave and batch (gate/up)
constexpr int kMaxU = 4;  // units per wave and batch (down)
static_assert(kMaxMidGB == kNW * kMaxG, "a gate/up block's groups are one batch");

// Which slots selected the expert of slot l (ids: lane i < n holds ids[i]).
__device__ __forceinline__ uint64_t same_expert(int my_id, int l, int n) {
  const int e = __shfl(my_id, l, 64);
  const int lane = threadIdx.x & 63;
  return __ballot(lane < n && my_id == e);
}

// The compiler would hoist the unpacking of the codes out of a loop over
// tokens and keep every unpacked value live across it; an empty asm that
// "modifies" the code words inside the loop keeps the unpacking per token.
__device__ __forceinline__ void keep_packed(u32x4 &q) {
  asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
}

// Slot of token t within the slot mask m (one slot per token at most).
__device__ __forceinline__ int token_slot(uint64_t m, int t, int k) {
  const uint64_t kmask = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
  const uint64_t part = (m >> (t * k)) & kmask;
  return part ? t * k + (int)__builtin_ctzll(part) : -1;
}

template <bool F16X>
__global__ __launch_bounds__(kNW * 64) void mid_glu_kernel(MidLaunch m) {
  // per-wave, per-token partial sums (each wave owns its rows)
  __shared__ float red[kNW][2][kMaxMidT][64];
  const ExpertLaunch &a = m.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, k = a.k, nsl = T * k, D = a.D, G = D / 64;
  const int rbr = a.F / 64, nrt = nsl * rbr, rbs = a.Fs / 64;
  // routed tiles in KSg splits, then the shared tiles in KSs splits (they
  // serve every token, so they are split finer); the tile index runs
  // fastest, so the blocks in flight together read neighbouring rows
  const int nr = nrt * m.KSg;
  const int b = blockIdx.x;
  const int ks = b < nr ? b / nrt : (b - nr) / rbs;
  const int tile = b < nr ? b - ks * nrt : nrt + (b - nr) - ks * rbs;
  const int KS = b < nr ? m.KSg : m.KSs;
  const int g0 = ks * G / KS, g1 = (ks + 1) * G / KS;  // at most kMaxMidGB groups

  const uint8_t *blob = nullptr;
  int F, rb;
  uint64_t smask = 0;   // routed: slots of the expert
  bool routed;
  if (tile < nrt) {
    routed = true;
    const int l = tile / rbr;
    rb = tile - l * rbr;
    // the slot's blob (resolved by the router) and all ids, in one round trip
    const uint8_t *sb = (const uint8_t *)as_const(a.slot_blob)[l];
    const int my_id = lane < nsl ? a.ids[lane] : -1;
    smask = same_expert(my_id, l, nsl);
    if ((int)__builtin_ctzll(smask) != l) return;  // served by the expert's first slot
    const int e = __shfl(my_id, l, 64);
    if (e >= 0 && e < a.E) blob = sb;
    F = a.F;
  } else {
    routed = false;
    rb = tile - nrt;
    blob = (const uint8_t *)a.sblobs[0];
    F = a.Fs;
  }
  // hidden offset (in h) of token t's slot for this expert, -1 if none
  auto slot_hoff = [&](int t) -> long {
    if (!routed) return (long)nsl * a.F + (long)t * a.Fs;
    const int s = token_slot(smask, t, k);
    return s < 0 ? -1L : (long)s * a.F;
  };

  // this wave's groups of the block (one batch: at most kMaxMidGB groups)
  const int j = rb * 64 + lane;
  u32x4 qg0[kMaxG], qg1[kMaxG], qu0[kMaxG], qu1[kMaxG];
  uint32_t mg[kMaxG], mu[kMaxG];
  if (blob) {
    const BlobLayout L = blob_layout(D, F);
    const gptr<u32x4> gc = as_global((const u32x4 *)(blob + L.gate_codes) + j);
    const gptr<u32x4> uc = as_global((const u32x4 *)(blob + L.up_codes) + j);
    const gptr<uint32_t> gm = as_global((const uint32_t *)(blob + L.gate_meta) + j);
    const gptr<uint32_t> um = as_global((const uint32_t *)(blob + L.up_meta) + j);
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
  const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);
  // tokens in the outer loop (not unrolled): each token's activations are
  // scalar loads issued together, its two sums stay in registers, and the
  // codes are unpacked again per token (registers, not arithmetic, bound
  // this kernel: unpacked once, the codes would hold 64 more)
#pragma unroll 1
  for (int t = 0; t < T; ++t) {
    if (slot_hoff(t) < 0) continue;
    float ag = 0.0f, au = 0.0f;
    if (blob) {
#pragma unroll
      for (int i = 0; i < kMaxG; ++i) {
        const int g = g0 + wave + i * kNW;
        if (g >= g1) break;
        keep_packed(qg0[i]);
        keep_packed(qg1[i]);
        keep_packed(qu0[i]);
        keep_packed(qu1[i]);
        uint32_t xg[32];
        load_uniform(a.xp + (size_t)t * (D / 2) + g * 32, xg);
        float dg = dot_chunk<F16X>(qg0[i], xg, 0.0f, magic);
        dg = dot_chunk<F16X>(qg1[i], xg + 16, dg, magic);
        float du = dot_chunk<F16X>(qu0[i], xg, 0.0f, magic);
        du = dot_chunk<F16X>(qu1[i], xg + 16, du, magic);
        const float xsg = as_const(a.xs)[(size_t)t * G + g];
        const float sg = f16_to_f32(mg[i]), bg = f16_to_f32(mg[i] >> 16);
        const float su = f16_to_f32(mu[i]), bu = f16_to_f32(mu[i] >> 16);
        ag = fmaf(sg, dg, ag);
        ag = fmaf(fmaf(-Magic<F16X>::offset, sg, bg), xsg, ag);
        au = fmaf(su, du, au);
        au = fmaf(fmaf(-Magic<F16X>::offset, su, bu), xsg, au);
      }
    }
    red[wave][0][t][lane] = ag;
    red[wave][1][t][lane] = au;
  }
  __syncthreads();
  if (wave != 0) return;

  if (KS > 1) {
    // each split adds its partials into 64-bit fixed-point accumulators (one
    // pair of 64 words per hidden unit of a token's slot); integer addition
    // makes the sums the same in any arrival order
    bool range_ok = true;
    for (int t = 0; t < T; ++t) {
      const long ho = slot_hoff(t);
      if (ho < 0) continue;
      float vg = 0.0f, vu = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        vg += red[w][0][t][lane];
        vu += red[w][1][t][lane];
      }
      range_ok = range_ok && fabsf(vg) * (float)KS < 2147483648.0f &&
                 fabsf(vu) * (float)KS < 2147483648.0f;
      uint64_t *acc = m.gacc + ((size_t)ho / 64 + rb) * 128 + lane;
      __hip_atomic_fetch_add(acc, (uint64_t)to_fixed32(vg), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(acc + 64, (uint64_t)to_fixed32(vu), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!__all(range_ok) && lane == 0) add_dev(m.err, 1u);  // a sum could wrap
    wait_all_memory();
    uint32_t old = 0;
    if (lane == 0) old = add_dev(m.gcnt + tile, 1u);
    old = __shfl(old, 0, 64);
    if (old != (uint32_t)(KS - 1)) return;
  }
  // the last split: every token's sums in flight at once
  float vg[kMaxMidT], vu[kMaxMidT];
#pragma unroll
  for (int t = 0; t < kMaxMidT; ++t) {
    vg[t] = vu[t] = 0.0f;
    const long ho = t < T ? slot_hoff(t) : -1L;
    if (ho < 0) continue;
    if (KS > 1) {
      const uint64_t *acc = m.gacc + ((size_t)ho / 64 + rb) * 128 + lane;
      vg[t] = from_fixed32((long long)ld_dev(acc));
      vu[t] = from_fixed32((long long)ld_dev(acc + 64));
    } else {
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        vg[t] += red[w][0][t][lane];
        vu[t] += red[w][1][t][lane];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxMidT; ++t) {
    const long ho = t < T ? slot_hoff(t) : -1L;
    if (ho < 0) continue;
    const float h = blob ? gelu_tanh(vg[t]) * vu[t] : 0.0f;
    const size_t unit = (size_t)ho + (size_t)rb * 64;
    a.h[unit + lane] = h;
    const float hsum = wave_sum(h);
    if (lane == 0) a.hs[unit / 64] = hsum;
    if (KS > 1) {
      uint64_t *acc = m.gacc + ((size_t)ho / 64 + rb) * 128 + lane;
      st_dev(acc, (uint64_t)0);
      st_dev(acc + 64, (uint64_t)0);
    }
  }
  if (KS > 1 && lane == 0) st_dev(m.gcnt + tile, 0u);
}

__global__ __launch_bounds__(kNW * 64) void mid_down_kernel(MidLaunch m) {
  constexpr int kRows = kMaxU * kMaxMidT;  // (unit, token) pairs of a wave's batch
  // per-wave, per-token partial sums (each wave owns its rows)
  __shared__ float red[kNW][kMaxMidT][64];
  // each wave's hidden values (64 per pair) and their sums
  __shared__ float hl[kNW][kRows][64];
  __shared__ float hsl[kNW][kRows];
  const ExpertLaunch &a = m.a;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = a.T, k = a.k, nsl = T * k, D = a.D;
  const int nb = blockIdx.x, ksd = blockIdx.y, KS = gridDim.y;
  const int n = nb * 64 + lane;
  const int Gf = a.F / 64, Gs = a.sblobs ? a.Fs / 64 : 0;
  const int U = nsl * Gf + Gs;
  // split ksd takes the units ksd, ksd + KS, ...: the shared units (every
  // token) and the routed ones (mostly one token) spread over all splits
  const int nu = (U - ksd + KS - 1) / KS;
  const int my_id = lane < nsl ? a.ids[lane] : -1;
  const float my_gate = lane < nsl ? a.gates[lane] : 0.0f;

  for (int t = 0; t < T; ++t) red[wave][t][lane] = 0.0f;
  for (int base = 0; base < nu; base += kNW * kMaxU) {
    u32x4 q0[kMaxU], q1[kMaxU];
    uint32_t mw[kMaxU];
    uint64_t sm[kMaxU];  // routed: slots of the unit's expert; 0: shared
    int gg[kMaxU];
    bool use[kMaxU];
#pragma unroll
    for (int i = 0; i < kMaxU; ++i) {
      const int u = ksd + KS * min(base + wave + i * kNW, nu - 1);
      use[i] = base + wave + i * kNW < nu;
      const uint8_t *blob;
      int Fb;
      if (u < nsl * Gf) {
        const int l = u / Gf;
        gg[i] = u - l * Gf;
        sm[i] = same_expert(my_id, l, nsl);
        const int e = __shfl(my_id, l, 64);
        const bool ok = e >= 0 && e < a.E;
        use[i] = use[i] && ok && (int)__builtin_ctzll(sm[i]) == l;
        blob = (const uint8_t *)as_const(a.slot_blob)[ok ? l : 0];
        Fb = a.F;
      } else {
        gg[i] = u - nsl * Gf;
        sm[i] = 0;
        blob = (const uint8_t *)a.sblobs[0];
        Fb = a.Fs;
      }
      const BlobLayout L = blob_layout(D, Fb);
      const gptr<u32x4> dc = as_global((const u32x4 *)(blob + L.down_codes) + n);
      q0[i] = dc[(size_t)(2 * gg[i]) * D];
      q1[i] = dc[(size_t)(2 * gg[i] + 1) * D];
      mw[i] = as_global((const uint32_t *)(blob + L.down_meta))[(size_t)gg[i] * D + n];
    }
    // hidden offset of pair (i, t) in h, -1 if unit i has no token t
    auto pair_hoff = [&](int i, int t) -> long {
      if (!use[i]) return -1L;
      if (!sm[i]) return (long)nsl * a.F + (long)t * a.Fs;
      const int sl = token_slot(sm[i], t, k);
      return sl < 0 ? -1L : (long)sl * a.F;
    };
    // the hidden values of every pair (row i T + t) in one round trip: each
    // lane loads 16-byte pieces of the rows, then they go through LDS
    constexpr int kPieces = kRows * 16 / 64;
    u32x4 hv[kPieces];
    const int nrow = kMaxU * T;
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int c = lane + 64 * q, row = c >> 4, col = c & 15;
      const int i = row / T, t = row - (row / T) * T;
      long ho = -1;
#pragma unroll
      for (int ii = 0; ii < kMaxU; ++ii)
        if (ii == i && row < nrow) ho = pair_hoff(ii, t);
      hv[q] = ho < 0 ? u32x4{0u, 0u, 0u, 0u}
                     : as_global((const u32x4 *)(a.h + ho + (size_t)gg[i & (kMaxU - 1)] * 64))[col];
    }
    float hsv = 0.0f;
    {
      const int i = lane / T, t = lane - (lane / T) * T;
      long ho = -1;
#pragma unroll
      for (int ii = 0; ii < kMaxU; ++ii)
        if (ii == i && lane < nrow) ho = pair_hoff(ii, t);
      if (ho >= 0) hsv = a.hs[ho / 64 + gg[i & (kMaxU - 1)]];
    }
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      const int c = lane + 64 * q, row = c >> 4, col = c & 15;
      if (row < nrow) *(u32x4 *)&hl[wave][row][col * 4] = hv[q];
    }
    if (lane < nrow) hsl[wave][lane] = hsv;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // tokens in the outer loop (not unrolled), units inside
#pragma unroll 1
    for (int t = 0; t < T; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < kMaxU; ++i) {
        const long ho = pair_hoff(i, t);
        if (ho < 0) continue;
        const float gate = sm[i] ? __shfl(my_gate, token_slot(sm[i], t, k), 64) : 1.0f;
        keep_packed(q0[i]);
        keep_packed(q1[i]);
        const float d = dot_group_f32(q0[i], q1[i], &hl[wave][i * T + t][0]);
        const float s = f16_to_f32(mw[i]), bb = f16_to_f32(mw[i] >> 16);
        acc = fmaf(gate, fmaf(s, d, bb * hsl[wave][i * T + t]), acc);
      }
      red[wave][t][lane] += acc;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (wave != 0) return;
  if (KS > 1) {
    // fixed-point accumulators of the output rows (as for gate/up)
    bool range_ok = true;
    for (int t = 0; t < T; ++t) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) v += red[w][t][lane];
      range_ok = range_ok && fabsf(v) * (float)KS < 2147483648.0f;
      __hip_atomic_fetch_add(m.dacc + (size_t)t * D + n, (uint64_t)to_fixed32(v),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!__all(range_ok) && lane == 0) add_dev(m.err, 1u);
    wait_all_memory();
    uint32_t old = 0;
    if (lane == 0) old = add_dev(m.dcnt + nb, 1u);
    old = __shfl(old, 0, 64);
    if (old != (uint32_t)(KS - 1)) return;
  }
  float v[kMaxMidT];
#pragma unroll
  for (int t = 0; t < kMaxMidT; ++t) {
    v[t] = 0.0f;
    if (t >= T) continue;
    if (KS > 1) {
      v[t] = from_fixed32((long long)ld_dev(m.dacc + (size_t)t * D + n));
    } else {
#pragma unroll
      for (int w = 0; w < kNW; ++w) v[t] += red[w][t][lane];
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxMidT; ++t) {
    if (t >= T) continue;
    const size_t idx = (size_t)t * D + n;
    if (a.out_dtype == MOE_F32)
      ((float *)a.out)[idx] = v[t];
    else if (a.out_dtype == MOE_BF16)
      ((uint16_t *)a.out)[idx] = (uint16_t)f32_to_bf16(v[t]);
    else
      ((uint16_t *)a.out)[idx] = (uint16_t)f32_to_f16(v[t]);
    if (KS > 1) st_dev(m.dacc + idx, (uint64_t)0);
  }
  if (KS > 1 && lane == 0) st_dev(m.dcnt + nb, 0u);
}

}  // namespace

// Splits of the two kernels: about 2,048 gate/up blocks (counting the tiles
// of repeated slots, which exit at once) with at least one 64-column group
// per wave, and down splits of about 16 units (4 per wave); both bounded by
// the workspace's partial areas.
void plan_mid(MidLaunch *m) {
  const ExpertLaunch &a = m->a;
  const int G = a.D / 64, nsl = a.T * a.k;
  const int tiles = nsl * (a.F / 64) + (a.sblobs ? a.Fs / 64 : 0);
  int ksg = tuning().mid_ksg > 0 ? tuning().mid_ksg : (1024 + tiles - 1) / tiles;
  // a block takes at most kMaxMidGB (= one group per wave and register slot)
  const int ksg_min = (G + kMaxMidGB - 1) / kMaxMidGB;
  if (ksg < ksg_min) ksg = ksg_min;
  if (ksg > G) ksg = G;
  if (ksg > kMaxMidKS) ksg = kMaxMidKS;
  const int U = nsl * (a.F / 64) + (a.sblobs ? a.Fs / 64 : 0);
  int ksd = tuning().mid_ksd > 0 ? tuning().mid_ksd : (U + kNW * kMaxU - 1) / (kNW * kMaxU);
  if (ksd > U) ksd = U;
  if (ksd > kMaxMidKSd) ksd = kMaxMidKSd;
  m->KSg = ksg < 1 ? 1 : ksg;
  m->KSd = ksd < 1 ? 1 : ksd;
  // the shared tiles: about one 64-column group per wave and token pair
  // (T tokens at one group per wave, fewer tokens at more), at least the
  // routed split
  int kss = tuning().mid_kss > 0 ? tuning().mid_kss
                                 : (G * a.T + kNW * 4 - 1) / (kNW * 4);
  if (kss < m->KSg) kss = m->KSg;
  if (kss > G) kss = G;
  if (kss > kMaxMidKS) kss = kMaxMidKS;
  m->KSs = kss;
  m->n_tiles = tiles;
  m->n_blocks = nsl * (a.F / 64) * m->KSg + (a.sblobs ? a.Fs / 64 : 0) * m->KSs;
}

hipError_t launch_mid(const MidLaunch &m, hipStream_t s) {
  const int NB = m.a.D / 64;
  if (m.a.f16x)
    hipLaunchKernelGGL((mid_glu_kernel<true>), dim3(m.n_blocks), dim3(kNW * 64), 0, s, m);
  else
    hipLaunchKernelGGL((mid_glu_kernel<false>), dim3(m.n_blocks), dim3(kNW * 64), 0, s, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mid_down_kernel, dim3(NB, m.KSd), dim3(kNW * 64), 0, s, m);
  return hipGetLastError();
}

}  // namespace moe
