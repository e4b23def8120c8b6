// One launch for the whole routed MoE layer of a decode step: router GEMV,
// top-k and gates, gate/up GLU of the selected and the shared experts, down
// projection and the weighted combine.
//
// Per token the pages score the experts with the resident 8-bit router, take
// the top 8, run the selected 4-bit experts and the resident shared expert,
// and add the two outputs (es.news.hada.io, "Proceso de generacion de
// tokens"; yodev.dev, "Por que funciona: el A4B del nombre").  Routing is a
// short chain of dependent steps; the shared expert does not depend on it.
// So the grid has three groups of blocks:
//   router blocks: the router rows (4 experts per block).  They publish their
//     logits; by default every routed block then ranks all of a token's
//     logits itself (layer_select 1), else wave 0 of every router block
//     ranks its own candidates against all logits and publishes the
//     selection lines (layer_select 0, and the streamed two-launch variant);
//   routed blocks: the routed gate/up tiles and the routed part of the down
//     projection.  They issue no weight loads before the selection arrives,
//     so their polls are not queued behind outstanding loads (a wave's loads
//     complete in order);
//   shared blocks: the shared expert's gate/up tiles and its part of the down
//     projection; they stream from the first cycle, while routing runs.
//
// Handoffs between blocks are tagged words: a 64-bit store of (value, tag)
// with device scope, where the tag is the call's epoch.  A reader loads until
// every word it needs carries the current tag, so nothing has to be reset
// between calls and no full-cache fence is needed.  Each block keeps its own
// copy of the epoch (bep[b]); every block advances all copies in lockstep, so
// they agree for any grid size.  The split reductions (gate/up over column
// groups, output over units) add fixed-point partials with integer atomics;
// the last split to arrive finishes (deterministic in any arrival order).
// All blocks of the grid must be resident at once (checked on the host);
// every wait is bounded and a timeout bumps an error counter.
//
// Work split (one token, k = 8, D = 2816, F = 704, F_s = 2112):
//   router:  32 blocks of 4 experts;
//   gate/up: 88 routed + 33 shared tiles of 64 hidden rows x KSg reduction
//            splits over the 44 column groups;
//   down:    44 tiles of 64 output rows x (KSdr splits of the 88 routed units
//            + KSds splits of the 33 shared units); a unit is 64 hidden rows
//            of one slot.
#include <float.h>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNW = 4;
constexpr int kThreads = kNW * 64;
constexpr int kRows = 4;                   // experts per router block
constexpr int kRT = 2;                     // tokens per router block
constexpr int kKL = kThreads / kRows;      // threads splitting one router row
constexpr long kSpin = 1L << 20;           // bounded waits, then the error counter

__device__ __forceinline__ uint64_t ld_dev64(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(uint32_t bits, uint32_t tag) {
  return (uint64_t)bits | ((uint64_t)tag << 32);
}
__device__ __forceinline__ bool has_tag(uint64_t v, uint32_t tag) {
  return (uint32_t)(v >> 32) == tag;
}

// Wave-wide: loads the rows p[j * stride + lane] (j < n <= N, lane < lanes)
// until every word carries `tag`, all rows in one round trip per try;
// out[j] = value word.
template <int N>
__device__ __forceinline__ int wait_rows(const uint64_t *p, size_t stride, int n, uint32_t tag,
                                         uint32_t *err, uint32_t (&out)[N], int lanes = 64) {
  const int lane = threadIdx.x & 63;
  for (long s = 0;; ++s) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      out[j] = 0u;
      if (j < n && lane < lanes) {
        const uint64_t v = ld_dev64(p + (size_t)j * stride + lane);
        ok = ok && has_tag(v, tag);
        out[j] = (uint32_t)v;
      }
    }
    if (__all(ok)) return (int)s;
    if (s > kSpin) {
      if (lane == 0) add_dev(err, 1u);
      return (int)s;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Wave-wide: polls one word per lane (p, or nothing where p is null) until
// each carries `tag`.  Waiting on one word per producer store keeps the
// polling traffic small; the data is read (and checked) afterwards.
// Two polls are in flight: the next one is issued before the previous one is
// checked, so a store is seen about half a round trip after it lands rather
// than a whole one.  Lanes with `active` false poll p too (any valid word)
// and count as done.
__device__ __forceinline__ int wait_hint(const uint64_t *p, bool active, uint32_t tag,
                                         uint32_t *err) {
  const int lane = threadIdx.x & 63;
  uint64_t w = ld_dev64(p);
  for (long s = 0;; ++s) {
    __builtin_amdgcn_s_sleep(1);
    const uint64_t nx = ld_dev64(p);
    if (__all(!active || has_tag(w, tag))) return (int)s;
    if (s > kSpin) {
      if (lane == 0) add_dev(err, 1u);
      return (int)s;
    }
    w = nx;
  }
}

// Counted fixed-point reduction, one device-scope atomic per value: the
// 64-bit word holds the sum of the partials, rounded to multiples of 2^-28,
// in bits 8..63 and the number of partials added so far in bits 0..7.  The
// returned word tells each lane whether its add completed the n partials;
// that lane alone gets the sum (integer addition: the same for any arrival
// order) and puts the word back to zero for the next call.  Sums must stay
// below 2^27 in magnitude; a partial that could break that counts in *err.
__device__ __forceinline__ bool counted_add(uint64_t *word, float v, int n, float *sum,
                                            uint32_t *err) {
  // a partial outside |v| < 2^27 / n (or not finite) could wrap the sum:
  // counted as an error of the call
  if (!(fabsf(v) * (float)n < 134217728.0f)) add_dev(err, 1u);
  const uint64_t add = ((uint64_t)__double2ll_rn((double)v * 268435456.0) << 8) + 1u;
  const uint64_t old =
      __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old & 0xFFu) != (uint64_t)(n - 1)) return false;
  *sum = (float)((double)((long long)(old + add) >> 8) * (1.0 / 268435456.0));
  st_dev64(word, 0u);
  return true;
}

// Two counted adds (as counted_add) whose atomics are issued together, so
// that both take one round trip: done0 / done1 tell whether this lane's add
// completed that word's n partials (then *s0 / *s1 hold the sum).
__device__ __forceinline__ void counted_add2(uint64_t *w0, float v0, uint64_t *w1, float v1, int n,
                                             bool *done0, float *s0, bool *done1, float *s1,
                                             uint32_t *err) {
  const uint64_t a0 = ((uint64_t)__double2ll_rn((double)v0 * 268435456.0) << 8) + 1u;
  const uint64_t a1 = ((uint64_t)__double2ll_rn((double)v1 * 268435456.0) << 8) + 1u;
  const uint64_t o0 = __hip_atomic_fetch_add(w0, a0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t o1 = __hip_atomic_fetch_add(w1, a1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // a partial outside |v| < 2^27 / n (or not finite) could wrap its sum
  if (!(fabsf(v0) * (float)n < 134217728.0f) || !(fabsf(v1) * (float)n < 134217728.0f))
    add_dev(err, 1u);
  *done0 = (o0 & 0xFFu) == (uint64_t)(n - 1);
  *done1 = (o1 & 0xFFu) == (uint64_t)(n - 1);
  if (*done0) {
    *s0 = (float)((double)((long long)(o0 + a0) >> 8) * (1.0 / 268435456.0));
    st_dev64(w0, 0u);
  }
  if (*done1) {
    *s1 = (float)((double)((long long)(o1 + a1) >> 8) * (1.0 / 268435456.0));
    st_dev64(w1, 0u);
  }
}

template <bool F16X>
__device__ __forceinline__ float x_to_f32(uint32_t v) {
  return F16X ? f16_to_f32(v) : bf16_to_f32(v);
}

struct Tile {
  int slot, t, j, rb, F;  // j: slot within the token (-1: shared expert)
  size_t hoff;
};

__device__ __forceinline__ Tile glu_tile(const LayerLaunch &L, int tile) {
  Tile g;
  const int rbr = L.F / 64, n_rt = L.T * L.k * rbr;
  if (tile < n_rt) {
    g.slot = tile / rbr;
    g.rb = tile - g.slot * rbr;
    g.t = g.slot / L.k;
    g.j = g.slot - g.t * L.k;
    g.F = L.F;
    g.hoff = (size_t)g.slot * L.F;
  } else {
    const int rbs = L.Fs / 64, b2 = tile - n_rt;
    g.t = b2 / rbs;
    g.rb = b2 - g.t * rbs;
    g.slot = L.T * L.k + g.t;
    g.j = -1;
    g.F = L.Fs;
    g.hoff = (size_t)L.T * L.k * L.F + (size_t)g.t * L.Fs;
  }
  return g;
}

// Selection for token t, shared by the router blocks of the token: once every
// logit of the token is published, each router block ranks its own kRows
// candidates against all E logits and publishes every candidate that ranks
// below k in that rank's place (in each copy of the selection line).  Keys
// are unique 64-bit values (order-preserving logit bits, then the
// complemented index), so the ranks of all candidates are a permutation and
// equal logits rank the lower index first.  The line then holds, at place r,
// the expert with the r-th largest logit and that logit; a consumer computes
// the softmax gates itself.  The block's own keys are in own[] (written when
// its logits were published); a rank is a count of set ballot bits.
struct __align__(16) SelectLds {
  uint64_t own[kRows];
};

// Wave 0 of a router block: polls the E logits of token t (lanes hold
// experts lane, lane + 64, ...), ranks the own candidates with ballots and
// publishes the winners.
template <bool HS>
__device__ void select_publish(const LayerLaunch &L, int t, int e0, uint32_t tag,
                               const SelectLds &S) {
  constexpr int NV = kMaxLayerE / 64;
  constexpr int LPC = 64 / kRows;  // lanes per candidate when publishing
  const int lane = threadIdx.x & 63, E = L.E, k = L.k;
  const uint64_t *lg = L.rlog + (size_t)t * E;
  // two polls in flight (see wait_hint); lanes past E poll expert E - 1
  uint64_t w[NV], nx[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) w[j] = ld_dev64(lg + min(lane + 64 * j, E - 1));
  for (long s = 0;; ++s) {
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < NV; ++j) nx[j] = ld_dev64(lg + min(lane + 64 * j, E - 1));
    bool ok = true;
#pragma unroll
    for (int j = 0; j < NV; ++j) ok = ok && (lane + 64 * j >= E || has_tag(w[j], tag));
    if (__all(ok)) break;
    if (s > kSpin) {
      if (lane == 0) add_dev(L.err, 1u);
      break;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) w[j] = nx[j];
  }
  uint64_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? ((uint64_t)order_key(__uint_as_float((uint32_t)w[j])) << 32) |
                         (uint64_t)(~(uint32_t)e)
                   : 0;
  }
  // rank of candidate c = number of keys above its key (keys past E are 0)
  const int c = lane / LPC, p = lane % LPC, e = e0 + c;
  uint32_t r = 0;
#pragma unroll
  for (int cc = 0; cc < kRows; ++cc) {
    const uint64_t kc = S.own[cc];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) cnt += (uint32_t)__popcll(__ballot(key[j] > kc));
    if (c == cc) r = cnt;
  }
  if (e < E && r < (uint32_t)k) {
    const uint32_t vbits = __float_as_uint(key_value((uint32_t)(S.own[c] >> 32)));
    for (int cp = p; cp < L.sel_copies; cp += LPC) {
      uint64_t *line = L.sel + ((size_t)t * L.sel_copies + cp) * L.sel_stride;
      st_dev64(line + r, tagged((uint32_t)e, tag));
      st_dev64(line + L.lid + r, tagged(vbits, tag));
    }
    if constexpr (HS) {
      if (p == 0)  // the host's copy of the selection (one 64-bit word)
        __hip_atomic_store(L.host_sel + (size_t)t * k + r, tagged((uint32_t)e, L.host_epoch),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// The selection of token t as published in one copy (wave-wide, bounded
// wait): lane r < k receives the blob of the r-th expert and its softmax gate
// (the max is the rank-0 logit; the same arithmetic, in the same order, as
// the router kernel's selection).  `report`: also write ids_out / gates_out.
template <bool BY_RANK = false>
__device__ void wait_selection(const LayerLaunch &L, int t, int copy, uint32_t tag,
                               const void *const *table, const uint8_t **blob_out,
                               float *gate_out, bool report) {
  const int lane = threadIdx.x & 63, k = L.k;
  const uint64_t *line = L.sel + ((size_t)t * L.sel_copies + copy) * L.sel_stride;
  // two polls in flight (see wait_hint); lanes past k poll place k - 1
  const int r = min(lane, k - 1);
  uint64_t wi = ld_dev64(line + r), wg = ld_dev64(line + L.lid + r);
  for (long s = 0;; ++s) {
    __builtin_amdgcn_s_sleep(1);
    const uint64_t ni = ld_dev64(line + r), ng = ld_dev64(line + L.lid + r);
    if (__all(lane >= k || (has_tag(wi, tag) && has_tag(wg, tag)))) break;
    if (s > kSpin) {
      if (lane == 0) add_dev(L.err, 1u);
      break;
    }
    wi = ni;
    wg = ng;
  }
  const uint32_t id = min((uint32_t)wi, (uint32_t)L.E - 1);
  if (lane < k) blob_out[lane] = (const uint8_t *)table[BY_RANK ? (uint32_t)lane : id];
  const float myv = lane < k ? __uint_as_float((uint32_t)wg) : 0.0f;
  const float m0 =
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myv), 0));
  const float z = lane < k ? expf(myv - m0) : 0.0f;
  const float sum = wave_sum(z);
  const float gate = z / sum;
  if (lane < k) {
    gate_out[lane] = gate;
    if (report) {
      if (L.ids_out) L.ids_out[(size_t)t * k + lane] = (int32_t)id;
      if (L.gates_out) L.gates_out[(size_t)t * k + lane] = gate;
    }
  }
}

// The selection of token t from its E logits in one copy (wave-wide, bounded
// wait, two polls in flight): the top k and their softmax gates by the same
// selection (larger logit first, ties to the lower index) and the same gate
// arithmetic as the router kernel's; lane r < k receives the blob of the
// r-th expert and its gate.  `report`: also write ids_out / gates_out.
__device__ void select_from_logits(const LayerLaunch &L, int t, int copy, uint32_t tag,
                                   const void *const *table, const uint8_t **blob_out,
                                   float *gate_out, bool report, uint2 *xch) {
  constexpr int NV = kMaxLayerE / 64;
  const int lane = threadIdx.x & 63, E = L.E, k = L.k;
  const uint64_t *lg = L.rlog + ((size_t)copy * L.T + t) * E;
  uint64_t w[NV], nx[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) w[j] = ld_dev64(lg + min(lane + 64 * j, E - 1));
  for (long s = 0;; ++s) {
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < NV; ++j) nx[j] = ld_dev64(lg + min(lane + 64 * j, E - 1));
    bool ok = true;
#pragma unroll
    for (int j = 0; j < NV; ++j) ok = ok && (lane + 64 * j >= E || has_tag(w[j], tag));
    if (__all(ok)) break;
    if (s > kSpin) {
      if (lane == 0) add_dev(L.err, 1u);
      break;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) w[j] = nx[j];
  }
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j)
    v[j] = lane + 64 * j < E ? __uint_as_float((uint32_t)w[j]) : -INFINITY;
  // k rounds of a wave maximum (two registers per lane up to 128 experts),
  // then the router kernel's gate arithmetic: same ids and gates, bit for bit
  int32_t id;
  float myv;
  if (E <= 128) {
    const float v2[2] = {v[0], v[1]};
    topk_rounds(v2, E, k, &id, &myv);
  } else {
    topk_rounds(v, E, k, &id, &myv);
  }
  if (lane >= k) myv = 0.0f;
  const float m0 =
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myv), 0));
  const float z = lane < k ? expf(myv - m0) : 0.0f;
  const float gate = z / wave_sum(z);
  (void)xch;
  const uint32_t ids = min((uint32_t)id, (uint32_t)E - 1);
  if (lane < k) {
    blob_out[lane] = (const uint8_t *)table[ids];
    gate_out[lane] = gate;
    if (report) {
      if (L.ids_out) L.ids_out[(size_t)t * k + lane] = (int32_t)ids;
      if (L.gates_out) L.gates_out[(size_t)t * k + lane] = gate;
    }
  }
}

constexpr int kMaxBlockGroups = 16;  // gate/up column groups of one block (4 waves x 4)
constexpr int kDW = kNW - 1;         // waves with down units (1..3)

// Weights of one block, held in registers from issue to use.  Every load is
// issued unconditionally (indices clamped into range where a block has less
// work), so each wave's loads count the same on every path and the waits
// the compiler places before a use cover exactly the loads that use needs
// (a wave's loads complete in order).
template <int M>
struct GluRegs {
  u32x4 qg0[M], qg1[M], qu0[M], qu1[M];
  uint32_t mg[M], mu[M];
};
template <int M>
struct DownRegs {
  u32x4 dq0[M], dq1[M];
  uint32_t dmw[M];
};

// gate/up rows rb*64 + lane of the 64-column groups g0 + wave + 4 i (clamped)
template <int M>
__device__ __forceinline__ void issue_glu(GluRegs<M> &R, const uint8_t *blob, int D, int F, int rb,
                                          int g0, int g1, int wave, int lane) {
  const int j = rb * 64 + lane;
  const BlobLayout BL = blob_layout(D, F);
  const gptr<u32x4> gc = as_global((const u32x4 *)(blob + BL.gate_codes) + j);
  const gptr<u32x4> uc = as_global((const u32x4 *)(blob + BL.up_codes) + j);
  const gptr<uint32_t> gm = as_global((const uint32_t *)(blob + BL.gate_meta) + j);
  const gptr<uint32_t> um = as_global((const uint32_t *)(blob + BL.up_meta) + j);
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int g = min(g0 + wave + i * kNW, g1 - 1);
    const size_t c0 = (size_t)(2 * g) * F;
    R.qg0[i] = gc[c0];
    R.qg1[i] = gc[c0 + F];
    R.qu0[i] = uc[c0];
    R.qu1[i] = uc[c0 + F];
    R.mg[i] = gm[(size_t)g * F];
    R.mu[i] = um[(size_t)g * F];
  }
}

// down weights of output row n, hidden group g (64 hidden rows) of a blob
template <int M>
__device__ __forceinline__ void issue_down(DownRegs<M> &R, int i, const uint8_t *blob, int D,
                                           int Fb, int g, int n) {
  const BlobLayout BL = blob_layout(D, Fb);
  const gptr<u32x4> dc = as_global((const u32x4 *)(blob + BL.down_codes) + n);
  R.dq0[i] = dc[(size_t)(2 * g) * D];
  R.dq1[i] = dc[(size_t)(2 * g + 1) * D];
  R.dmw[i] = as_global((const uint32_t *)(blob + BL.down_meta))[(size_t)g * D + n];
}

// x of token t, columns [64 g0, 64 g1): thread i < 8 (g1 - g0) loads columns
// 8i..8i+7 (clamped for the others)
__device__ __forceinline__ u32x4 issue_x(const LayerLaunch &L, int t, int g0, int g1, int tid) {
  const int c = min(tid, (g1 - g0) * 8 - 1);
  return as_global((const u32x4 *)((const uint16_t *)L.x + (size_t)t * L.D + 64 * g0))[c];
}

// activation pairs (x[8w + m], x[8w + m + 4]) and 64-column sums into LDS
template <bool F16X>
__device__ __forceinline__ void stage_x(u32x4 xq, int n8, int tid, uint32_t *s_xp, float *s_xs) {
  const uint32_t a0 = xq.x, a1 = xq.y, a2 = xq.z, a3 = xq.w;
  u32x4 pq;
  pq.x = (a0 & 0xFFFFu) | (a2 << 16);
  pq.y = (a0 >> 16) | (a2 & 0xFFFF0000u);
  pq.z = (a1 & 0xFFFFu) | (a3 << 16);
  pq.w = (a1 >> 16) | (a3 & 0xFFFF0000u);
  const uint32_t w[4] = {a0, a1, a2, a3};
  float s8 = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    s8 += x_to_f32<F16X>(w[m] & 0xFFFFu);
    s8 += x_to_f32<F16X>(w[m] >> 16);
  }
  const float sg = sum8_lanes(s8);
  if (tid < n8) {
    *(u32x4 *)&s_xp[4 * tid] = pq;
    if ((tid & 7) == 0) s_xs[tid / 8] = sg;
  }
}

// Gate/up dot products of hidden row l on the matrix cores: lane l holds
// word w (8 columns) of row l as the B operand; lanes 0, 20, 40, 60 hold the
// activation pairs of word w as A rows 0, 4, 8, 12 (the other lanes zero),
// so D row 4q, column c -- register 0 of lane 16q + c -- accumulates row l's
// dot product.  Per 64-column group the affine terms fold in fp32.
template <bool F16X, int M>
__device__ __forceinline__ void glu_dots(const GluRegs<M> &R, const uint32_t *s_xp,
                                         const float *s_xs, int g0, int g1, int wave, int lane,
                                         float &accg, float &accu) {
  const bool xa_lane = (lane & 15) == 4 * (lane >> 4);
  const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);
  accg = 0.0f;
  accu = 0.0f;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int gi = wave + i * kNW;  // group g0 + gi
    if (g0 + gi < g1) {
      f32x4 dg = {0.0f, 0.0f, 0.0f, 0.0f}, du = {0.0f, 0.0f, 0.0f, 0.0f};
      const uint32_t wg[8] = {R.qg0[i].x, R.qg0[i].y, R.qg0[i].z, R.qg0[i].w,
                              R.qg1[i].x, R.qg1[i].y, R.qg1[i].z, R.qg1[i].w};
      const uint32_t wu[8] = {R.qu0[i].x, R.qu0[i].y, R.qu0[i].z, R.qu0[i].w,
                              R.qu1[i].x, R.qu1[i].y, R.qu1[i].z, R.qu1[i].w};
      // the four A lanes read all 8 words at once, the other lanes keep zeros
      u32x4 a[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) a[w] = u32x4{0u, 0u, 0u, 0u};
      if (xa_lane) {
#pragma unroll
        for (int w = 0; w < 8; ++w) a[w] = *(const u32x4 *)&s_xp[32 * gi + 4 * w];
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        dg = mma16<F16X>(a[w], code_pairs(wg[w], magic), dg);
        du = mma16<F16X>(a[w], code_pairs(wu[w], magic), du);
      }
      const float xsg = s_xs[gi];
      const float sg = f16_to_f32(R.mg[i]), bg = f16_to_f32(R.mg[i] >> 16);
      const float su = f16_to_f32(R.mu[i]), bu = f16_to_f32(R.mu[i] >> 16);
      accg = fmaf(sg, dg[0], accg);
      accg = fmaf(fmaf(-Magic<F16X>::offset, sg, bg), xsg, accg);
      accu = fmaf(su, du[0], accu);
      accu = fmaf(fmaf(-Magic<F16X>::offset, su, bu), xsg, accu);
    }
  }
}

// Block-wide sum of the gate/up partials (each wave has put its partials in
// red[]), then the split reduction: the split that completes a gate sum
// publishes gelu(gate), the one that completes an up sum publishes up (the
// consumer multiplies).
template <bool PAIR>
__device__ __forceinline__ void glu_publish(const LayerLaunch &L, float (&red)[kNW][2][64],
                                            int tile, size_t ho, int wave, int lane,
                                            uint32_t tag) {
  __syncthreads();
  if (wave == 0) {
    float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      v0 += red[w][0][lane];
      v1 += red[w][1][lane];
    }
    float g = v0, u = v1;
    bool last_g = true, last_u = true;
    if (L.KSg > 1) {
      // the two atomics in one round trip (PAIR), or one after the other:
      // measured, the pair is faster in the residual block's kernel (20.0
      // against 20.8 us per step) and slower in the plain layer's (16.7
      // against 16.2 us)
      uint64_t *wg = L.gacc + (size_t)tile * 128 + lane;
      if constexpr (PAIR) {
        counted_add2(wg, v0, wg + 64, v1, L.KSg, &last_g, &g, &last_u, &u, L.err);
      } else {
        last_g = counted_add(wg, v0, L.KSg, &g, L.err);
        last_u = counted_add(wg + 64, v1, L.KSg, &u, L.err);
      }
    }
    if (last_g) st_dev64(L.hg + ho + lane, tagged(__float_as_uint(gelu_tanh(g)), tag));
    if (last_u) st_dev64(L.hu + ho + lane, tagged(__float_as_uint(u), tag));
  }
}

// The residual block's post-norm of token t, by a router block once its
// routing is done.  The lanes that complete output elements store them as
// tagged words and add their number to the token's counter; one wave polls
// that single word until it reaches D (polling the whole row instead put
// kilobytes of device-scope loads per round on a few memory channels and
// slowed the layer), then the block reads the row, checking every word's
// epoch (a count may land before its stores), normalises it (w_post) and
// adds the residual row x into out.  Thread tid takes chunks tid, tid + 256,
// ..., the fixed summation order of the separate post-norm kernel (same
// bits).  The counter goes back to zero for the next call.
template <bool F16X, int NX>
__device__ __forceinline__ void post_norm_poll(const LayerLaunch &L, int t, uint32_t tag,
                                               float *red4) {
  const int tid = threadIdx.x, D = L.D, nch = D / 8;
  const uint64_t *yr = L.ybuf + (size_t)t * D;
  const gptr<u32x4> xr = as_global((const u32x4 *)((const uint16_t *)L.x + (size_t)t * D));
  const float4 *w4 = (const float4 *)L.w_post;
  u32x4 xq[NX];
  float4 wa[NX], wb[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int c = min(tid + i * kThreads, nch - 1);
    xq[i] = xr[c];
    wa[i] = w4[2 * c];
    wb[i] = w4[2 * c + 1];
  }
  if (threadIdx.x < 64) {
    for (long s = 0;; ++s) {
      if (ld_dev(L.ocnt + t) >= (uint32_t)D) break;
      if (s > kSpin) {
        if (tid == 0) add_dev(L.err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  float yv[NX][8];
  for (long s = 0;; ++s) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int c = min(tid + i * kThreads, nch - 1);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint64_t v = ld_dev64(yr + 8 * c + m);
        ok = ok && has_tag(v, tag);
        yv[i][m] = __uint_as_float((uint32_t)v);
      }
    }
    if (__syncthreads_and(ok)) break;
    if (s > kSpin) {
      if (tid == 0) add_dev(L.err, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  float p = 0.0f;
#pragma unroll
  for (int i = 0; i < NX; ++i)
    if (tid + i * kThreads < nch) p = sumsq8(yv[i], p);
  const float inv = norm_inv(row_sumsq_block(p, red4), D, L.eps);
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int c = tid + i * kThreads;
    if (c >= nch) continue;
    float xv[8], r[8];
    unpack8<F16X>(xq[i], xv);
    const float wv[8] = {wa[i].x, wa[i].y, wa[i].z, wa[i].w, wb[i].x, wb[i].y, wb[i].z, wb[i].w};
#pragma unroll
    for (int m = 0; m < 8; ++m) r[m] = xv[m] + norm_scale(yv[i][m], inv, wv[m]);
    const size_t o = (size_t)t * D + 8 * c;
    if (L.out_dtype == MOE_F32) {
      ((float4 *)((float *)L.out + o))[0] = float4{r[0], r[1], r[2], r[3]};
      ((float4 *)((float *)L.out + o))[1] = float4{r[4], r[5], r[6], r[7]};
    } else {
      uint32_t h[8];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        h[m] = L.out_dtype == MOE_BF16 ? f32_to_bf16(r[m]) : f32_to_f16(r[m]);
      *(u32x4 *)((uint16_t *)L.out + o) = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                               h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
  }
  if (tid == 0) st_dev(L.ocnt + t, 0u);
}

// Down projection of output row n over this wave's units, then the split
// reduction over the blocks of the output tile, which writes the output (or,
// NORM, the tagged word the post-norm polls).  Unit i: hidden rows hp[i] ..
// hp[i] + 63, gelu(gate) in L.hg and up in L.hu (tagged words), weight
// gate[i].
template <int M, bool NORM = false>
__device__ __forceinline__ void down_and_combine(const LayerLaunch &L, const DownRegs<M> &R,
                                                 const size_t (&hp)[M], const float (&gate)[M],
                                                 const bool (&use)[M], uint32_t (&hpl)[kNW][M][3][32],
                                                 float (&red)[kNW][2][64], int ot, size_t out_idx,
                                                 int wave, int lane, uint32_t tag) {
  float acc = 0.0f;
  // Each unit is taken as soon as its hidden values are published: lanes
  // 2i, 2i + 1 poll one word of unit i's rows (the hint, two polls in
  // flight); every round, the units whose hints have landed read their
  // values (checked), go through LDS as three bf16 planes and meet their
  // down codes on the matrix cores.  The units' contributions are added in
  // unit order at the end, so the sum does not depend on the order in which
  // the units arrived.
  const uint64_t *hint = L.hg + hp[0];
  uint32_t pending = 0;  // wave-uniform: units still to take
#pragma unroll
  for (int i = 0; i < M; ++i) {
    if (use[i]) pending |= 1u << i;
    if (lane == 2 * i) hint = L.hg + hp[i];
    if (lane == 2 * i + 1) hint = L.hu + hp[i];
  }
  // matrix cores: lane l holds word w (8 hidden rows) of output row l as
  // B (codes as 1 + q / 16); lanes with l % 16 = 4 (l / 16) + p, p < 3,
  // hold plane p of h as A row 4 (l / 16) + p, so registers 0..2 of lane l
  // accumulate the three planes' dot products of output row l.
  const int plane = (lane & 15) - 4 * (lane >> 4);
  const bool ha_lane = plane >= 0 && plane < 3;
  const uint32_t umagic = opaque_vgpr(0x3F803F80u);
  const int pos = 2 * (4 * (lane >> 3) + (lane & 3)) + ((lane >> 2) & 1);
  float vunit[M];
#pragma unroll
  for (int i = 0; i < M; ++i) vunit[i] = 0.0f;
  uint64_t hw = ld_dev64(hint);
  for (long s = 0; pending;) {
    __builtin_amdgcn_s_sleep(1);
    const uint64_t nx = ld_dev64(hint);
    const uint64_t b = __ballot(has_tag(hw, tag));
    uint32_t ready = 0;
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (((b >> (2 * i)) & 3u) == 3u) ready |= 1u << i;
    ready &= pending;
    hw = nx;
    if (!ready) {
      if (++s > kSpin) {
        if (lane == 0) add_dev(L.err, 1u);
        break;
      }
      continue;
    }
    pending &= ~ready;
    // the ready units' values, read until every word carries the epoch (a
    // hint may land before the other words of its unit)
    uint64_t wg[M], wu[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      wg[i] = 0;
      wu[i] = 0;
      if (ready >> i & 1u) {
        wg[i] = ld_dev64(L.hg + hp[i] + lane);
        wu[i] = ld_dev64(L.hu + hp[i] + lane);
      }
    }
    for (long r = 0;; ++r) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < M; ++i)
        ok = ok && (!(ready >> i & 1u) || (has_tag(wg[i], tag) && has_tag(wu[i], tag)));
      if (__all(ok)) break;
      if (r > kSpin) {
        if (lane == 0) add_dev(L.err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int i = 0; i < M; ++i) {
        if (ready >> i & 1u) {
          wg[i] = ld_dev64(L.hg + hp[i] + lane);
          wu[i] = ld_dev64(L.hu + hp[i] + lane);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (!(ready >> i & 1u)) continue;
      const float hv = __uint_as_float((uint32_t)wg[i]) * __uint_as_float((uint32_t)wu[i]);
      // h as three bf16 planes (hi + mid + lo = the fp32 value) in LDS, as
      // pairs (h[8w + m], h[8w + m + 4]) like the activations of gate/up
      const uint32_t p0 = f32_to_bf16(hv);
      const float r1 = hv - __uint_as_float(p0 << 16);
      const uint32_t p1 = f32_to_bf16(r1);
      const uint32_t p2 = f32_to_bf16(r1 - __uint_as_float(p1 << 16));
      uint16_t *hp16 = (uint16_t *)&hpl[wave][i][0][0];
      hp16[pos] = (uint16_t)p0;
      hp16[64 + pos] = (uint16_t)p1;
      hp16[128 + pos] = (uint16_t)p2;
      const float hsum = wave_sum(hv);
      __builtin_amdgcn_wave_barrier();
      // the codes pass an empty asm here, or the compiler would unpack every
      // unit's codes ahead of the polling loop and hold them all in registers
      u32x4 q0 = R.dq0[i], q1 = R.dq1[i];
      asm volatile("" : "+v"(q0.x), "+v"(q0.y), "+v"(q0.z), "+v"(q0.w));
      asm volatile("" : "+v"(q1.x), "+v"(q1.y), "+v"(q1.z), "+v"(q1.w));
      const uint32_t wd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      u32x4 a[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) a[w] = u32x4{0u, 0u, 0u, 0u};
      if (ha_lane) {
#pragma unroll
        for (int w = 0; w < 8; ++w) a[w] = *(const u32x4 *)&hpl[wave][i][plane][4 * w];
      }
      // two accumulation chains (even and odd words)
      f32x4 d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < 8; w += 2) {
        d0 = mma16<false>(a[w], code_pairs_unit(wd[w], umagic), d0);
        d1 = mma16<false>(a[w + 1], code_pairs_unit(wd[w + 1], umagic), d1);
      }
      // sum (1 + q/16) h = sum h + sum q h / 16, three planes
      const float dsum = ((d0[0] + d1[0]) + (d0[1] + d1[1])) + (d0[2] + d1[2]);
      const float sc = f16_to_f32(R.dmw[i]), bi = f16_to_f32(R.dmw[i] >> 16);
      vunit[i] = fmaf(16.0f * sc, dsum, fmaf(-16.0f, sc, bi) * hsum);
    }
  }
#pragma unroll
  for (int i = 0; i < M; ++i)
    if (use[i]) acc = fmaf(gate[i], vunit[i], acc);
  __syncthreads();  // red[] is reused
  red[wave][0][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) s += red[w][0][lane];
    const int nsp = L.KSdr + L.KSds;
    const bool done = nsp == 1 || counted_add(L.dacc + (size_t)ot * 64 + lane, s, nsp, &s, L.err);
    if constexpr (!NORM) {
      if (done) {
        if (L.out_dtype == MOE_F32)
          ((float *)L.out)[out_idx] = s;
        else if (L.out_dtype == MOE_BF16)
          ((uint16_t *)L.out)[out_idx] = (uint16_t)f32_to_bf16(s);
        else
          ((uint16_t *)L.out)[out_idx] = (uint16_t)f32_to_f16(s);
      }
    } else {
      // the output element goes to ybuf as a tagged word for the post-norm,
      // and the wave's number of completed elements to the token's counter
      if (done) st_dev64(L.ybuf + out_idx, tagged(__float_as_uint(s), tag));
      const uint32_t cnt = (uint32_t)__popcll(__ballot(done));
      if (cnt && lane == 0)
        __hip_atomic_fetch_add(L.ocnt + out_idx / (size_t)L.D, cnt, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Router rows e0 .. e0 + kRows - 1 of kRT tokens t0, t0 + 1 (the codes are
// read once; each token's x is staged and dotted in turn, with the same split
// and summation order as the router kernel) and, unless the routed blocks
// rank the logits themselves, the selection of each token (waves 0.. of the
// block one token each).  They head the chain of dependent steps, so these
// blocks do nothing else.  RT = 1 (one token per call) builds the one-token
// code only: the kernel's size matters to the instruction cache.
// s_select[kRT], red4[4 kRT].
template <bool F16X, int MAXC, bool HS = false, int PRIO = 1, bool NORM = false, int RT = 1>
__device__ __forceinline__ void router_role(const LayerLaunch &L, int b, uint32_t &tag, uint8_t *dsm,
                                            SelectLds *s_select, float *red4) {
  constexpr int MAXX = MAXC == 3 ? 2 : 4;  // 16-byte pieces of x per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int D = L.D, E = L.E;
  const int nrb = (E + kRows - 1) / kRows;
  const int grp = b / nrb, r_e0 = (b - grp * nrb) * kRows;
  const int t0 = grp * kRT, nt = min(kRT, L.T - t0);
  __builtin_amdgcn_s_setprio(PRIO);
  const int nch = D / 16;
  float *sx = (float *)dsm;   // x as fp32 [D]
  float *sxs = sx + D;        // 16-column sums [D/16]
  float *rred = sxs + nch;    // partial logits [kKL][kRows]
  const int rr = tid % kRows, kl = tid / kRows;  // chunks kl, kl + kKL, ... of row rr
  u32x4 xr[RT][MAXX], rq[MAXC];
  uint32_t rmw[MAXC];
  const uint16_t *x = (const uint16_t *)L.x;
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const gptr<u32x4> xt = as_global((const u32x4 *)(x + (size_t)(t0 + min(j, nt - 1)) * D));
#pragma unroll
    for (int i = 0; i < MAXX; ++i) xr[j][i] = xt[min(tid + i * kThreads, D / 8 - 1)];
  }
  float4 wn[NORM ? MAXX : 1][2];
  if constexpr (NORM) {
    const float4 *w4 = (const float4 *)L.w_pre;
#pragma unroll
    for (int i = 0; i < MAXX; ++i) {
      const int c = min(tid + i * kThreads, D / 8 - 1);
      wn[i][0] = w4[2 * c];
      wn[i][1] = w4[2 * c + 1];
    }
  }
  const int e = min(r_e0 + rr, E - 1);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = min(kl + i * kKL, nch - 1);
    rq[i] = as_global((const u32x4 *)L.rcodes)[(size_t)c * E + e];
    rmw[i] = as_global(L.rmeta)[(size_t)c / 4 * E + e];
  }
  // the epoch (a vector load, after the loads above) and the logit bias
  tag = __hip_atomic_load(L.bep + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + 1u;
  float lbias = 0.0f;
  if (L.logit_bias && wave == 0 && lane < kRows) lbias = L.logit_bias[min(r_e0 + lane, E - 1)];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    if (j >= nt) continue;  // uniform over the block
    const int rt = t0 + j;
    u32x4 (&xj)[MAXX] = xr[j];
    if (j > 0) __syncthreads();  // the previous token is done with sx and rred
    if constexpr (NORM) {
      // the layer's input u: this thread's chunks are those of the fixed
      // summation order (chunks tid, tid + 256, ...)
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < MAXX; ++i) {
        if (tid + i * kThreads < D / 8) {
          float v[8];
          unpack8<F16X>(xj[i], v);
          p = sumsq8(v, p);
        }
      }
      const float inv = norm_inv(row_sumsq_block(p, red4 + kNW * j), D, L.eps);
#pragma unroll
      for (int i = 0; i < MAXX; ++i) xj[i] = norm_chunk<F16X>(xj[i], inv, wn[i][0], wn[i][1]);
      if (L.u_out && r_e0 == 0) {
#pragma unroll
        for (int i = 0; i < MAXX; ++i)
          if (tid + i * kThreads < D / 8)
            ((u32x4 *)(L.u_out + (size_t)rt * D))[tid + i * kThreads] = xj[i];
      }
    }
#pragma unroll
    for (int i = 0; i < MAXX; ++i) {
      const int c = tid + i * kThreads;
      if (c < D / 8) {
        const uint32_t w[4] = {xj[i].x, xj[i].y, xj[i].z, xj[i].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          sx[8 * c + 2 * m] = x_to_f32<F16X>(w[m] & 0xFFFFu);
          sx[8 * c + 2 * m + 1] = x_to_f32<F16X>(w[m] >> 16);
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < nch; i += kThreads) {
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) s += sx[16 * i + q];
      sxs[i] = s;
    }
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int c = kl + i * kKL;
      if (c < nch) {
        const float sc = f16_to_f32(rmw[i]), bi = f16_to_f32(rmw[i] >> 16);
        const uint32_t w[4] = {rq[i].x, rq[i].y, rq[i].z, rq[i].w};
        const float *xv = sx + c * 16;
        float d = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
            d = fmaf(xv[4 * u + bb], (float)((w[u] >> (8 * bb)) & 0xFFu), d);
        acc = fmaf(sc, d, acc);
        acc = fmaf(bi, sxs[c], acc);
      }
    }
    rred[kl * kRows + rr] = acc;
    __syncthreads();
    if (L.select == 1) {
      // the routed blocks rank the logits themselves: publish this block's
      // logits into every copy (lane: row lane % kRows, copy lane / kRows)
      if (wave == 0) {
        float s = 0.0f;
        const int r = lane % kRows;
        for (int q = 0; q < kKL; ++q) s += rred[q * kRows + r];
        if (L.logit_bias) s += __shfl(lbias, r, 64);
        const int e2 = r_e0 + r;
        for (int cp = lane / kRows; cp < L.log_copies; cp += 64 / kRows)
          if (e2 < E)
            st_dev64(L.rlog + ((size_t)cp * L.T + rt) * E + e2, tagged(__float_as_uint(s), tag));
      }
    } else if (wave == 0 && lane < kRows) {
      float s = 0.0f;
      for (int q = 0; q < kKL; ++q) s += rred[q * kRows + lane];
      const int e2 = r_e0 + lane;
      uint64_t own = 0;  // below every real key
      if (e2 < E) {
        if (L.logit_bias) s += lbias;
        st_dev64(L.rlog + (size_t)rt * E + e2, tagged(__float_as_uint(s), tag));
        own = ((uint64_t)order_key(s) << 32) | (uint64_t)(~(uint32_t)e2);
      }
      s_select[j].own[lane] = own;
    }
  }
  if (L.select != 1) {
    // every token's logits are out; wave j ranks token t0 + j's candidates
    if (nt > 1) __syncthreads();
    if (wave < nt) select_publish<HS>(L, t0 + wave, r_e0, tag, s_select[wave]);
  }
  __builtin_amdgcn_s_setprio(0);
}

// The pre-norm in a gate/up block: the row's chunks of the fixed summation
// order (tid, tid + 256, ...) and the norm weights of the thread's own chunk
// (the one issue_x loads) are requested with x; finish_norm sums, and turns
// the thread's chunk into the layer's input u.  Every thread of the block
// takes part (a barrier).
template <int NX>
struct NormIn {
  u32x4 q[NX];
  float4 w0, w1;
};
template <int NX>
__device__ __forceinline__ void issue_norm(const LayerLaunch &L, int t, int g0, int g1, int tid,
                                           NormIn<NX> &n) {
  const int nch = L.D / 8;
  const gptr<u32x4> xr = as_global((const u32x4 *)((const uint16_t *)L.x + (size_t)t * L.D));
#pragma unroll
  for (int i = 0; i < NX; ++i) n.q[i] = xr[min(tid + i * kThreads, nch - 1)];
  const int c = 8 * g0 + min(tid, (g1 - g0) * 8 - 1);
  const float4 *w4 = (const float4 *)L.w_pre;
  n.w0 = w4[2 * c];
  n.w1 = w4[2 * c + 1];
}
template <bool F16X, int NX>
__device__ __forceinline__ u32x4 finish_norm(const LayerLaunch &L, const NormIn<NX> &n, u32x4 xq,
                                             float *red4) {
  const int tid = threadIdx.x, nch = L.D / 8;
  float p = 0.0f;
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    if (tid + i * kThreads < nch) {
      float v[8];
      unpack8<F16X>(n.q[i], v);
      p = sumsq8(v, p);
    }
  }
  const float inv = norm_inv(row_sumsq_block(p, red4), L.D, L.eps);
  return norm_chunk<F16X>(xq, inv, n.w0, n.w1);
}

// TWO: the streamed variant in two launches (router and shared blocks, then
// the routed blocks); its router blocks also store the selection into host
// memory and its routed blocks take each rank's blob from given_blob.
// NORM: the residual block fused around the layer (resident experts, one
// launch): x is the residual stream, every role normalises it into the
// layer's input, and the output rows get the post-norm and the residual.
template <bool F16X, int M, int MAXC, bool TWO, bool NORM = false, int RT = 1>
__global__ __launch_bounds__(kThreads, (NORM && MAXC == 8) ? 3 : 4) void decode_layer_kernel(LayerLaunch L) {
  extern __shared__ __align__(16) uint8_t dsm[];
  __shared__ float red[kNW][2][64];
  __shared__ __align__(16) uint32_t hpl[kNW][M][3][32];  // h planes as bf16 pairs
  __shared__ __align__(16) uint32_t s_xp[kMaxBlockGroups * 32];  // activation pairs
  __shared__ float s_xs[kMaxBlockGroups];                        // 64-column sums
  __shared__ const uint8_t *s_blob[2][kMaxK];  // [0]: gate/up token, [1]: down token
  __shared__ float s_gate[2][kMaxK];
  __shared__ SelectLds s_select[kRT];
  __shared__ uint2 s_xch[2][128];  // top-k exchange of the selecting waves
  __shared__ float s_red4[kNW * kRT];  // the norms' wave sums
  constexpr int NX = MAXC == 3 ? 2 : 4;  // chunks of x per thread in the pre-norm

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int D = L.D, E = L.E, k = L.k, T = L.T;
  const int G = D / 64, NB = D / 64;
  const int Gf = L.F / 64, Gs = L.sblobs ? L.Fs / 64 : 0;
  // roles: router blocks [0, nr0), routed blocks [nr0, NR), shared
  // blocks [NR, grid).  Each role runs straight through its own code.  With
  // order 1 the shared blocks are dispatched right after the router blocks
  // (their loads depend on nothing and then drain before the routing's
  // hand-offs); b is the logical index either way.
  const int nrb = (E + kRows - 1) / kRows;
  const int nr0 = (T + kRT - 1) / kRT * nrb;  // router blocks: kRT tokens each
  const int p = TWO ? L.blk0 + blockIdx.x : blockIdx.x, ns = L.grid_full - L.NR;
  const int b = !L.order ? (TWO ? p : L.blk0 + p)
                         : p < nr0 ? p : p < nr0 + ns ? L.NR + (p - nr0) : p - ns;
  // the epoch is read by each role after its first loads are issued, with a
  // vector load (an atomic one): nothing waits for it before its first use
  uint32_t tag = 0;
  auto load_tag = [&]() {
    tag = __hip_atomic_load(L.bep + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + 1u;
  };
  const int n_rt = T * k * Gf;                 // routed gate/up tiles, then the shared ones
  // down units: waves 1..3 (wave 0 mirrors wave 1 and does the gate/up
  // reduction's atomics), or all four waves (dw4: more units per block, for
  // grids that would not be resident otherwise)
  const int dwc = L.dw4 ? kNW : kDW;
  const int dw = L.dw4 ? wave : max(wave - 1, 0);
  const bool dwave = L.dw4 || wave > 0;

  if (b < nr0) {
    // ---------------- router rows and the selection of the token.  They
    // head the chain of dependent steps, so these blocks do nothing else.
    router_role<F16X, MAXC, TWO, 1, NORM, RT>(L, b, tag, dsm, s_select, s_red4);
    // router block i of a token group then does the post-norm of the
    // group's token i (the tokens' polls run side by side; with fewer router
    // blocks than tokens in a group, block i takes tokens i, i + nrb, ...)
    if constexpr (NORM) {
      const int t0 = b / nrb * kRT, i = b % nrb;
      if (i < RT && t0 + i < T) post_norm_poll<F16X, NX>(L, t0 + i, tag, s_red4);
      if (RT > 1 && nrb == 1 && t0 + 1 < T) post_norm_poll<F16X, NX>(L, t0 + 1, tag, s_red4);
    }
  } else if (b >= L.NR) {
    // ---------------- shared expert: its gate/up tiles and its part of the
    // down projection; nothing waits on the routing
    const int sb = b - L.NR;
    const int n_st = L.n_gtiles - n_rt;
    const bool has_g = sb < n_st * L.KSg;
    const int gsb = min(sb, n_st * L.KSg - 1);
    const int tile = n_rt + gsb / L.KSg, ks = gsb % L.KSg;
    const Tile gt = glu_tile(L, tile);
    const int g0 = ks * G / L.KSg, g1 = (ks + 1) * G / L.KSg;
    const bool has_d = sb < T * NB * L.KSds;
    const int dsb = min(sb, T * NB * L.KSds - 1);
    const int ot = dsb / L.KSds, ksd = dsb % L.KSds;
    const int t_out = ot / NB, n = (ot - t_out * NB) * 64 + lane;
    const int u0 = ksd * Gs / L.KSds, u1 = (ksd + 1) * Gs / L.KSds;

    const uint8_t *sblob = (const uint8_t *)as_global(L.sblobs)[0];
    u32x4 xq = issue_x(L, gt.t, g0, g1, tid);
    NormIn<NX> nx;
    if constexpr (NORM) issue_norm(L, gt.t, g0, g1, tid, nx);
    load_tag();
    GluRegs<M> gr;
    issue_glu(gr, sblob, D, L.Fs, gt.rb, g0, g1, wave, lane);
    DownRegs<M> dr;
    auto load_down = [&]() {
#pragma unroll
      for (int i = 0; i < M; ++i)
        issue_down(dr, i, sblob, D, L.Fs, min(u0 + dw + i * dwc, u1 - 1), n);
    };
    if constexpr (NORM) xq = finish_norm<F16X>(L, nx, xq, s_red4);
    stage_x<F16X>(xq, (g1 - g0) * 8, tid, s_xp, s_xs);
    __syncthreads();
    if (has_g) {
      float accg, accu;
      glu_dots<F16X, M>(gr, s_xp, s_xs, g0, g1, wave, lane, accg, accu);
      red[wave][0][lane] = accg;
      red[wave][1][lane] = accu;
    }
    // down weights of waves 1..3 after the split reduction (requested with
    // the gate/up weights they would queue in front of them); wave 0 does
    // the reduction's atomics
    if (has_g) glu_publish<NORM>(L, red, tile, gt.hoff + (size_t)gt.rb * 64, wave, lane, tag);
    if (dwave) load_down();
    if (has_d) {
      size_t hp[M];
      float gate[M];
      bool use[M];
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int u = min(u0 + dw + i * dwc, u1 - 1);
        use[i] = dwave && u0 + dw + i * dwc < u1;
        gate[i] = 1.0f;
        hp[i] = (size_t)T * k * L.F + (size_t)t_out * L.Fs + (size_t)u * 64;
      }
      down_and_combine<M, NORM>(L, dr, hp, gate, use, hpl, red, ot, (size_t)t_out * D + n, wave,
                                lane, tag);
    }
  } else {
    // ---------------- routed blocks: gate/up tiles and the routed part of
    // the down projection of the selected experts.  No weight load is issued
    // before the selection arrives, so the polls do not queue behind loads.
    const int sb = b - nr0;
    const bool has_g = sb < n_rt * L.KSg;
    const int gsb = min(sb, n_rt * L.KSg - 1);
    const int tile = gsb / L.KSg, ks = gsb % L.KSg;
    const Tile gt = glu_tile(L, tile);
    const int g0 = ks * G / L.KSg, g1 = (ks + 1) * G / L.KSg;
    const bool has_d = sb < T * NB * L.KSdr;
    const int dsb = min(sb, T * NB * L.KSdr - 1);
    const int ot = dsb / L.KSdr, ksd = dsb % L.KSdr;
    const int t_out = ot / NB, n = (ot - t_out * NB) * 64 + lane;
    const int Ur = k * Gf;
    const int u0 = ksd * Ur / L.KSdr, u1 = (ksd + 1) * Ur / L.KSdr;

    u32x4 xq = issue_x(L, gt.t, g0, g1, tid);
    NormIn<NX> nx;
    if constexpr (NORM) issue_norm(L, gt.t, g0, g1, tid, nx);
    load_tag();
    if constexpr (NORM) xq = finish_norm<F16X>(L, nx, xq, s_red4);
    const void **s_table = (const void **)(dsm + L.table_off);
    if constexpr (!TWO) {
      constexpr int kTab = kMaxLayerE / kThreads;
      const void *tb[kTab];
#pragma unroll
      for (int i = 0; i < kTab; ++i) tb[i] = as_global(L.rblobs)[min(tid + i * kThreads, E - 1)];
      stage_x<F16X>(xq, (g1 - g0) * 8, tid, s_xp, s_xs);
#pragma unroll
      for (int i = 0; i < kTab; ++i)
        if (tid + i * kThreads < E) s_table[tid + i * kThreads] = tb[i];
    } else {
      stage_x<F16X>(xq, (g1 - g0) * 8, tid, s_xp, s_xs);
    }
    __syncthreads();
    const int copy = sb % L.sel_copies;
    // the first block of each token's first gate/up tile reports the selection
    const bool report = has_g && gt.j == 0 && gt.rb == 0 && ks == 0;
    if (!TWO && L.select == 1) {
      const int lc = sb % L.log_copies;
      if (wave == 0)
        select_from_logits(L, gt.t, lc, tag, s_table, s_blob[0], s_gate[0], report, s_xch[0]);
      if (wave == 1 && t_out != gt.t)
        select_from_logits(L, t_out, lc, tag, s_table, s_blob[1], s_gate[1], false, s_xch[1]);
    } else {
      // the blob table: by expert id, or (two launches) by rank per token
      const void *const *t0 = TWO ? L.given_blob + (size_t)gt.t * k : s_table;
      const void *const *t1 = TWO ? L.given_blob + (size_t)t_out * k : s_table;
      if (wave == 0)
        wait_selection<TWO>(L, gt.t, copy, tag, t0, s_blob[0], s_gate[0], report);
      if (wave == 1 && t_out != gt.t)
        wait_selection<TWO>(L, t_out, copy, tag, t1, s_blob[1], s_gate[1], false);
    }
    __syncthreads();
    const int ds = t_out == gt.t ? 0 : 1;  // selection of the down token
    // gate/up weights, then the down weights (every wave; wave 0 mirrors
    // wave 1's units): the gate/up arithmetic waits for its own loads only
    GluRegs<M> gr;
    issue_glu(gr, s_blob[0][gt.j], D, L.F, gt.rb, g0, g1, wave, lane);
    DownRegs<M> dr;
    auto load_down = [&]() {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int u = min(u0 + dw + i * dwc, u1 - 1);
        const int jj = u / Gf;
        issue_down(dr, i, s_blob[ds][jj], D, L.F, u - jj * Gf, n);
      }
    };
    if (has_g) {
      float accg, accu;
      glu_dots<F16X, M>(gr, s_xp, s_xs, g0, g1, wave, lane, accg, accu);
      red[wave][0][lane] = accg;
      red[wave][1][lane] = accu;
    }
    // down weights of waves 1..3 after the split reduction (requested with
    // the gate/up weights they would queue in front of them); wave 0 does
    // the reduction's atomics
    if (has_g) glu_publish<NORM>(L, red, tile, gt.hoff + (size_t)gt.rb * 64, wave, lane, tag);
    if (dwave) load_down();
    if (has_d) {
      size_t hp[M];
      float gate[M];
      bool use[M];
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int u = min(u0 + dw + i * dwc, u1 - 1);
        const int jj = u / Gf;
        use[i] = dwave && u0 + dw + i * dwc < u1;
        gate[i] = s_gate[ds][jj];
        hp[i] = (size_t)(t_out * k + jj) * L.F + (size_t)(u - jj * Gf) * 64;
      }
      down_and_combine<M, NORM>(L, dr, hp, gate, use, hpl, red, ot, (size_t)t_out * D + n, wave,
                                lane, tag);
    }
  }

  // ---------------- advance every copy of the epoch (block b: b, b + grid, ...)
  if (tid == 0)
    for (int j = b; j < kMaxLayerGrid; j += L.grid_full) st_dev(L.bep + j, tag);
}

using KernelFn = void (*)(LayerLaunch);
template <bool F16X, int MAXC, int RT>
KernelFn pick_m(int m, bool two, bool norm) {
  if (norm) {
    if (two) return nullptr;
    if (m == 2) return decode_layer_kernel<F16X, 2, MAXC, false, true, RT>;
    if (m == 3) return decode_layer_kernel<F16X, 3, MAXC, false, true, RT>;
    if (m == 4) return decode_layer_kernel<F16X, 4, MAXC, false, true, RT>;
    return nullptr;
  }
  if (two) {
    if (m == 2) return decode_layer_kernel<F16X, 2, MAXC, true, false, RT>;
    if (m == 3) return decode_layer_kernel<F16X, 3, MAXC, true, false, RT>;
    if (m == 4) return decode_layer_kernel<F16X, 4, MAXC, true, false, RT>;
    return nullptr;
  }
  if (m == 2) return decode_layer_kernel<F16X, 2, MAXC, false, false, RT>;
  if (m == 3) return decode_layer_kernel<F16X, 3, MAXC, false, false, RT>;
  if (m == 4) return decode_layer_kernel<F16X, 4, MAXC, false, false, RT>;
  return nullptr;
}
template <bool F16X, int MAXC>
KernelFn pick(int m, bool two, bool norm, bool multi) {
  return multi ? pick_m<F16X, MAXC, kRT>(m, two, norm) : pick_m<F16X, MAXC, 1>(m, two, norm);
}
KernelFn pick_layer(const LayerLaunch &L, int m) {
  const bool small_d = L.D <= 3072;  // router chunks per thread: 3 (D <= 3072) or 8
  // kernels for one token per call carry one token's router code only
  const bool two = L.two != 0, nm = L.w_pre != nullptr, multi = L.T > 1;
  if (L.f16x) return small_d ? pick<true, 3>(m, two, nm, multi) : pick<true, 8>(m, two, nm, multi);
  return small_d ? pick<false, 3>(m, two, nm, multi) : pick<false, 8>(m, two, nm, multi);
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

int g_layer_capacity[2][3][2][2][3][64];  // [T > 1][resident, two, norm][f16x][MAXC 3/8][m - 2][device]

}  // namespace

int layer_m(const LayerLaunch &L) {
  const int Gf = L.F / 64, Gs = L.sblobs ? L.Fs / 64 : 0;
  const int dwc = L.dw4 ? kNW : kNW - 1;  // waves with down units
  int m = ceil_div(ceil_div(L.D / 64, L.KSg), kNW);
  m = max(m, ceil_div(ceil_div(L.k * Gf, L.KSdr), dwc));
  if (L.KSds > 0) m = max(m, ceil_div(ceil_div(Gs, L.KSds), dwc));
  return m < 2 ? 2 : m;
}

int layer_router_blocks(const LayerLaunch &L) {
  return (L.T + kRT - 1) / kRT * ((L.E + kRows - 1) / kRows);
}

// routed blocks (router rows, routed gate/up tiles, routed down splits) and
// shared blocks (shared gate/up tiles, shared down splits)
int layer_routed_blocks(const LayerLaunch &L) {
  const int n_rt = L.T * L.k * (L.F / 64);
  const int r = layer_router_blocks(L);  // router blocks come first
  return r + max(n_rt * L.KSg, L.T * (L.D / 64) * L.KSdr);
}
int layer_shared_blocks(const LayerLaunch &L) {
  const int n_st = L.n_gtiles - L.T * L.k * (L.F / 64);
  return max(n_st * L.KSg, L.T * (L.D / 64) * L.KSds);
}
int layer_grid(const LayerLaunch &L) { return layer_routed_blocks(L) + layer_shared_blocks(L); }

size_t layer_table_off(const LayerLaunch &L) {
  // router staging: x as fp32, 16-column sums, partial logits; full-K gate/up
  // blocks: activation pairs and 64-column sums of every group
  size_t stage = sizeof(float) * ((size_t)L.D + L.D / 16 + kThreads);
  return align_up(stage);
}
size_t layer_smem(const LayerLaunch &L) { return layer_table_off(L) + sizeof(void *) * (size_t)L.E; }

hipError_t layer_capacity(const LayerLaunch &L, int *cap) {
  *cap = 0;
  const int m = layer_m(L);
  KernelFn k = pick_layer(L, m);
  if (!k) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int &slot = g_layer_capacity[L.T > 1 ? 1 : 0][L.two ? 1 : L.w_pre ? 2 : 0][L.f16x ? 1 : 0]
                              [L.D <= 3072 ? 0 : 1]
                              [m - 2][dev];
  const size_t smem = layer_smem(L);
  if (smem > 64 * 1024) return hipSuccess;
  if (!slot) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k, kThreads, smem);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // at most 4 blocks per CU: with 5 (the smallest register counts) the
    // widest split gives a grid of 1,242 blocks for one token, measured no
    // faster for the layer and 4.5 us slower for the residual block than the
    // 1,000 blocks of 4 per CU
    slot = (per_cu < 4 ? per_cu : 4) * cus;
  }
  *cap = slot;
  return hipSuccess;
}

hipError_t launch_layer_range(LayerLaunch L, int blk0, int n, hipStream_t s) {
  KernelFn k = pick_layer(L, layer_m(L));
  if (!k) return hipErrorInvalidValue;
  if (n <= 0) return hipSuccess;
  L.blk0 = blk0;
  L.grid_full = layer_grid(L);
  // the block order applies to whole-grid launches only (ranges are logical)
  if (blk0 != 0 || n != L.grid_full) L.order = 0;
  hipLaunchKernelGGL(k, dim3(n), dim3(kThreads), layer_smem(L), s, L);
  return hipGetLastError();
}

hipError_t launch_layer(const LayerLaunch &L, hipStream_t s) {
  return launch_layer_range(L, 0, layer_grid(L), s);
}

hipError_t launch_layer_ordered(LayerLaunch L, int first, int n, hipStream_t s) {
  KernelFn k = pick_layer(L, layer_m(L));
  if (!k || !L.two) return hipErrorInvalidValue;
  L.grid_full = layer_grid(L);
  if (first < 0 || n < 0 || first + n > L.grid_full) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  L.blk0 = first;
  hipLaunchKernelGGL(k, dim3(n), dim3(kThreads), layer_smem(L), s, L);
  return hipGetLastError();
}

}  // namespace moe
