// C ABI of libmoe: argument checks, workspace carve-up and kernel dispatch.
#include <cmath>
#include <string.h>

#include <new>

#include "moe_internal.h"
#include "pool.h"

namespace moe {

Tuning &tuning() {
  static Tuning t;
  return t;
}

namespace {
struct ProfileEvents {
  void *const *events = nullptr;
  int n = 0, next = 0;
};
ProfileEvents g_prof;

// Records the probe's begin event of the next pair (returns the pair index).
int prof_begin(hipStream_t s) {
  if (!g_prof.events || g_prof.n <= 0) return -1;
  const int i = g_prof.next;
  g_prof.next = (g_prof.next + 1) % g_prof.n;
  (void)hipEventRecord((hipEvent_t)g_prof.events[2 * i], s);
  return i;
}
hipError_t prof_end(int i, hipStream_t s, hipError_t e) {
  if (i >= 0) (void)hipEventRecord((hipEvent_t)g_prof.events[2 * i + 1], s);
  return e;
}
}  // namespace

namespace {

// Reserves aligned regions of a workspace in a fixed order.  With base ==
// nullptr it only measures.
struct Carver {
  uint8_t *base;
  size_t off = 0;
  template <class P>
  P *take(size_t count, size_t elem) {
    P *p = base ? (P *)(base + off) : nullptr;
    off = align_up(off + count * elem);
    return p;
  }
};

// counters of the one-launch expert phase: slots, and the replicated
// slot-ready flags (one 32-word line per copy)
size_t fused_counter_words(const Dims &d) {
  const size_t slots = (size_t)d.T * (d.k + 1);
  return slots + slots * kFlagCopies * 32 + 64;
}

Workspace carve(void *base, const Dims &d) {
  Carver c{(uint8_t *)base};
  Workspace w;
  w.layer = c.take<uint8_t>(kLayerRegionBytes, 1);
  w.err = base ? (uint32_t *)(w.layer + kErrOff) : nullptr;
  const size_t T = d.T, k = d.k;
  const size_t units = T * k * d.F + T * d.Fs;
  w.xp = c.take<uint32_t>(T * d.D / 2, 4);
  w.xs = c.take<float>(T * (d.D / 64), 4);
  w.logits = c.take<float>(T * d.E, 4);
  w.ids = c.take<int32_t>(T * k, 4);
  w.gates = c.take<float>(T * k, 4);
  w.slot_blob = c.take<const void *>(T * k, sizeof(void *));
  w.h = c.take<float>(units, 4);
  w.hs = c.take<float>(units / 64 + 1, 4);
  w.part = c.take<float>((size_t)kMaxSplitBlocks * 128, 4);
  w.counters = c.take<uint32_t>((size_t)kMaxSplitBlocks + T, 4);
  w.dpart = c.take<float>((size_t)kMaxSplitBlocks * 64, 4);
  w.fcounters = c.take<uint32_t>(fused_counter_words(d), 4);
  w.perm_counts = c.take<int32_t>(d.E, 4);
  w.perm_offsets = c.take<int32_t>(d.E + 1, 4);
  // at most one partial chunk per expert: sum ceil(c / R) <= E + T k / R
  w.perm_items = c.take<int32_t>((size_t)d.E + (T * k + kPrefillRows - 1) / kPrefillRows, 4);
  w.perm_n_items = c.take<int32_t>(1, 4);
  w.perm_info = c.take<int2>((size_t)d.E + (T * k + kPrefillRows - 1) / kPrefillRows, 8);
  w.perm_iblob =
      c.take<const void *>((size_t)d.E + (T * k + kPrefillRows - 1) / kPrefillRows, 8);
  w.perm = c.take<int32_t>(T * k, 4);
  w.perm_inv = c.take<int32_t>(T * k, 4);
  w.hplanes = c.take<uint16_t>(3 * units, 2);
  w.hsum = c.take<float>(units / 64 + 1, 4);
  w.y = c.take<float>(T * k * (size_t)d.D, 4);
  w.ys = c.take<float>(kMaxSharedSplits * T * (size_t)d.D, 4);
  // batched decode (T <= kMaxMidT): split sums of the two kernels
  const bool mid = T <= (size_t)kMaxMidT && T * k <= 64;
  w.mgacc = c.take<uint64_t>(mid ? 2 * units : 0, 8);
  w.mdacc = c.take<uint64_t>(mid ? T * d.D : 0, 8);
  w.total = c.off;
  return w;
}

bool dtype_x_ok(int dt) { return dt == MOE_F16 || dt == MOE_BF16; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool dtype_out_ok(int dt) { return dt == MOE_F16 || dt == MOE_BF16 || dt == MOE_F32; }

moe_status check_router(const moe_qmat *r) {
  if (!r || !r->codes || !r->meta) return MOE_E_INVALID;
  if (r->rows < 1 || r->rows > kMaxE || r->cols < 64 || r->cols % 64) return MOE_E_INVALID;
  if (r->cols > 8192) return MOE_E_UNSUPPORTED;
  if (r->bits != 8) return r->bits == 4 ? MOE_E_UNSUPPORTED : MOE_E_INVALID;
  return MOE_OK;
}

moe_status check_bank(const moe_bank *b, int D) {
  if (!b || !b->blobs) return MOE_E_INVALID;
  if (b->E < 1 || b->D != D || b->F < 64 || b->F % 64 || b->D % 64) return MOE_E_INVALID;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Accumulators and counters of the deterministic split reductions: fixed
// places in the workspace's layer region, zero between calls.
void set_split_accumulators(const Workspace &w, uint64_t **gacc, uint64_t **dacc, uint32_t **gcnt,
                            uint32_t **dcnt) {
  *gacc = (uint64_t *)(w.layer + kAccGluOff);
  *dacc = (uint64_t *)(w.layer + kAccOutOff);
  *gcnt = (uint32_t *)(w.layer + kCntGluOff);
  *dcnt = (uint32_t *)(w.layer + kCntOutOff);
}

// Reduction splits shared by both one-launch kernels (same splits, same
// bits): gate/up splits over the column groups, aiming at about two blocks per
// compute unit, and down splits over the routed units and over the shared
// units, at most 16 groups or 12 units per block.
struct Splits {
  int ksg, ksdr, ksds;
};
Splits plan_splits(int T, int k, int D, int F, int Fs, int ksg_override, int ksd_override,
                   int units_per_block = 12) {
  const int G = D / 64, NB = D / 64;
  const int n_rt = T * k * (F / 64), n_st = T * (Fs / 64);
  const int Ur = k * (F / 64), Us = Fs / 64;
  const int target = 512;
  Splits sp;
  sp.ksg = ksg_override > 0 ? ksg_override : (target + n_rt + n_st - 1) / (n_rt + n_st);
  sp.ksg = clampi(sp.ksg, (G + 15) / 16, G < kMaxKS ? G : kMaxKS);
  // about one down item per gate/up item in each group of blocks
  int ksdr = ksd_override > 0 ? ksd_override : (n_rt * sp.ksg + T * NB - 1) / (T * NB);
  const int upb = units_per_block;
  sp.ksdr = clampi(ksdr, (Ur + upb - 1) / upb, Ur < kMaxFusedKSd ? Ur : kMaxFusedKSd);
  sp.ksds = 0;
  if (Us > 0) {
    int ksds = ksd_override > 0 ? ksd_override : (n_st * sp.ksg + T * NB - 1) / (T * NB);
    sp.ksds = clampi(ksds, (Us + upb - 1) / upb, Us < kMaxFusedKSd ? Us : kMaxFusedKSd);
  }
  return sp;
}

// Choose the splits of the one-launch expert phase; false if its grid would
// not be resident all at once (then the three-kernel path runs).
bool plan_fused(const ExpertLaunch &a, const Workspace &w, FusedLaunch *f) {
  const int G = a.D / 64, NB = a.D / 64;
  const int n_gtiles = a.T * a.k * (a.F / 64) + (a.sblobs ? a.T * (a.Fs / 64) : 0);
  const Splits sp = plan_splits(a.T, a.k, a.D, a.F, a.sblobs ? a.Fs : 0, tuning().fused_ksg,
                                tuning().fused_ksd);
  const int Ur = a.k * (a.F / 64), Us = a.sblobs ? a.Fs / 64 : 0;
  if ((G + sp.ksg - 1) / sp.ksg > 16 || (Ur + sp.ksdr - 1) / sp.ksdr > 16 ||
      (sp.ksds > 0 && (Us + sp.ksds - 1) / sp.ksds > 16))
    return false;
  f->a = a;
  f->KSg = sp.ksg;
  f->KSdr = sp.ksdr;
  f->KSds = sp.ksds;
  f->KSd = sp.ksdr + sp.ksds;
  f->n_gtiles = n_gtiles;
  f->tile_begin = 0;
  f->tile_end = n_gtiles;
  f->do_down = 1;
  int cap = 0;
  if (fused_capacity(*f, &cap) != hipSuccess || cap <= 0) return false;
  const int grid = fused_grid(*f);
  if (grid > cap || n_gtiles > kMaxAccTiles || a.T * NB > kMaxOutTiles) return false;
  // slot counters (cleared by the router kernel), then the flag lines
  f->slot_cnt = w.fcounters;
  f->slot_flag = w.fcounters + (size_t)a.T * (a.k + 1);
  f->slot_flag += (32 - ((uintptr_t)f->slot_flag / 4) % 32) % 32;  // 128-byte lines
  f->err = w.err;
  set_split_accumulators(w, &f->gacc, &f->dacc, &f->gcnt, &f->dcnt);
  return true;
}

// Choose the splits of the one-launch decode layer and place its tagged words
// in the workspace's fixed region; false if it does not apply (then the router
// kernel and the expert kernels run).
bool plan_layer(const Workspace &w, LayerLaunch *L) {
  const int T = L->T, k = L->k, E = L->E, D = L->D, F = L->F;
  const int Fs = L->sblobs ? L->Fs : 0;
  if (!tuning().layer || T > kMaxLayerT || E > kMaxLayerE || k > kMaxK || D > 8192) return false;
  const int NB = D / 64, G = D / 64;
  const int n_gtiles = T * k * (F / 64) + T * (Fs / 64);
  L->n_gtiles = n_gtiles;
  L->order = tuning().layer_order;
  L->select = tuning().layer_select == 1 ? 1 : 0;
  L->log_copies = L->select ? min(max(tuning().layer_log_copies, 1), 64) : 1;
  bool found = false;
  // the most gate/up splits (and with them down splits) whose grid is still
  // resident all at once: more, smaller blocks overlap more of the transfer.
  // Several tokens: if no grid fits with three waves of down units per
  // block, every wave takes down units (16 per block instead of 12)
  const int ksg_hi = tuning().layer_ksg > 0 ? tuning().layer_ksg : (G < kMaxKS ? G : kMaxKS);
  const int ksg_lo = tuning().layer_ksg > 0 ? tuning().layer_ksg : 1;
  for (int dw4 = 0; dw4 <= (T > 1 && !L->two ? 1 : 0) && !found; ++dw4) {
    L->dw4 = dw4;
    for (int ksg = ksg_hi; ksg >= ksg_lo && !found; --ksg) {
      const Splits sp = plan_splits(T, k, D, F, Fs, ksg, tuning().layer_ksd, dw4 ? 16 : 12);
      L->KSg = sp.ksg;
      L->KSdr = sp.ksdr;
      L->KSds = sp.ksds;
      L->NR = layer_routed_blocks(*L);
      if (layer_m(*L) > 4) continue;
      const int grid = layer_grid(*L);
      int cap = 0;
      if (layer_capacity(*L, &cap) != hipSuccess) return false;
      found = grid <= cap && grid <= kMaxLayerGrid;
    }
  }
  if (!found) return false;
  if (n_gtiles > kMaxAccTiles || T * NB > kMaxOutTiles) return false;
  L->bep = (uint32_t *)w.layer;
  set_split_accumulators(w, &L->gacc, &L->dacc, &L->gcnt, &L->dcnt);
  // tagged words: logits, hidden activations
  Carver c{w.layer + kTaggedOff};
  L->rlog = c.take<uint64_t>((size_t)L->log_copies * T * E, 8);
  // copies of each selection line (spread the polling)
  L->sel_copies = min(max(tuning().layer_sel_copies, 1), 256);
  L->lid = (k + 15) / 16 * 16;
  L->sel_stride = max(tuning().layer_sel_stride, 2 * L->lid);
  if (L->sel_stride > 4096) L->sel_stride = 4096;
  L->sel = c.take<uint64_t>((size_t)T * L->sel_copies * L->sel_stride, 8);
  L->hg = c.take<uint64_t>((size_t)T * k * F + (size_t)T * Fs, 8);
  L->hu = c.take<uint64_t>((size_t)T * k * F + (size_t)T * Fs, 8);
  if (kTaggedOff + c.off > kRowTagOff) return false;
  L->table_off = layer_table_off(*L);
  L->err = w.err;
  return true;
}

}  // namespace

moe_status layer_forward_args(const void *x, int x_dtype, int T, const moe_qmat *router, int k,
                              const moe_bank *routed, const moe_bank *shared, moe_pool *pool,
                              int layer, const void *out, int out_dtype, Dims *d) {
  if (!x || !aligned16(x) || !dtype_x_ok(x_dtype) || T < 1 || !out || !dtype_out_ok(out_dtype))
    return MOE_E_INVALID;
  moe_status st = check_router(router);
  if (st) return st;
  const int E = router->rows, D = router->cols;
  if (k < 1 || k > E || k > kMaxK) return MOE_E_INVALID;
  int F = 0;
  if (pool) {
    st = pool_check(pool, layer, E, D, k);
    if (st) return st;
    F = pool_F(pool);
  } else {
    st = check_bank(routed, D);
    if (st) return st;
    if (routed->E != E) return MOE_E_INVALID;
    F = routed->F;
  }
  if (shared) {
    st = check_bank(shared, D);
    if (st) return st;
  }
  *d = Dims{T, k, E, D, F, shared ? shared->F : 0};
  return MOE_OK;
}

Workspace carve_workspace(void *base, const Dims &d) { return carve(base, d); }

void init_layer_launch(LayerLaunch *L, const void *x, int x_dtype, const Dims &d,
                       const moe_qmat *router, const float *logit_bias, int k,
                       const moe_bank *routed, const moe_bank *shared, moe_pool *pool, void *out,
                       int out_dtype, int32_t *ids_out, float *gates_out) {
  L->f16x = x_dtype == MOE_F16; L->T = d.T; L->k = k; L->E = d.E; L->D = d.D; L->F = d.F;
  L->Fs = d.Fs;
  L->x = x; L->rcodes = (const uint8_t *)router->codes; L->rmeta = (const uint32_t *)router->meta;
  L->logit_bias = logit_bias; L->rblobs = pool ? nullptr : routed->blobs;
  L->sblobs = shared ? shared->blobs : nullptr;
  L->ids_out = ids_out; L->gates_out = gates_out; L->out = out; L->out_dtype = out_dtype;
  L->two = pool != nullptr;  // streamed experts: the two-launch variant (its occupancy)
}
size_t workspace_bytes(const Dims &d) { return carve(nullptr, d).total; }

// The residual block's buffers after the layer's workspace: the normalised
// input u [T, D] 16-bit, the layer's output y [T, D] fp32 (separate
// kernels), the one-launch path's tagged output words [min(T, 4), D] and its
// per-token counters [4] (zero between calls).
BlockTail block_tail(size_t layer_bytes, int T, int D) {
  BlockTail b;
  b.u_off = align_up(layer_bytes);
  b.y_off = align_up(b.u_off + (size_t)T * D * 2);
  b.yt_off = align_up(b.y_off + (size_t)T * D * 4);
  b.cnt_off = align_up(b.yt_off + (size_t)min(T, kMaxLayerT) * D * 8);
  b.total = align_up(b.cnt_off + (size_t)kMaxLayerT * 4);
  return b;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_blob_bytes(int32_t D, int32_t F) {
  if (D < 64 || F < 64 || D % 64 || F % 64) return 0;
  return blob_layout(D, F).total;
}

size_t moe_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t D, int32_t F,
                           int32_t F_shared) {
  if (T < 1 || k < 1 || E < 1 || D < 64 || F < 0 || F_shared < 0) return 0;
  return workspace_bytes(Dims{T, k, E, D, F, F_shared});
}

const char *moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_E_INVALID: return "invalid argument";
    case MOE_E_UNSUPPORTED: return "unsupported argument";
    case MOE_E_HIP: return "HIP runtime error";
    case MOE_E_WORKSPACE: return "workspace too small";
    case MOE_E_POOL: return "expert pool error";
    default: return "unknown status";
  }
}

moe_status moe_workspace_timeouts(const void *ws, size_t ws_bytes, uint32_t *count,
                                  void *stream) {
  if (!ws || !count || ws_bytes < kLayerRegionBytes) return !ws || !count ? MOE_E_INVALID
                                                                          : MOE_E_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, (const uint8_t *)ws + kErrOff, sizeof(v),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return MOE_E_HIP;
  *count = v;
  return MOE_OK;
}

moe_status moe_set_profile_events(void *const *events, int32_t n_pairs) {
  if (events && n_pairs <= 0) return MOE_E_INVALID;
  g_prof.events = n_pairs > 0 ? events : nullptr;
  g_prof.n = events ? n_pairs : 0;
  g_prof.next = 0;
  return MOE_OK;
}

moe_status moe_set_tuning(const char *key, int32_t value) {
  if (!key || value < 0) return MOE_E_INVALID;
  if (!strcmp(key, "glu_ks")) {
    tuning().glu_ks = value;
  } else if (!strcmp(key, "down_ks")) {
    tuning().down_ks = value;
  } else if (!strcmp(key, "fused")) {
    tuning().fused = value;
  } else if (!strcmp(key, "fused_ksg")) {
    tuning().fused_ksg = value;
  } else if (!strcmp(key, "fused_ksd")) {
    tuning().fused_ksd = value;
  } else if (!strcmp(key, "layer")) {
    if (value > 1) return MOE_E_INVALID;
    tuning().layer = value;
  } else if (!strcmp(key, "layer_ksg")) {
    tuning().layer_ksg = value;
  } else if (!strcmp(key, "layer_ksd")) {
    tuning().layer_ksd = value;
  } else if (!strcmp(key, "layer_order")) {
    tuning().layer_order = value;
  } else if (!strcmp(key, "layer_select")) {
    tuning().layer_select = value;
  } else if (!strcmp(key, "layer_log_copies")) {
    tuning().layer_log_copies = value;
  } else if (!strcmp(key, "layer_sel_copies")) {
    tuning().layer_sel_copies = value;
  } else if (!strcmp(key, "layer_sel_stride")) {
    tuning().layer_sel_stride = value;
  } else if (!strcmp(key, "block_fused")) {
    tuning().block_fused = value;
  } else if (!strcmp(key, "mid")) {
    tuning().mid = value;
  } else if (!strcmp(key, "mid_min_t")) {
    tuning().mid_min_t = value;
  } else if (!strcmp(key, "mid_max_t")) {
    tuning().mid_max_t = value;
  } else if (!strcmp(key, "mid_ksg")) {
    tuning().mid_ksg = value;
  } else if (!strcmp(key, "mid_ksd")) {
    tuning().mid_ksd = value;
  } else if (!strcmp(key, "mid_kss")) {
    tuning().mid_kss = value;
  } else if (!strcmp(key, "prefill_min_t")) {
    tuning().prefill_min_t = value;
  } else if (!strcmp(key, "route_mfma")) {
    tuning().route_mfma = value;
  } else {
    return MOE_E_INVALID;
  }
  return MOE_OK;
}

moe_status moe_route(const void *x, int32_t x_dtype, int32_t T, const moe_qmat *router,
                     const float *logit_bias, int32_t k, int32_t *ids, float *gates,
                     float *logits, void *ws, size_t ws_bytes, void *stream) {
  if (!x || !aligned16(x) || !dtype_x_ok(x_dtype) || T < 1 || !ids || !gates || !ws)
    return MOE_E_INVALID;
  moe_status st = check_router(router);
  if (st) return st;
  const int E = router->rows, D = router->cols;
  if (k < 1 || k > E || k > kMaxK) return MOE_E_INVALID;
  const Dims d{T, k, E, D, 64, 0};
  if (ws_bytes < workspace_bytes(d)) return MOE_E_WORKSPACE;
  Workspace w = carve(ws, d);
  RouteLaunch a{};
  a.x = x; a.f16x = x_dtype == MOE_F16; a.T = T; a.D = D; a.E = E; a.k = k;
  a.codes = (const uint8_t *)router->codes; a.meta = (const uint32_t *)router->meta;
  a.logit_bias = logit_bias;
  a.logits = logits ? logits : w.logits; a.ids = ids; a.gates = gates;
  a.xp = w.xp; a.xs = w.xs; a.counters = w.counters;
  a.table = nullptr; a.slot_blob = nullptr;
  a.zero = nullptr; a.zero_words = 0; a.zero2 = nullptr; a.zero2_count = 0; a.zero2_stride = 0;
  a.rtag = (uint64_t *)(w.layer + kRouteTagOff); a.rep = (uint32_t *)(w.layer + kRouteEpochOff);
  a.rowtag = (uint64_t *)(w.layer + kRowTagOff); a.rowep = (uint32_t *)(w.layer + kRowEpochOff);
  a.err = w.err;
  return hip_status(launch_route(a, (hipStream_t)stream));
}

moe_status moe_expert_ffn(const void *x, int32_t x_dtype, int32_t T, const moe_bank *bank,
                          const int32_t *ids, int32_t k, float *y, void *ws, size_t ws_bytes,
                          void *stream) {
  if (!x || !aligned16(x) || !dtype_x_ok(x_dtype) || T < 1 || !y || !ws) return MOE_E_INVALID;
  if (!bank) return MOE_E_INVALID;
  moe_status st = check_bank(bank, bank->D);
  if (st) return st;
  if (k < 1 || k > kMaxK || (!ids && k != 1)) return MOE_E_INVALID;
  const Dims d{T, k, bank->E, bank->D, bank->F, 0};
  if (ws_bytes < workspace_bytes(d)) return MOE_E_WORKSPACE;
  Workspace w = carve(ws, d);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_prep_x(x, x_dtype == MOE_F16, T, bank->D, w.xp, w.xs, s);
  if (e != hipSuccess) return MOE_E_HIP;
  ExpertLaunch a{};
  a.f16x = x_dtype == MOE_F16; a.T = T; a.k = k; a.D = bank->D; a.E = bank->E;
  a.xp = w.xp; a.xs = w.xs; a.ids = ids; a.gates = nullptr; a.slot_blob = nullptr;
  a.rblobs = bank->blobs; a.F = bank->F; a.sblobs = nullptr; a.Fs = 0;
  a.h = w.h; a.hs = w.hs; a.part = w.part; a.counters = w.counters;
  a.y = y; a.out = nullptr; a.out_dtype = MOE_F32;
  a.glu_first = 0; a.glu_count = glu_blocks(a); a.glu_ks = 0;
  e = launch_glu(a, s);
  if (e != hipSuccess) return MOE_E_HIP;
  return hip_status(launch_down(a, false, s));
}

moe_status moe_combine(const float *y, const float *gates, const float *y_shared, int32_t T,
                       int32_t k, int32_t D, void *out, int32_t out_dtype, void *stream) {
  if (!y || !gates || !out || T < 1 || k < 1 || D < 1 || !dtype_out_ok(out_dtype))
    return MOE_E_INVALID;
  return hip_status(
      launch_combine(y, gates, y_shared, T, k, D, out, out_dtype, (hipStream_t)stream));
}

moe_status moe_permute(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv, void *stream) {
  if (!ids || !counts || !offsets || !perm || !inv) return MOE_E_INVALID;
  if (T < 1 || k < 1 || E < 1 || E > kMaxE || (long)T * k > 65536) return MOE_E_INVALID;
  return hip_status(launch_permute(ids, T, k, E, counts, offsets, perm, inv, nullptr, nullptr,
                                   0, (hipStream_t)stream));
}

moe_status moe_layer_forward(const void *x, int32_t x_dtype, int32_t T, const moe_qmat *router,
                             const float *logit_bias, int32_t k, const moe_bank *routed,
                             const moe_bank *shared, moe_pool *pool, int32_t layer, void *out,
                             int32_t out_dtype, int32_t *ids_out, float *gates_out, void *ws,
                             size_t ws_bytes, void *stream) {
  if (!ws) return MOE_E_INVALID;
  Dims d;
  moe_status st = layer_forward_args(x, x_dtype, T, router, k, routed, shared, pool, layer, out,
                                     out_dtype, &d);
  if (st) return st;
  const int E = d.E, D = d.D, F = d.F, Fs = d.Fs;
  if (ws_bytes < workspace_bytes(d)) return MOE_E_WORKSPACE;
  Workspace w = carve(ws, d);
  hipStream_t s = (hipStream_t)stream;

  // decode: router, selection, experts and combine in one launch
  LayerLaunch L{};
  init_layer_launch(&L, x, x_dtype, d, router, logit_bias, k, routed, shared, pool, out,
                    out_dtype, ids_out, gates_out);
  // Streamed experts run the layer kernel in two launches with the slot plan
  // between them; only when every expert of the call is sure to fit the
  // slots, so that the plan cannot fail once the first launch has left its
  // blocks' epochs and partial sums waiting for the second.
  const bool use_layer = (!pool || T * k <= pool_slots(pool)) && plan_layer(w, &L);
  if (use_layer && !pool) {
    const int pi = prof_begin(s);
    return hip_status(prof_end(pi, s, launch_layer(L, s)));
  }

  if (use_layer && pool) {
    // Streamed experts, two launches of the layer kernel.  First its router
    // blocks and the shared expert's blocks (dispatch order 1: router,
    // shared, routed); the ranking waves also store the selection into host
    // memory.  The host plans the slots from it and the side stream copies
    // the missing experts while the shared blocks run; then the routed
    // blocks take the ids and gates from the selection lines, as in the
    // resident launch, and each rank's blob from the pool.  Same blocks,
    // same splits: the output is bitwise the resident one.
    L.select = 0;
    L.order = 1;
    st = pool_layer_sel(pool, T, k, &L.host_sel, &L.host_epoch);
    if (st) return st;
    const int grid = layer_grid(L);
    const int first = layer_router_blocks(L) + layer_shared_blocks(L);
    if (launch_layer_ordered(L, 0, first, s) != hipSuccess) return MOE_E_HIP;
    st = pool_fetch_ids(pool, nullptr, T * k, s);
    if (st) return st;
    const void *const *slots = nullptr;
    st = pool_plan_and_copy(pool, layer, T, k, s, nullptr, &slots);
    if (st) return st;
    L.host_sel = nullptr;
    L.given_blob = slots;
    if (launch_layer_ordered(L, first, grid - first, s) != hipSuccess) return MOE_E_HIP;
    return pool_slots_read(pool, s);
  }

  RouteLaunch r{};
  r.zero = nullptr; r.zero_words = 0; r.zero2 = nullptr; r.zero2_count = 0; r.zero2_stride = 0;
  r.x = x; r.f16x = x_dtype == MOE_F16; r.T = T; r.D = D; r.E = E; r.k = k;
  r.codes = (const uint8_t *)router->codes; r.meta = (const uint32_t *)router->meta;
  r.logit_bias = logit_bias;
  r.logits = w.logits; r.ids = ids_out ? ids_out : w.ids; r.gates = gates_out ? gates_out : w.gates;
  r.xp = w.xp; r.xs = w.xs; r.counters = w.counters;
  r.rtag = (uint64_t *)(w.layer + kRouteTagOff); r.rep = (uint32_t *)(w.layer + kRouteEpochOff);
  r.rowtag = (uint64_t *)(w.layer + kRowTagOff); r.rowep = (uint32_t *)(w.layer + kRowEpochOff);
  r.err = w.err;
  // resident experts: the router also resolves each selected expert's blob;
  // streamed experts: the pool writes the slot addresses after its copies
  r.table = pool ? nullptr : routed->blobs;
  r.slot_blob = pool ? nullptr : w.slot_blob;
  if (pool) {
    st = pool_route_ids(pool, T, k, &r.host_ids, &r.host_flag, &r.host_epoch);
    if (st) return st;
  }

  ExpertLaunch a{};
  a.f16x = r.f16x; a.T = T; a.k = k; a.D = D; a.E = E;
  a.xp = w.xp; a.xs = w.xs; a.ids = r.ids; a.gates = r.gates; a.slot_blob = w.slot_blob;
  a.rblobs = pool ? nullptr : routed->blobs; a.F = F;
  a.sblobs = shared ? shared->blobs : nullptr; a.Fs = Fs;
  a.h = w.h; a.hs = w.hs; a.part = w.part; a.counters = w.counters;
  a.y = nullptr; a.out = out; a.out_dtype = out_dtype;
  // batched decode: each distinct expert and the shared expert read once for
  // every token that uses it (router kernel, then the two kernels)
  if (!pool && !use_layer && tuning().mid && T >= tuning().mid_min_t && T <= tuning().mid_max_t &&
      T <= kMaxMidT && T * k <= 64 && T < tuning().prefill_min_t) {
    MidLaunch m{};
    m.a = a;
    m.a.rblobs = routed->blobs;
    m.gacc = w.mgacc;
    m.dacc = w.mdacc;
    m.err = w.err;
    plan_mid(&m);
    m.gcnt = w.counters;
    m.dcnt = w.counters + m.n_tiles;
    if (m.n_tiles + D / 64 > kMaxSplitBlocks) return MOE_E_UNSUPPORTED;
    if (launch_route(r, s) != hipSuccess) return MOE_E_HIP;
    const int pi = prof_begin(s);
    return hip_status(prof_end(pi, s, launch_mid(m, s)));
  }
  // streamed experts whose call may need more experts than the slots hold:
  // grouped kernels in slot-sized batches of experts
  const bool batched = pool && T * k > pool_slots(pool);
  if (batched && (T * k > 65536 || D / 64 > kMaxDGroups || F / 64 > kMaxHGroups ||
                  Fs / 64 > kMaxHGroups))
    return MOE_E_UNSUPPORTED;
  FusedLaunch f;
  const bool fused = !use_layer && !batched && tuning().fused && plan_fused(a, w, &f);
  if (fused) {
    r.zero = f.slot_cnt;
    r.zero_words = T * (k + 1);
    r.zero2 = f.slot_flag;
    r.zero2_count = T * (k + 1) * kFlagCopies;
    r.zero2_stride = 32;
  }
  if (launch_route(r, s) != hipSuccess) return MOE_E_HIP;
  // the grouped kernels' launch (prefill chunks, batched streamed calls)
  auto prefill_launch = [&](const void *const *rblobs) {
    PrefillLaunch pl{};
    pl.f16x = r.f16x; pl.T = T; pl.k = k; pl.E = E; pl.D = D; pl.F = F; pl.Fs = Fs;
    pl.counts = w.perm_counts; pl.offsets = w.perm_offsets; pl.perm = w.perm; pl.inv = w.perm_inv;
    pl.items = w.perm_items; pl.n_items = w.perm_n_items;
    pl.item_info = w.perm_info; pl.item_blob = w.perm_iblob;
    pl.gates = r.gates; pl.rblobs = rblobs; pl.sblobs = shared ? shared->blobs : nullptr;
    pl.xp = w.xp; pl.xs = w.xs;
    pl.hp = w.hplanes; pl.plane = (size_t)T * k * F + (size_t)T * Fs;
    pl.hsum = w.hsum; pl.y = w.y; pl.ys = w.ys; pl.out = out; pl.out_dtype = out_dtype;
    // the shared down projection in as many splits as make its blocks no
    // longer than a routed expert's
    pl.sks = shared ? min(kMaxSharedSplits, max(1, (Fs / 64 + F / 64 - 1) / (F / 64))) : 1;
    pl.batch_blob = nullptr;
    pl.skip_combine = 0;
    return pl;
  };
  if (batched) {
    // Streamed call with more (token, slot) pairs than slots: the work list
    // of the grouped kernels, the ids back to the host, then for each batch
    // of at most `slots` distinct experts (first-use order) the pool fetches
    // the batch's misses and the gate/up and down kernels run the batch's
    // items only (the shared expert with the first batch); one combine at
    // the end.  Each item computes as in the resident call: the output is
    // bitwise the resident grouped path's.
    const void *const *ltab = pool_table(pool, layer);
    if (launch_permute(r.ids, T, k, E, w.perm_counts, w.perm_offsets, w.perm, w.perm_inv,
                       w.perm_items, w.perm_n_items, kPrefillRows, s, w.perm_info,
                       w.perm_iblob, ltab) != hipSuccess)
      return MOE_E_HIP;
    st = pool_fetch_ids(pool, r.ids, T * k, s);
    if (st) return st;
    std::vector<std::vector<int>> batches;
    st = pool_batches(pool, T, k, &batches);
    if (st) return st;
    PrefillLaunch pl = prefill_launch(ltab);
    pl.skip_combine = 1;
    for (size_t b = 0; b < batches.size(); ++b) {
      const void *const *bt = nullptr;
      st = pool_plan_batch(pool, layer, (int)b, batches[b], T, k, s, &bt);
      if (st) return st;
      pl.batch_blob = bt;
      pl.sblobs = b == 0 && shared ? shared->blobs : nullptr;
      if (launch_prefill_experts(pl, s) != hipSuccess) return MOE_E_HIP;
      st = pool_batch_done(pool, s);
      if (st) return st;
    }
    pl.sblobs = shared ? shared->blobs : nullptr;
    pl.batch_blob = nullptr;
    if (launch_prefill_combine(pl, s) != hipSuccess) return MOE_E_HIP;
    return pool_batches_read(pool, s);
  }
  if (fused && !pool) {
    const int pi = prof_begin(s);
    return hip_status(prof_end(pi, s, launch_fused(f, s)));
  }

  if (pool && fused) {
    // Streamed experts: ids back to the host; the shared expert's gate/up
    // tiles run while the host plans and the side stream copies the missing
    // experts into HBM slots; then the routed tiles, down and combine.  The
    // splits are those of the resident launch, so results are bitwise equal.
    st = pool_fetch_ids(pool, r.ids, T * k, s);
    if (st) return st;
    const int n_routed_tiles = T * k * (F / 64);
    FusedLaunch fs = f;
    fs.tile_begin = n_routed_tiles;
    fs.do_down = 0;
    if (launch_fused(fs, s) != hipSuccess) return MOE_E_HIP;
    const void *const *slots = nullptr;
    st = pool_plan_and_copy(pool, layer, T, k, s, nullptr, &slots);
    if (st) return st;
    FusedLaunch fr = f;
    fr.a.slot_blob = slots;
    fr.tile_end = n_routed_tiles;
    if (launch_fused(fr, s) != hipSuccess) return MOE_E_HIP;
    return pool_slots_read(pool, s);
  }
  // prefill chunk: group the (token, slot) pairs by expert, then matrix cores
  if (!pool && T >= tuning().prefill_min_t && T * k <= 65536 && D / 64 <= kMaxDGroups &&
      F / 64 <= kMaxHGroups && Fs / 64 <= kMaxHGroups) {
    if (launch_permute(r.ids, T, k, E, w.perm_counts, w.perm_offsets, w.perm, w.perm_inv,
                       w.perm_items, w.perm_n_items, kPrefillRows, s, w.perm_info,
                       w.perm_iblob, routed->blobs) !=
        hipSuccess)
      return MOE_E_HIP;
    const PrefillLaunch pl = prefill_launch(routed->blobs);
    const int pi = prof_begin(s);
    return hip_status(prof_end(pi, s, launch_prefill_experts(pl, s)));
  }

  const int routed_blocks = T * k * (F / 64);
  const int all_blocks = glu_blocks(a);
  a.slot_blob = pool ? nullptr : w.slot_blob;
  // one reduction split for the whole layer, so the streamed path (shared and
  // routed tiles launched apart) sums in the same order as the resident one
  a.glu_ks = pick_ks(all_blocks, D / 64, glu_min_ks(D), tuning().glu_ks);

  if (!pool) {
    a.glu_first = 0; a.glu_count = all_blocks;
    if (launch_glu(a, s) != hipSuccess) return MOE_E_HIP;
    return hip_status(launch_down(a, true, s));
  }

  // streamed experts, three-kernel shape (when the one-launch grid does not fit)
  st = pool_fetch_ids(pool, r.ids, T * k, s);
  if (st) return st;
  if (shared) {
    a.glu_first = routed_blocks; a.glu_count = all_blocks - routed_blocks;
    if (launch_glu(a, s) != hipSuccess) return MOE_E_HIP;
  }
  const void *const *table = nullptr;
  st = pool_plan_and_copy(pool, layer, T, k, s, &table, nullptr);
  if (st) return st;
  a.rblobs = table;
  a.glu_first = 0; a.glu_count = routed_blocks;
  if (launch_glu(a, s) != hipSuccess) return MOE_E_HIP;
  return hip_status(launch_down(a, true, s));
}


size_t moe_block_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t D, int32_t F,
                                 int32_t F_shared) {
  const size_t layer = moe_workspace_bytes(T, k, E, D, F, F_shared);
  if (!layer) return 0;
  return block_tail(layer, T, D).total;
}

moe_status moe_block_forward(const void *x, int32_t x_dtype, int32_t T, const float *w_pre,
                             const float *w_post, float eps, const moe_qmat *router,
                             const float *logit_bias, int32_t k, const moe_bank *routed,
                             const moe_bank *shared, moe_pool *pool, int32_t layer, void *out,
                             int32_t out_dtype, void *u_out, int32_t *ids_out, float *gates_out,
                             void *ws, size_t ws_bytes, void *stream) {
  if (!ws || !w_pre || !w_post || !(eps >= 0.0f) || !std::isfinite(eps)) return MOE_E_INVALID;
  Dims d;
  moe_status st = layer_forward_args(x, x_dtype, T, router, k, routed, shared, pool, layer, out,
                                     out_dtype, &d);
  if (st) return st;
  if (d.D > kBlockMaxD) return MOE_E_INVALID;
  if ((u_out && ((uintptr_t)u_out % 16)) || (uintptr_t)out % 16 || (uintptr_t)w_pre % 16 ||
      (uintptr_t)w_post % 16)
    return MOE_E_INVALID;
  // out may be x itself (the residual stream updated in place: each element
  // is read, then written, by one thread) but no other overlap
  const size_t xb = (size_t)T * d.D * 2;
  const size_t ob = (size_t)T * d.D * (out_dtype == MOE_F32 ? 4 : 2);
  const uintptr_t xa = (uintptr_t)x, oa = (uintptr_t)out;
  if (oa < xa + xb && xa < oa + ob && !(oa == xa && ob == xb)) return MOE_E_INVALID;
  if (u_out) {
    const uintptr_t ua = (uintptr_t)u_out;
    if ((ua < xa + xb && xa < ua + xb) || (ua < oa + ob && oa < ua + xb)) return MOE_E_INVALID;
  }
  const size_t lb = workspace_bytes(d);
  const BlockTail bt = block_tail(lb, T, d.D);
  if (ws_bytes < bt.total) return MOE_E_WORKSPACE;
  uint16_t *u = u_out ? (uint16_t *)u_out : (uint16_t *)((uint8_t *)ws + bt.u_off);
  float *y = (float *)((uint8_t *)ws + bt.y_off);
  hipStream_t s = (hipStream_t)stream;
  const int f16x = x_dtype == MOE_F16;
  if (!pool && tuning().block_fused && tuning().layer) {
    // one launch: the decode layer kernel normalises x in every role and
    // adds the post-norm and the residual to each completed output row
    LayerLaunch L{};
    init_layer_launch(&L, x, x_dtype, d, router, logit_bias, k, routed, shared, nullptr, out,
                      out_dtype, ids_out, gates_out);
    L.w_pre = w_pre; L.w_post = w_post; L.eps = eps;
    L.ybuf = (uint64_t *)((uint8_t *)ws + bt.yt_off); L.u_out = (uint16_t *)u_out;
    L.ocnt = (uint32_t *)((uint8_t *)ws + bt.cnt_off);
    Workspace w = carve(ws, d);
    if (plan_layer(w, &L)) {
      const int pi = prof_begin(s);
      return hip_status(prof_end(pi, s, launch_layer(L, s)));
    }
  }
  if (launch_block_pre(x, f16x, T, d.D, w_pre, eps, u, s) != hipSuccess) return MOE_E_HIP;
  st = moe_layer_forward(u, x_dtype, T, router, logit_bias, k, routed, shared, pool, layer, y,
                         MOE_F32, ids_out, gates_out, ws, lb, stream);
  if (st) return st;
  return hip_status(launch_block_post(y, x, f16x, T, d.D, w_post, eps, out, out_dtype, s));
}

}  // extern "C"
