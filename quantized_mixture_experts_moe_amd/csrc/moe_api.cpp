// C ABI of libmoe: argument checks, workspace carve-up and kernel dispatch.
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

Workspace carve(void *base, const Dims &d) {
  Carver c{(uint8_t *)base};
  Workspace w;
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
  w.perm_counts = c.take<int32_t>(d.E, 4);
  w.perm_offsets = c.take<int32_t>(d.E + 1, 4);
  w.perm = c.take<int32_t>(T * k, 4);
  w.perm_inv = c.take<int32_t>(T * k, 4);
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

}  // namespace

Workspace carve_workspace(void *base, const Dims &d) { return carve(base, d); }
size_t workspace_bytes(const Dims &d) { return carve(nullptr, d).total; }

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

moe_status moe_set_tuning(const char *key, int32_t value) {
  if (!key || value < 0) return MOE_E_INVALID;
  if (!strcmp(key, "glu_ks")) {
    tuning().glu_ks = value;
  } else if (!strcmp(key, "down_ks")) {
    tuning().down_ks = value;
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
  RouteLaunch a;
  a.x = x; a.f16x = x_dtype == MOE_F16; a.T = T; a.D = D; a.E = E; a.k = k;
  a.codes = (const uint8_t *)router->codes; a.meta = (const uint32_t *)router->meta;
  a.logit_bias = logit_bias;
  a.logits = logits ? logits : w.logits; a.ids = ids; a.gates = gates;
  a.xp = w.xp; a.xs = w.xs; a.counters = w.counters;
  a.table = nullptr; a.slot_blob = nullptr;
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
  return hip_status(launch_permute(ids, T, k, E, counts, offsets, perm, inv,
                                   (hipStream_t)stream));
}

moe_status moe_layer_forward(const void *x, int32_t x_dtype, int32_t T, const moe_qmat *router,
                             const float *logit_bias, int32_t k, const moe_bank *routed,
                             const moe_bank *shared, moe_pool *pool, int32_t layer, void *out,
                             int32_t out_dtype, int32_t *ids_out, float *gates_out, void *ws,
                             size_t ws_bytes, void *stream) {
  if (!x || !aligned16(x) || !dtype_x_ok(x_dtype) || T < 1 || !out || !dtype_out_ok(out_dtype) ||
      !ws)
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
  const int Fs = shared ? shared->F : 0;
  const Dims d{T, k, E, D, F, Fs};
  if (ws_bytes < workspace_bytes(d)) return MOE_E_WORKSPACE;
  Workspace w = carve(ws, d);
  hipStream_t s = (hipStream_t)stream;

  RouteLaunch r;
  r.x = x; r.f16x = x_dtype == MOE_F16; r.T = T; r.D = D; r.E = E; r.k = k;
  r.codes = (const uint8_t *)router->codes; r.meta = (const uint32_t *)router->meta;
  r.logit_bias = logit_bias;
  r.logits = w.logits; r.ids = ids_out ? ids_out : w.ids; r.gates = gates_out ? gates_out : w.gates;
  r.xp = w.xp; r.xs = w.xs; r.counters = w.counters;
  // resident experts: the router also resolves each selected expert's blob
  r.table = pool ? nullptr : routed->blobs;
  r.slot_blob = pool ? nullptr : w.slot_blob;
  if (launch_route(r, s) != hipSuccess) return MOE_E_HIP;

  ExpertLaunch a{};
  a.f16x = r.f16x; a.T = T; a.k = k; a.D = D; a.E = E;
  a.xp = w.xp; a.xs = w.xs; a.ids = r.ids; a.gates = r.gates; a.slot_blob = r.slot_blob;
  a.rblobs = pool ? nullptr : routed->blobs; a.F = F;
  a.sblobs = shared ? shared->blobs : nullptr; a.Fs = Fs;
  a.h = w.h; a.hs = w.hs; a.part = w.part; a.counters = w.counters;
  a.y = nullptr; a.out = out; a.out_dtype = out_dtype;
  const int routed_blocks = T * k * (F / 64);
  const int all_blocks = glu_blocks(a);
  // one reduction split for the whole layer, so the streamed path (shared and
  // routed tiles launched apart) sums in the same order as the resident one
  a.glu_ks = pick_ks(all_blocks, D / 64, glu_min_ks(D), tuning().glu_ks);

  if (!pool) {
    a.glu_first = 0; a.glu_count = all_blocks;
    if (launch_glu(a, s) != hipSuccess) return MOE_E_HIP;
    return hip_status(launch_down(a, true, s));
  }

  // Streamed experts: ids back to the host, shared expert on the GPU while the
  // host plans and the side stream copies the misses into HBM slots.
  st = pool_fetch_ids(pool, r.ids, T * k, s);
  if (st) return st;
  if (shared) {
    a.glu_first = routed_blocks; a.glu_count = all_blocks - routed_blocks;
    if (launch_glu(a, s) != hipSuccess) return MOE_E_HIP;
  }
  const void *const *table = nullptr;
  st = pool_plan_and_copy(pool, layer, T, k, s, &table);
  if (st) return st;
  a.rblobs = table;
  a.glu_first = 0; a.glu_count = routed_blocks;
  if (launch_glu(a, s) != hipSuccess) return MOE_E_HIP;
  return hip_status(launch_down(a, true, s));
}

}  // extern "C"
