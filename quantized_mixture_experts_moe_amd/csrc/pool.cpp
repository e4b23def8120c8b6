// HBM expert slot pool: per-layer slots refilled from pinned host memory.
//
// The pages keep 16 expert slots per layer, plan the fetches of each token's
// top-8 experts on the CPU against a least-frequently-used cache, and read the
// misses while the GPU computes the resident shared expert (es.news.hada.io,
// "Proceso de generacion de tokens"; stork.ai blog, "Mas inteligente que tu
// RAM"; yodev.dev, "El loop por token").  On MI355X the slots live in HBM and
// the misses come from page-locked host memory by hipMemcpyAsync on a side
// stream; the main stream waits on an event before the routed experts run.
#include "pool.h"

#include "store.h"

#include <string.h>

#include <algorithm>
#include <chrono>
#include <new>

struct moe_pool {
  int n_layers = 0, slots = 0, E = 0, D = 0, F = 0;
  size_t blob_bytes = 0;
  std::vector<const void *> host_blobs;       // [n_layers * E], pinned host
  std::vector<moe::LfuPlanner> planners;      // per layer
  uint8_t *slot_mem = nullptr;                // device [n_layers][slots][blob]
  const void **d_tables = nullptr;            // device [n_layers][E] blob pointers
  const void **h_tables = nullptr;            // pinned host mirror of d_tables
  int32_t *h_ids = nullptr;                   // pinned host ids of the last call
  const void **h_slot = nullptr;              // pinned per-pair slot addresses, read by the kernels
  const void *const *d_slot = nullptr;        // the device's address of h_slot
  int ids_cap = 0;
  hipStream_t side = nullptr;
  hipEvent_t ev_ids = nullptr, ev_copies = nullptr;
  hipEvent_t ev_slot = nullptr;               // after the last kernel that reads h_slot
  bool slot_pending = false;
  // ids written by the router kernel straight into host memory (fewer than
  // 16 tokens): per-token flags carry the call's epoch
  uint32_t *h_flag = nullptr;                 // pinned [ids_cap]
  int32_t *d_ids_host = nullptr;              // device addresses of h_ids and h_flag
  uint32_t *d_flag_host = nullptr;
  // or, from the one-launch layer's router blocks, (id, epoch) words
  uint64_t *h_sel = nullptr;                  // pinned [ids_cap]
  uint64_t *d_sel_host = nullptr;
  uint32_t epoch = 0;
  int ids_mode = 0;                           // this call's ids: 0 copied, 1 ids + flags, 2 words
  moe_pool_stats stats{};
  // the device table of a layer is uploaded by the next call that reads it
  // whenever the host table has changed since its last upload
  std::vector<char> table_dirty;
  hipEvent_t ev_table = nullptr;              // after the last upload (its source is h_tables)
  bool table_pending = false;
  int fail_copy_at = -1;                      // test hook: copies to let through before one fails
  // misses read from a store: page-locked staging buffers, one per slot
  // index (shared by the layers), each reusable once its copy is done
  moe_store *store = nullptr;
  size_t store_chunk = 0;
  uint8_t *staging = nullptr;
  std::vector<hipEvent_t> stg_ev;
  std::vector<char> stg_pending;
  // calls with more distinct experts than slots run in batches of at most
  // `slots` experts: one device-readable table per batch (pinned, coherent:
  // expert -> slot address, null for experts of other batches)
  const void **h_btab = nullptr;              // [max_batches][E]
  const void *const *d_btab = nullptr;
  int max_batches = 0;
  hipEvent_t ev_btab = nullptr;               // after the last kernel that reads h_btab
  bool btab_pending = false;
  hipEvent_t ev_batch = nullptr;              // after a batch's kernels (the next batch's copies wait)
};

namespace moe {

moe_status pool_check(const moe_pool *p, int layer, int E, int D, int k) {
  if (!p || layer < 0 || layer >= p->n_layers) return MOE_E_INVALID;
  if (p->E != E || p->D != D) return MOE_E_INVALID;
  if (k > p->slots) return MOE_E_POOL;
  return MOE_OK;
}

int pool_F(const moe_pool *p) { return p->F; }
int pool_slots(const moe_pool *p) { return p->slots; }

static moe_status ensure_ids(moe_pool *p, int n) {
  if (n > p->ids_cap) {
    // the kernels of earlier calls may still read h_slot
    if (p->slot_pending && hipEventSynchronize(p->ev_slot) != hipSuccess) return MOE_E_HIP;
    p->slot_pending = false;
    // and every earlier router kernel that writes h_ids and h_flag
    if (hipEventSynchronize(p->ev_ids) != hipSuccess) return MOE_E_HIP;
    if (p->h_ids) (void)hipHostFree(p->h_ids);
    if (p->h_slot) (void)hipHostFree(p->h_slot);
    if (p->h_flag) (void)hipHostFree(p->h_flag);
    if (p->h_sel) (void)hipHostFree(p->h_sel);
    p->h_ids = nullptr;
    p->h_slot = nullptr;
    p->h_flag = nullptr;
    p->h_sel = nullptr;
    p->ids_cap = 0;
    // coherent (uncached on the device): the kernels read what the host
    // wrote before their launch, and the host polls what they write
    const unsigned fl = hipHostMallocCoherent;
    if (hipHostMalloc((void **)&p->h_ids, sizeof(int32_t) * n, fl) != hipSuccess ||
        hipHostMalloc((void **)&p->h_slot, sizeof(void *) * n, fl) != hipSuccess ||
        hipHostMalloc((void **)&p->h_flag, sizeof(uint32_t) * n, fl) != hipSuccess ||
        hipHostMalloc((void **)&p->h_sel, sizeof(uint64_t) * n, fl) != hipSuccess)
      return MOE_E_HIP;
    for (int i = 0; i < n; ++i) p->h_flag[i] = 0u, p->h_sel[i] = 0u;
    p->epoch = 0;
    void *dv = nullptr, *di = nullptr, *df = nullptr, *ds = nullptr;
    if (hipHostGetDevicePointer(&dv, p->h_slot, 0) != hipSuccess ||
        hipHostGetDevicePointer(&di, p->h_ids, 0) != hipSuccess ||
        hipHostGetDevicePointer(&df, p->h_flag, 0) != hipSuccess ||
        hipHostGetDevicePointer(&ds, p->h_sel, 0) != hipSuccess)
      return MOE_E_HIP;
    p->d_slot = (const void *const *)dv;
    p->d_ids_host = (int32_t *)di;
    p->d_flag_host = (uint32_t *)df;
    p->d_sel_host = (uint64_t *)ds;
    p->ids_cap = n;
  }
  return MOE_OK;
}

// The next call's epoch (flags and words of earlier calls hold older ones).
static void next_epoch(moe_pool *p) {
  if (++p->epoch == 0) {  // wrapped: no flag or word may hold the new epoch already
    for (int i = 0; i < p->ids_cap; ++i) p->h_flag[i] = 0u, p->h_sel[i] = 0u;
    p->epoch = 1;
  }
}

moe_status pool_route_ids(moe_pool *p, int T, int k, int32_t **host_ids, uint32_t **host_flag,
                          uint32_t *epoch) {
  *host_ids = nullptr;
  *host_flag = nullptr;
  *epoch = 0;
  p->ids_mode = 0;
  if (T >= 16) return MOE_OK;  // the matrix-core router: ids copied back
  const moe_status st = ensure_ids(p, T * k);
  if (st) return st;
  next_epoch(p);
  *host_ids = p->d_ids_host;
  *host_flag = p->d_flag_host;
  *epoch = p->epoch;
  p->ids_mode = 1;
  return MOE_OK;
}

moe_status pool_layer_sel(moe_pool *p, int T, int k, uint64_t **host_sel, uint32_t *epoch) {
  const moe_status st = ensure_ids(p, T * k);
  if (st) return st;
  next_epoch(p);
  *host_sel = p->d_sel_host;
  *epoch = p->epoch;
  p->ids_mode = 2;
  return MOE_OK;
}

moe_status pool_fetch_ids(moe_pool *p, const int32_t *d_ids, int n, hipStream_t s) {
  if (p->ids_mode) {
    // a kernel writes them into host memory; the event is the fallback wait
    return hipEventRecord(p->ev_ids, s) == hipSuccess ? MOE_OK : MOE_E_HIP;
  }
  const moe_status st = ensure_ids(p, n);
  if (st) return st;
  if (hipMemcpyAsync(p->h_ids, d_ids, sizeof(int32_t) * n, hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return MOE_E_HIP;
  if (hipEventRecord(p->ev_ids, s) != hipSuccess) return MOE_E_HIP;
  return MOE_OK;
}

// Waits until the router kernel's per-token flags carry the call's epoch:
// a short spin (the ids arrive a few microseconds after the kernel ends),
// then a blocking wait for the kernel, after which they must be there.
static moe_status wait_direct_ids(moe_pool *p, int T, int k) {
  auto ready = [&]() {
    if (p->ids_mode == 1) {
      for (int t = 0; t < T; ++t)
        if (__atomic_load_n(p->h_flag + t, __ATOMIC_ACQUIRE) != p->epoch) return false;
      return true;
    }
    for (int i = 0; i < T * k; ++i) {
      const uint64_t v = __atomic_load_n(p->h_sel + i, __ATOMIC_ACQUIRE);
      if ((uint32_t)(v >> 32) != p->epoch) return false;
      p->h_ids[i] = (int32_t)(uint32_t)v;
    }
    return true;
  };
  const auto t0 = std::chrono::steady_clock::now();
  while (!ready()) {
    if (std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(2000)) {
      if (hipEventSynchronize(p->ev_ids) != hipSuccess) return MOE_E_HIP;
      return ready() ? MOE_OK : MOE_E_HIP;
    }
  }
  return MOE_OK;
}

// The call's ids are in h_ids (copied back, or written by the router kernel).
static moe_status wait_ids(moe_pool *p, int T, int k) {
  return p->ids_mode ? wait_direct_ids(p, T, k)
                     : (hipEventSynchronize(p->ev_ids) == hipSuccess ? MOE_OK : MOE_E_HIP);
}

namespace {
// Misses go host -> HBM by hipMemcpyAsync on the pool's side stream.
struct HipCopyEngine final : CopyEngine {
  hipStream_t side;
  explicit HipCopyEngine(hipStream_t s) : side(s) {}
  int copy(int, int, void *dst, const void *src, size_t bytes) override {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, side) == hipSuccess ? 0 : 1;
  }
};

// Misses read from the store: copy() records them; flush() reads all of the
// call's missing blobs at once (every piece of every blob spread over the
// store's threads) into the staging buffers of their slots, then enqueues the
// host -> HBM copies on the side stream.
struct StoreCopyEngine final : CopyEngine {
  moe_pool *p;
  int layer;
  std::vector<int32_t> experts;
  std::vector<int> slots;
  std::vector<void *> dsts;
  StoreCopyEngine(moe_pool *pool, int l) : p(pool), layer(l) {}
  int copy(int expert, int slot, void *dst, const void *, size_t) override {
    experts.push_back(expert);
    slots.push_back(slot);
    dsts.push_back(dst);
    return 0;
  }
  int flush() override {
    if (experts.empty()) return 0;
    const size_t stride = store_stride_of(p->store);
    std::vector<void *> stg(experts.size());
    for (size_t i = 0; i < experts.size(); ++i) {
      const int s = slots[i];
      // the staging buffer's previous copy (any layer) has left it
      if (p->stg_pending[s]) {
        if (hipEventSynchronize(p->stg_ev[s]) != hipSuccess) return 1;
        p->stg_pending[s] = 0;
      }
      stg[i] = p->staging + (size_t)s * stride;
    }
    if (store_read(p->store, layer, experts.data(), (int)experts.size(), stg.data(),
                   p->store_chunk) != MOE_OK)
      return 1;
    for (size_t i = 0; i < experts.size(); ++i) {
      if (hipMemcpyAsync(dsts[i], stg[i], p->blob_bytes, hipMemcpyHostToDevice, p->side) !=
              hipSuccess ||
          hipEventRecord(p->stg_ev[slots[i]], p->side) != hipSuccess)
        return 1;
      p->stg_pending[slots[i]] = 1;
    }
    return 0;
  }
};
}  // namespace

moe_status pool_plan_and_copy(moe_pool *p, int layer, int T, int k, hipStream_t s,
                              const void *const **table, const void *const **slot_blob) {
  const moe_status ws = wait_ids(p, T, k);
  if (ws) return ws;
  // the host table may still be the source of an earlier upload
  if (p->table_pending) {
    if (hipEventSynchronize(p->ev_table) != hipSuccess) return MOE_E_HIP;
    p->table_pending = false;
  }
  const void **tab = p->h_tables + (size_t)layer * p->E;
  uint8_t *base = p->slot_mem + (size_t)layer * p->slots * p->blob_bytes;
  LayerPlanArgs a;
  a.ids = p->h_ids; a.n = T * k; a.E = p->E;
  a.slot_base = base; a.blob_bytes = p->blob_bytes;
  a.host_blobs = p->store ? nullptr : p->host_blobs.data() + (size_t)layer * p->E;
  a.table = tab;
  HipCopyEngine hip_eng(p->side);
  StoreCopyEngine store_eng(p, layer);
  CopyEngine *ce = p->store ? (CopyEngine *)&store_eng : (CopyEngine *)&hip_eng;
  FailingCopyEngine fail(ce, p->fail_copy_at);
  if (p->fail_copy_at >= 0) ce = &fail;
  const PlanResult r = plan_layer_call(p->planners[layer], a, *ce, &p->stats);
  if (p->fail_copy_at >= 0) p->fail_copy_at = fail.remaining();
  // a failed copy may have changed the table too (invalidated slots)
  p->table_dirty[layer] = true;
  if (r.status) return r.status;
  bool queued = r.copies > 0;
  if (table && p->table_dirty[layer]) {
    // every change of the host table since the last upload (this call's and
    // those of calls that only read the per-pair slot addresses)
    if (hipMemcpyAsync(p->d_tables + (size_t)layer * p->E, tab, sizeof(void *) * p->E,
                       hipMemcpyHostToDevice, p->side) != hipSuccess)
      return MOE_E_HIP;
    if (hipEventRecord(p->ev_table, p->side) != hipSuccess) return MOE_E_HIP;
    p->table_pending = true;
    p->table_dirty[layer] = false;
    queued = true;
  }
  if (slot_blob) {
    // the kernels read the addresses from pinned host memory: no copy, and
    // with every expert resident nothing for stream s to wait on.  The
    // previous reader has finished (it precedes this call's id readback on
    // the stream; the event covers callers that switch streams).
    if (p->slot_pending && hipEventSynchronize(p->ev_slot) != hipSuccess) return MOE_E_HIP;
    for (int i = 0; i < T * k; ++i) p->h_slot[i] = tab[p->h_ids[i]];
    *slot_blob = p->d_slot;
  }
  if (queued) {
    if (hipEventRecord(p->ev_copies, p->side) != hipSuccess) return MOE_E_HIP;
    if (hipStreamWaitEvent(s, p->ev_copies, 0) != hipSuccess) return MOE_E_HIP;
  }
  if (table) *table = p->d_tables + (size_t)layer * p->E;
  return MOE_OK;
}

moe_status pool_batches(moe_pool *p, int T, int k, std::vector<std::vector<int>> *batches) {
  const moe_status ws = wait_ids(p, T, k);
  if (ws) return ws;
  std::vector<char> seen(p->E, 0);
  std::vector<int> order;
  for (int i = 0; i < T * k; ++i) {
    const int e = p->h_ids[i];
    if (e < 0 || e >= p->E) return MOE_E_POOL;
    if (!seen[e]) {
      seen[e] = 1;
      order.push_back(e);
    }
  }
  batches->clear();
  for (size_t i = 0; i < order.size(); i += p->slots)
    batches->emplace_back(order.begin() + i,
                          order.begin() + std::min(order.size(), i + (size_t)p->slots));
  return (int)batches->size() <= p->max_batches ? MOE_OK : MOE_E_POOL;
}

moe_status pool_plan_batch(moe_pool *p, int layer, int b, const std::vector<int> &experts, int T,
                           int k, hipStream_t s, const void *const **btab) {
  if (b < 0 || b >= p->max_batches) return MOE_E_POOL;
  // the previous batch's kernels read slots this batch may evict
  if (b > 0 && hipStreamWaitEvent(p->side, p->ev_batch, 0) != hipSuccess) return MOE_E_HIP;
  // the kernels of an earlier call may still read the batch tables
  if (b == 0 && p->btab_pending) {
    if (hipEventSynchronize(p->ev_btab) != hipSuccess) return MOE_E_HIP;
    p->btab_pending = false;
  }
  if (p->table_pending) {
    if (hipEventSynchronize(p->ev_table) != hipSuccess) return MOE_E_HIP;
    p->table_pending = false;
  }
  // this batch's uses, in (token, slot) order: one lookup each
  std::vector<char> in(p->E, 0);
  for (int e : experts) in[e] = 1;
  std::vector<int32_t> uses;
  for (int i = 0; i < T * k; ++i)
    if (in[p->h_ids[i]]) uses.push_back(p->h_ids[i]);
  const void **tab = p->h_tables + (size_t)layer * p->E;
  LayerPlanArgs a;
  a.ids = uses.data(); a.n = (int)uses.size(); a.E = p->E;
  a.slot_base = p->slot_mem + (size_t)layer * p->slots * p->blob_bytes;
  a.blob_bytes = p->blob_bytes;
  a.host_blobs = p->store ? nullptr : p->host_blobs.data() + (size_t)layer * p->E;
  a.table = tab;
  HipCopyEngine hip_eng(p->side);
  StoreCopyEngine store_eng(p, layer);
  CopyEngine *ce = p->store ? (CopyEngine *)&store_eng : (CopyEngine *)&hip_eng;
  FailingCopyEngine fail(ce, p->fail_copy_at);
  if (p->fail_copy_at >= 0) ce = &fail;
  const PlanResult r = plan_layer_call(p->planners[layer], a, *ce, &p->stats);
  if (p->fail_copy_at >= 0) p->fail_copy_at = fail.remaining();
  p->table_dirty[layer] = true;
  if (r.status) return r.status;
  const void **bt = p->h_btab + (size_t)b * p->E;
  for (int e = 0; e < p->E; ++e) bt[e] = nullptr;
  for (int e : experts) bt[e] = tab[e];
  if (r.copies > 0) {
    if (hipEventRecord(p->ev_copies, p->side) != hipSuccess) return MOE_E_HIP;
    if (hipStreamWaitEvent(s, p->ev_copies, 0) != hipSuccess) return MOE_E_HIP;
  }
  *btab = p->d_btab + (size_t)b * p->E;
  return MOE_OK;
}

moe_status pool_batch_done(moe_pool *p, hipStream_t s) {
  return hipEventRecord(p->ev_batch, s) == hipSuccess ? MOE_OK : MOE_E_HIP;
}

moe_status pool_batches_read(moe_pool *p, hipStream_t s) {
  if (hipEventRecord(p->ev_btab, s) != hipSuccess) return MOE_E_HIP;
  p->btab_pending = true;
  return MOE_OK;
}

const void *const *pool_table(const moe_pool *p, int layer) {
  return p->d_tables + (size_t)layer * p->E;
}

moe_status pool_slots_read(moe_pool *p, hipStream_t s) {
  if (hipEventRecord(p->ev_slot, s) != hipSuccess) return MOE_E_HIP;
  p->slot_pending = true;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_lfu_replay(int32_t slots, int32_t E, int32_t k, int32_t n_tokens,
                          const int32_t *ids, int32_t *events) {
  return moe_cache_replay(0, slots, E, k, n_tokens, ids, events);
}

moe_status moe_pool_fail_copy(moe_pool *p, int32_t after) {
  if (!p || after < -1) return MOE_E_INVALID;
  p->fail_copy_at = after;
  return MOE_OK;
}

moe_status moe_pool_set_policy(moe_pool *p, int32_t policy) {
  if (!p || policy < 0 || policy > 1) return MOE_E_INVALID;
  for (auto &pl : p->planners) pl.set_policy(policy);
  return MOE_OK;
}

moe_status moe_cache_replay(int32_t policy, int32_t slots, int32_t E, int32_t k,
                            int32_t n_tokens, const int32_t *ids, int32_t *events) {
  if (slots < 1 || E < 1 || k < 1 || k > slots || n_tokens < 0 || !ids || !events ||
      policy < 0 || policy > 1)
    return MOE_E_INVALID;
  LfuPlanner pl(slots, E);
  pl.set_policy(policy);
  std::vector<LfuPlanner::Event> ev;
  for (int t = 0; t < n_tokens; ++t) {
    const int32_t *row = ids + (size_t)t * k;
    for (int j = 0; j < k; ++j) {
      if (row[j] < 0 || row[j] >= E) return MOE_E_INVALID;
      for (int i = 0; i < j; ++i)
        if (row[i] == row[j]) return MOE_E_INVALID;
    }
    ev.clear();
    if (!pl.access(row, k, &ev)) return MOE_E_POOL;
    for (int j = 0; j < k; ++j) {
      int32_t *o = events + ((size_t)t * k + j) * 4;
      o[0] = ev[j].expert;
      o[1] = ev[j].slot;
      o[2] = ev[j].hit;
      o[3] = ev[j].evicted;
    }
  }
  return MOE_OK;
}

static moe_status pool_create(moe_pool **out, int32_t n_layers, int32_t slots, int32_t E,
                              int32_t D, int32_t F, const void *const *host_blobs,
                              moe_store *store, size_t chunk) {
  moe_pool *p = new (std::nothrow) moe_pool;
  if (!p) return MOE_E_POOL;
  p->n_layers = n_layers; p->slots = slots; p->E = E; p->D = D; p->F = F;
  p->blob_bytes = blob_layout(D, F).total;
  if (host_blobs) p->host_blobs.assign(host_blobs, host_blobs + (size_t)n_layers * E);
  p->store = store;
  p->store_chunk = chunk;
  for (int l = 0; l < n_layers; ++l) p->planners.emplace_back(slots, E);
  p->table_dirty.assign(n_layers, 0);
  bool ok = hipMalloc((void **)&p->slot_mem, (size_t)n_layers * slots * p->blob_bytes) ==
            hipSuccess;
  ok = ok && hipMalloc((void **)&p->d_tables, sizeof(void *) * n_layers * E) == hipSuccess;
  ok = ok && hipHostMalloc((void **)&p->h_tables, sizeof(void *) * n_layers * E,
                           hipHostMallocDefault) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_ids, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_copies, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_slot, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_table, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_btab, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_batch, hipEventDisableTiming) == hipSuccess;
  p->max_batches = (E + slots - 1) / slots;
  ok = ok && hipHostMalloc((void **)&p->h_btab, sizeof(void *) * p->max_batches * E,
                           hipHostMallocCoherent) == hipSuccess;
  if (ok) {
    void *dv = nullptr;
    ok = hipHostGetDevicePointer(&dv, p->h_btab, 0) == hipSuccess;
    p->d_btab = (const void *const *)dv;
  }
  if (ok) {
    // every table entry starts at the layer's first slot (nothing resident yet)
    for (int l = 0; l < n_layers; ++l)
      for (int e = 0; e < E; ++e)
        p->h_tables[(size_t)l * E + e] = p->slot_mem + (size_t)l * slots * p->blob_bytes;
    ok = hipMemcpy(p->d_tables, p->h_tables, sizeof(void *) * n_layers * E,
                   hipMemcpyHostToDevice) == hipSuccess;
  }
  if (ok && store) {
    ok = hipHostMalloc((void **)&p->staging, (size_t)slots * store_stride_of(store),
                       hipHostMallocDefault) == hipSuccess;
    p->stg_ev.assign(slots, nullptr);
    p->stg_pending.assign(slots, 0);
    for (int s = 0; ok && s < slots; ++s)
      ok = hipEventCreateWithFlags(&p->stg_ev[s], hipEventDisableTiming) == hipSuccess;
  }
  if (!ok) {
    moe_pool_destroy(p);
    return MOE_E_HIP;
  }
  *out = p;
  return MOE_OK;
}

moe_status moe_pool_create(moe_pool **out, int32_t n_layers, int32_t slots, int32_t E, int32_t D,
                           int32_t F, const void *const *host_blobs) {
  if (!out || n_layers < 1 || slots < 1 || E < 1 || slots > E || !host_blobs) return MOE_E_INVALID;
  if (D < 64 || F < 64 || D % 64 || F % 64) return MOE_E_INVALID;
  for (size_t i = 0; i < (size_t)n_layers * E; ++i)
    if (!host_blobs[i]) return MOE_E_INVALID;
  return pool_create(out, n_layers, slots, E, D, F, host_blobs, nullptr, 0);
}

moe_status moe_pool_create_store(moe_pool **out, int32_t slots, moe_store *store,
                                 size_t chunk_bytes) {
  if (!out || !store) return MOE_E_INVALID;
  const int E = store_E(store);
  if (slots < 1 || slots > E) return MOE_E_INVALID;
  return pool_create(out, store_layers(store), slots, E, store_D(store), store_F(store), nullptr,
                     store, chunk_bytes);
}

moe_status moe_pool_destroy(moe_pool *p) {
  if (!p) return MOE_E_INVALID;
  if (p->side) (void)hipStreamSynchronize(p->side);
  if (p->slot_pending) (void)hipEventSynchronize(p->ev_slot);
  if (p->btab_pending) (void)hipEventSynchronize(p->ev_btab);
  if (p->slot_mem) (void)hipFree(p->slot_mem);
  if (p->d_tables) (void)hipFree(p->d_tables);
  if (p->h_tables) (void)hipHostFree(p->h_tables);
  if (p->h_ids) (void)hipHostFree(p->h_ids);
  if (p->h_slot) (void)hipHostFree(p->h_slot);
  if (p->h_flag) (void)hipHostFree(p->h_flag);
  if (p->h_sel) (void)hipHostFree(p->h_sel);
  if (p->ev_ids) (void)hipEventDestroy(p->ev_ids);
  if (p->ev_copies) (void)hipEventDestroy(p->ev_copies);
  if (p->ev_slot) (void)hipEventDestroy(p->ev_slot);
  if (p->ev_table) (void)hipEventDestroy(p->ev_table);
  if (p->ev_btab) (void)hipEventDestroy(p->ev_btab);
  if (p->ev_batch) (void)hipEventDestroy(p->ev_batch);
  if (p->h_btab) (void)hipHostFree(p->h_btab);
  for (auto e : p->stg_ev)
    if (e) (void)hipEventDestroy(e);
  if (p->staging) (void)hipHostFree(p->staging);
  if (p->side) (void)hipStreamDestroy(p->side);
  delete p;
  return MOE_OK;
}

moe_status moe_pool_get_stats(const moe_pool *p, moe_pool_stats *st) {
  if (!p || !st) return MOE_E_INVALID;
  *st = p->stats;
  return MOE_OK;
}

moe_status moe_pool_reset_stats(moe_pool *p) {
  if (!p) return MOE_E_INVALID;
  p->stats = moe_pool_stats{};
  return MOE_OK;
}

}  // extern "C"
