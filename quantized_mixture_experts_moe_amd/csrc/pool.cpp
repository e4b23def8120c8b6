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

#include <string.h>

#include <algorithm>
#include <chrono>
#include <new>

namespace moe {

LfuPlanner::LfuPlanner(int slots, int E)
    : slots_(slots), count_(E, 0), last_(E, -1), slot_of_(E, -1), expert_in_(slots, -1) {}

bool LfuPlanner::access(const int *experts, int n, std::vector<Event> *events) {
  if (n > slots_) return false;
  for (int i = 0; i < n; ++i) {
    count_[experts[i]] += 1;
    last_[experts[i]] = now_;
  }
  for (int i = 0; i < n; ++i) {
    const int e = experts[i];
    if (slot_of_[e] >= 0) {
      if (events) events->push_back({e, slot_of_[e], 1, -1});
      continue;
    }
    int slot = -1, victim = -1;
    for (int s = 0; s < slots_; ++s) {
      if (expert_in_[s] < 0) {
        slot = s;
        break;
      }
    }
    if (slot < 0) {
      for (int s = 0; s < slots_; ++s) {
        const int v = expert_in_[s];
        bool needed = false;
        for (int j = 0; j < n; ++j) needed |= experts[j] == v;
        if (needed) continue;
        const bool older = lru_ ? last_[v] < last_[victim]
                                : count_[v] < count_[victim] ||
                                      (count_[v] == count_[victim] && last_[v] < last_[victim]);
        if (victim < 0 || older) {
          victim = v;
          slot = s;
        }
      }
      if (slot < 0) return false;
      slot_of_[victim] = -1;
    }
    expert_in_[slot] = e;
    slot_of_[e] = slot;
    if (events) events->push_back({e, slot, 0, victim});
  }
  ++now_;
  return true;
}

}  // namespace moe

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

moe_status pool_plan_and_copy(moe_pool *p, int layer, int T, int k, hipStream_t s,
                              const void *const **table, const void *const **slot_blob) {
  const moe_status ws = p->ids_mode ? wait_direct_ids(p, T, k)
                                      : (hipEventSynchronize(p->ev_ids) == hipSuccess ? MOE_OK
                                                                                       : MOE_E_HIP);
  if (ws) return ws;
  // distinct experts of the call in first-use order
  std::vector<int> need;
  need.reserve(T * k);
  for (int i = 0; i < T * k; ++i) {
    const int e = p->h_ids[i];
    if (e < 0 || e >= p->E) return MOE_E_POOL;
    if (std::find(need.begin(), need.end(), e) == need.end()) need.push_back(e);
  }
  std::vector<LfuPlanner::Event> ev;
  if (!p->planners[layer].access(need.data(), (int)need.size(), &ev)) return MOE_E_POOL;
  // counts: one lookup per (token, slot) use; the call's first use of a
  // missing expert is its miss, repeated uses inside the call are hits
  p->stats.lookups += (uint64_t)T * k;
  const void **tab = p->h_tables + (size_t)layer * p->E;
  uint8_t *base = p->slot_mem + (size_t)layer * p->slots * p->blob_bytes;
  int copies = 0;
  for (const auto &e : ev) {
    if (e.hit) continue;
    uint8_t *dst = base + (size_t)e.slot * p->blob_bytes;
    const void *src = p->host_blobs[(size_t)layer * p->E + e.expert];
    if (hipMemcpyAsync(dst, src, p->blob_bytes, hipMemcpyHostToDevice, p->side) != hipSuccess)
      return MOE_E_HIP;
    if (e.evicted >= 0) {
      tab[e.evicted] = base;  // not resident; never read for a call that does not select it
      p->stats.evictions += 1;
    }
    tab[e.expert] = dst;
    p->stats.misses += 1;
    p->stats.bytes_h2d += p->blob_bytes;
    ++copies;
  }
  p->stats.hits += (uint64_t)T * k - copies;
  bool queued = copies > 0;
  if (copies && table) {
    if (hipMemcpyAsync(p->d_tables + (size_t)layer * p->E, tab, sizeof(void *) * p->E,
                       hipMemcpyHostToDevice, p->side) != hipSuccess)
      return MOE_E_HIP;
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

moe_status moe_pool_create(moe_pool **out, int32_t n_layers, int32_t slots, int32_t E, int32_t D,
                           int32_t F, const void *const *host_blobs) {
  if (!out || n_layers < 1 || slots < 1 || E < 1 || slots > E || !host_blobs) return MOE_E_INVALID;
  if (D < 64 || F < 64 || D % 64 || F % 64) return MOE_E_INVALID;
  for (size_t i = 0; i < (size_t)n_layers * E; ++i)
    if (!host_blobs[i]) return MOE_E_INVALID;
  moe_pool *p = new (std::nothrow) moe_pool;
  if (!p) return MOE_E_POOL;
  p->n_layers = n_layers; p->slots = slots; p->E = E; p->D = D; p->F = F;
  p->blob_bytes = blob_layout(D, F).total;
  p->host_blobs.assign(host_blobs, host_blobs + (size_t)n_layers * E);
  for (int l = 0; l < n_layers; ++l) p->planners.emplace_back(slots, E);
  bool ok = hipMalloc((void **)&p->slot_mem, (size_t)n_layers * slots * p->blob_bytes) ==
            hipSuccess;
  ok = ok && hipMalloc((void **)&p->d_tables, sizeof(void *) * n_layers * E) == hipSuccess;
  ok = ok && hipHostMalloc((void **)&p->h_tables, sizeof(void *) * n_layers * E,
                           hipHostMallocDefault) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&p->side, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_ids, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_copies, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&p->ev_slot, hipEventDisableTiming) == hipSuccess;
  if (ok) {
    // every table entry starts at the layer's first slot (nothing resident yet)
    for (int l = 0; l < n_layers; ++l)
      for (int e = 0; e < E; ++e)
        p->h_tables[(size_t)l * E + e] = p->slot_mem + (size_t)l * slots * p->blob_bytes;
    ok = hipMemcpy(p->d_tables, p->h_tables, sizeof(void *) * n_layers * E,
                   hipMemcpyHostToDevice) == hipSuccess;
  }
  if (!ok) {
    moe_pool_destroy(p);
    return MOE_E_HIP;
  }
  *out = p;
  return MOE_OK;
}

moe_status moe_pool_destroy(moe_pool *p) {
  if (!p) return MOE_E_INVALID;
  if (p->side) (void)hipStreamSynchronize(p->side);
  if (p->slot_pending) (void)hipEventSynchronize(p->ev_slot);
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
