// Host-side planning of the HBM expert slot pool: the replacement policy and
// the bookkeeping of one call's fetches, free of any HIP type so that it also
// builds and runs on a machine without a GPU (with a recording copy engine).
//
// The pages keep 16 expert slots per layer, plan each token's fetches on the
// CPU against a least-frequently-used cache and read the misses into the
// freed slots (stork.ai blog, "Mas inteligente que tu RAM"; es.news.hada.io,
// "Proceso de generacion de tokens").
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "moe.h"

namespace moe {

// Slot planner of one layer.  Least frequently used: use counts are per
// expert, cumulative, and kept after eviction; the victim is a resident
// expert the current call does not need with the smallest count, ties to the
// least recently used, then the lowest slot; empty slots fill in slot order.
// Least recently used (for comparison): the victim is the resident expert
// not needed now that was used longest ago, ties to the lowest slot.
class LfuPlanner {
 public:
  struct Event {
    int expert, slot, hit, evicted;
  };
  LfuPlanner(int slots, int E)
      : slots_(slots), count_(E, 0), last_(E, -1), slot_of_(E, -1), expert_in_(slots, -1) {}
  // 0: least frequently used (the pages' policy); 1: least recently used
  void set_policy(int policy) { lru_ = policy == 1; }
  // Serves the experts of one call (distinct, in first-use order).  Returns
  // false, and changes nothing, if they do not fit the slots.
  bool access(const int *experts, int n, std::vector<Event> *events) {
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
          if (victim < 0 || older(v, victim)) {
            victim = v;
            slot = s;
          }
        }
        // n <= slots, so some resident expert is not needed
        slot_of_[victim] = -1;
      }
      expert_in_[slot] = e;
      slot_of_[e] = slot;
      if (events) events->push_back({e, slot, 0, victim});
    }
    ++now_;
    return true;
  }
  // Forgets whatever slot s holds (its bytes can no longer be trusted): the
  // next call that needs that expert fetches it again.
  void invalidate_slot(int s) {
    if (s < 0 || s >= slots_) return;
    const int e = expert_in_[s];
    if (e >= 0) slot_of_[e] = -1;
    expert_in_[s] = -1;
  }
  int slot_of(int e) const { return slot_of_[e]; }
  int expert_in(int s) const { return expert_in_[s]; }
  int slots() const { return slots_; }

 private:
  // is resident expert v a better victim than resident expert w?
  bool older(int v, int w) const {
    if (lru_) return last_[v] < last_[w];
    return count_[v] < count_[w] || (count_[v] == count_[w] && last_[v] < last_[w]);
  }
  int slots_;
  bool lru_ = false;
  long now_ = 0;
  std::vector<long> count_, last_;
  std::vector<int> slot_of_, expert_in_;
};

// Where the bytes of one miss go.  Returns 0 once the copy is enqueued
// (or done), nonzero if it could not be; after a failure the destination may
// hold any bytes.
// copy() may also only record the copy and flush() carry out all of the
// call's copies at once (0: all enqueued; nonzero: the slots of every copy
// recorded since the last flush may hold any bytes).
struct CopyEngine {
  virtual ~CopyEngine() = default;
  virtual int copy(int expert, int slot, void *dst, const void *src, size_t bytes) = 0;
  virtual int flush() { return 0; }
};

// Test hook: passes `pass` copies through to `inner`, then fails the next one
// (without calling `inner`), then passes everything again.
struct FailingCopyEngine final : CopyEngine {
  CopyEngine *inner;
  int left;  // copies still to pass before the failure; -1: already failed
  FailingCopyEngine(CopyEngine *e, int pass) : inner(e), left(pass) {}
  int copy(int expert, int slot, void *dst, const void *src, size_t bytes) override {
    if (left == 0) {
      left = -1;
      return 1;
    }
    if (left > 0) --left;
    return inner->copy(expert, slot, dst, src, bytes);
  }
  int flush() override { return inner->flush(); }
  int remaining() const { return left; }
};

// One call's plan for one layer.
struct LayerPlanArgs {
  const int32_t *ids;                 // host [n] expert ids of the call, in (token, slot) order
  int n, E;
  uint8_t *slot_base;                 // device address of the layer's first slot
  size_t blob_bytes;
  const void *const *host_blobs;      // [E] the layer's blobs in host memory (null: the
                                      // copy engine finds them itself)
  const void **table;                 // [E] host table: expert -> blob address (slot or placeholder)
};

struct PlanResult {
  int copies = 0;
  moe_status status = MOE_OK;
};

// Plans the call's experts on a copy of the planner, enqueues every miss's
// copy into its slot, and only then commits: the planner, the table and the
// stats change together, so a failed copy never leaves an expert marked
// resident in a slot that was not filled.  On a failed copy the slots that
// this call may have written are invalidated (their old experts are no longer
// resident, and the call's new experts are not either), so the next call that
// needs any of them fetches it again.  A call whose distinct experts do not
// fit the slots, or with an id outside [0, E), changes nothing and returns
// MOE_E_POOL.
// After a failed copy: the slots of the first n events' misses may hold any
// bytes; their old experts are no longer resident (and nothing new is).
inline void invalidate_misses(LfuPlanner &planner, const LayerPlanArgs &a,
                              const std::vector<LfuPlanner::Event> &ev, size_t n) {
  for (size_t j = 0; j < n; ++j) {
    if (ev[j].hit) continue;
    const int old = planner.expert_in(ev[j].slot);
    if (old >= 0) a.table[old] = a.slot_base;
    planner.invalidate_slot(ev[j].slot);
  }
}

inline PlanResult plan_layer_call(LfuPlanner &planner, const LayerPlanArgs &a, CopyEngine &eng,
                                  moe_pool_stats *stats) {
  PlanResult r;
  std::vector<int> need;
  need.reserve(a.n);
  for (int i = 0; i < a.n; ++i) {
    const int e = a.ids[i];
    if (e < 0 || e >= a.E) {
      r.status = MOE_E_POOL;
      return r;
    }
    if (std::find(need.begin(), need.end(), e) == need.end()) need.push_back(e);
  }
  LfuPlanner trial = planner;
  std::vector<LfuPlanner::Event> ev;
  if (!trial.access(need.data(), (int)need.size(), &ev)) {
    r.status = MOE_E_POOL;
    return r;
  }
  for (size_t i = 0; i < ev.size(); ++i) {
    if (ev[i].hit) continue;
    uint8_t *dst = a.slot_base + (size_t)ev[i].slot * a.blob_bytes;
    const void *src = a.host_blobs ? a.host_blobs[ev[i].expert] : nullptr;
    if (eng.copy(ev[i].expert, ev[i].slot, dst, src, a.blob_bytes) != 0) {
      // slots of this and the earlier misses may hold new or partial bytes
      invalidate_misses(planner, a, ev, i + 1);
      r.status = MOE_E_HIP;
      return r;
    }
    ++r.copies;
  }
  if (eng.flush() != 0) {
    invalidate_misses(planner, a, ev, ev.size());
    r.status = MOE_E_HIP;
    r.copies = 0;
    return r;
  }
  planner = trial;
  for (const auto &e : ev) {
    if (e.hit) continue;
    if (e.evicted >= 0) {
      a.table[e.evicted] = a.slot_base;  // placeholder: never read for a call that does not select it
      if (stats) stats->evictions += 1;
    }
    a.table[e.expert] = a.slot_base + (size_t)e.slot * a.blob_bytes;
  }
  if (stats) {
    // one lookup per (token, slot) use; the call's first use of a missing
    // expert is its miss, repeated uses inside the call are hits
    stats->lookups += (uint64_t)a.n;
    stats->misses += (uint64_t)r.copies;
    stats->hits += (uint64_t)a.n - (uint64_t)r.copies;
    stats->bytes_h2d += (uint64_t)r.copies * a.blob_bytes;
  }
  return r;
}

}  // namespace moe
