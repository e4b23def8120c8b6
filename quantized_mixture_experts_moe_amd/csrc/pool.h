// HBM expert slot pool (internal interface used by moe_layer_forward).
#pragma once

#include <vector>

#include "moe_internal.h"

namespace moe {

// Least-frequently-used slot planner of one layer.  Use counts are per
// expert, cumulative, and kept after eviction; the victim is a resident
// expert the current call does not need with the smallest count, ties to the
// least recently used, then the lowest slot; empty slots fill in slot order.
class LfuPlanner {
 public:
  struct Event {
    int expert, slot, hit, evicted;
  };
  LfuPlanner(int slots, int E);
  // 0: least frequently used (the pages' policy); 1: least recently used
  // (victim: the resident expert not needed now that was used longest ago,
  // ties to the lowest slot), for comparison
  void set_policy(int policy) { lru_ = policy == 1; }
  // Serve the experts of one call (distinct, in first-use order).  Returns
  // false if they do not fit the slots.
  bool access(const int *experts, int n, std::vector<Event> *events);
  int slot_of(int e) const { return slot_of_[e]; }

 private:
  int slots_;
  bool lru_ = false;
  long now_ = 0;
  std::vector<long> count_, last_;
  std::vector<int> slot_of_, expert_in_;
};

moe_status pool_check(const moe_pool *p, int layer, int E, int D, int k);
int pool_F(const moe_pool *p);
int pool_slots(const moe_pool *p);
// Before the router kernel: with fewer than 16 tokens, where it writes the
// ids in host memory and the epoch of this call's flags (null otherwise).
moe_status pool_route_ids(moe_pool *p, int T, int k, int32_t **host_ids, uint32_t **host_flag,
                          uint32_t *epoch);
// Before the first of two launches of the one-launch decode layer (router
// and shared blocks): where its router blocks store the (id, epoch) words
// of the selection, and this call's epoch.
moe_status pool_layer_sel(moe_pool *p, int T, int k, uint64_t **host_sel, uint32_t *epoch);
// After it: the ids back to the host (a copy, unless the kernel writes them).
moe_status pool_fetch_ids(moe_pool *p, const int32_t *d_ids, int n, hipStream_t s);
// Plans the call's experts, copies the misses into HBM slots on the side
// stream and makes stream s wait for them.  Publishes the layer's device
// pointer table (*table, if non-null) and, if slot_blob is non-null, a
// device-readable array (pinned host memory) with the slot address of every
// (token, slot) pair; the caller reports the kernels that read it with
// pool_slots_read once they are enqueued.
moe_status pool_plan_and_copy(moe_pool *p, int layer, int T, int k, hipStream_t s,
                              const void *const **table, const void *const **slot_blob);
moe_status pool_slots_read(moe_pool *p, hipStream_t s);

}  // namespace moe
