// HBM expert slot pool (internal interface used by moe_layer_forward).
#pragma once

#include <vector>

#include "moe_internal.h"
#include "pool_plan.h"

namespace moe {

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
// Calls with more distinct experts than slots run in batches of at most
// `slots` experts.  pool_batches waits for the call's ids and splits its
// distinct experts, in first-use order, into batches.  pool_plan_batch plans
// batch b against the slots and copies its misses (the side stream first
// waits for the previous batch's kernels, recorded by pool_batch_done, since
// this batch may evict their experts), makes stream s wait for the copies and
// publishes a device-readable table *btab [E]: the slot of each expert of the
// batch, null for every other expert.  pool_batches_read: after the last
// kernel that reads the tables.
moe_status pool_batches(moe_pool *p, int T, int k, std::vector<std::vector<int>> *batches);
moe_status pool_plan_batch(moe_pool *p, int layer, int b, const std::vector<int> &experts, int T,
                           int k, hipStream_t s, const void *const **btab);
moe_status pool_batch_done(moe_pool *p, hipStream_t s);
moe_status pool_batches_read(moe_pool *p, hipStream_t s);
// The layer's device table (expert -> slot address or a placeholder).
const void *const *pool_table(const moe_pool *p, int layer);

}  // namespace moe
