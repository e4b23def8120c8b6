// CPU driver of the pool's host-side planning (csrc/pool_plan.h) with a
// recording copy engine: no GPU, built with the address and undefined-
// behaviour sanitizers by the tests.
//
// Reads commands from stdin, one per line:
//   pool <slots> <E> <policy>      start a pool of one layer (policy 0 LFU, 1 LRU)
//   fail <n>                       let n copies through, then fail the next one
//   call <id> <id> ...             one call's (token, slot) expert ids
// and prints, per call:
//   call status=<s> copies=<n> [copy <expert> <slot>]... resident=<e0,e1,...> table_ok=<0|1>
//       stats=<lookups,hits,misses,evictions,bytes>
// where resident lists the expert in each slot (-1 empty) and table_ok
// checks that the host table points every resident expert at its slot.
#include <stdio.h>
#include <stdlib.h>

#include <iostream>
#include <memory>
#include <sstream>
#include <string>
#include <vector>

#include "pool_plan.h"

namespace {

constexpr size_t kBlob = 4096;

struct RecordingEngine final : moe::CopyEngine {
  uint8_t *slot_base = nullptr;
  const std::vector<std::vector<uint8_t>> *host = nullptr;
  std::vector<std::pair<int, int>> log;  // (expert, slot) of each copy
  int copy(int, int, void *dst, const void *src, size_t bytes) override {
    const size_t off = (uint8_t *)dst - slot_base;
    if (off % kBlob != 0 || bytes != kBlob) {
      fprintf(stderr, "bad copy: offset %zu bytes %zu\n", off, bytes);
      exit(2);
    }
    int expert = -1;
    for (size_t e = 0; e < host->size(); ++e)
      if ((*host)[e].data() == src) expert = (int)e;
    if (expert < 0) {
      fprintf(stderr, "copy from an unknown source\n");
      exit(2);
    }
    // the "device": slot memory is plain host memory here
    std::copy((const uint8_t *)src, (const uint8_t *)src + bytes, (uint8_t *)dst);
    log.emplace_back(expert, (int)(off / kBlob));
    return 0;
  }
};

}  // namespace

int main() {
  std::unique_ptr<moe::LfuPlanner> planner;
  std::vector<std::vector<uint8_t>> host;
  std::vector<const void *> host_ptr;
  std::vector<uint8_t> slots_mem;
  std::vector<const void *> table;
  moe_pool_stats stats{};
  int fail_at = -1, slots = 0, E = 0;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "pool") {
      int policy = 0;
      in >> slots >> E >> policy;
      planner.reset(new moe::LfuPlanner(slots, E));
      planner->set_policy(policy);
      host.assign(E, std::vector<uint8_t>(kBlob));
      host_ptr.clear();
      for (int e = 0; e < E; ++e) {
        for (size_t i = 0; i < kBlob; ++i) host[e][i] = (uint8_t)(e * 31 + i);
        host_ptr.push_back(host[e].data());
      }
      slots_mem.assign((size_t)slots * kBlob, 0xEE);
      table.assign(E, slots_mem.data());
      stats = moe_pool_stats{};
      fail_at = -1;
    } else if (cmd == "fail") {
      in >> fail_at;
    } else if (cmd == "call") {
      std::vector<int32_t> ids;
      int v;
      while (in >> v) ids.push_back(v);
      RecordingEngine rec;
      rec.slot_base = slots_mem.data();
      rec.host = &host;
      moe::FailingCopyEngine fail(&rec, fail_at);
      moe::CopyEngine *eng = fail_at >= 0 ? (moe::CopyEngine *)&fail : &rec;
      moe::LayerPlanArgs a;
      a.ids = ids.data();
      a.n = (int)ids.size();
      a.E = E;
      a.slot_base = slots_mem.data();
      a.blob_bytes = kBlob;
      a.host_blobs = host_ptr.data();
      a.table = table.data();
      const moe::PlanResult r = moe::plan_layer_call(*planner, a, *eng, &stats);
      if (fail_at >= 0) fail_at = fail.remaining();
      printf("call status=%d copies=%d", r.status, r.copies);
      for (auto &c : rec.log) printf(" copy %d %d", c.first, c.second);
      printf(" resident=");
      bool table_ok = true;
      for (int s = 0; s < slots; ++s) {
        const int e = planner->expert_in(s);
        printf(s ? ",%d" : "%d", e);
        if (e >= 0) {
          // the table points at the slot, and the slot holds that expert's bytes
          table_ok = table_ok && table[e] == slots_mem.data() + (size_t)s * kBlob;
          table_ok = table_ok && std::equal(host[e].begin(), host[e].end(),
                                            slots_mem.begin() + (size_t)s * kBlob);
          table_ok = table_ok && planner->slot_of(e) == s;
        }
      }
      printf(" table_ok=%d stats=%llu,%llu,%llu,%llu,%llu\n", table_ok ? 1 : 0,
             (unsigned long long)stats.lookups, (unsigned long long)stats.hits,
             (unsigned long long)stats.misses, (unsigned long long)stats.evictions,
             (unsigned long long)stats.bytes_h2d);
    } else {
      fprintf(stderr, "unknown command %s\n", cmd.c_str());
      return 2;
    }
  }
  return 0;
}
