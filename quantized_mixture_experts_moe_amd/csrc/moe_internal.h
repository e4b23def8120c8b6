// Internal declarations of libmoe (HIP, gfx950).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kGroup = 64;      // columns per scale/bias pair (MLX affine group 64)
constexpr size_t kAlign = 256;  // section alignment inside a blob and the workspace
constexpr int kMaxE = 1024;     // router width handled by the top-k wave
constexpr int kPrefillRows = 32; // token rows per block of the grouped prefill kernels
constexpr int kMaxK = 64;       // experts per token
constexpr int kMaxKS = 16;      // split of a reduction over blocks
constexpr int kMaxSplitBlocks = 4096;  // blocks of a split launch (partial tiles)
constexpr int kMaxFusedKSd = 16;       // output splits of the one-launch expert phase
constexpr int kMaxDGroups = 128;       // model width / 64 handled by the prefill kernels
constexpr int kMaxHGroups = 64;        // hidden width / 64 handled by the prefill kernels
constexpr int kMaxLayerGrid = 4096;    // blocks of the one-launch decode layer
constexpr int kMaxLayerT = 4;          // tokens of the one-launch decode layer
constexpr int kMaxLayerE = 256;        // experts of the one-launch decode layer
constexpr int kMaxMidT = 8;            // tokens of the batched-decode expert phase
constexpr int kMaxMidKS = 16;          // its gate/up splits
constexpr int kMaxMidGB = 16;          // column groups of one of its gate/up blocks
constexpr int kMaxMidKSd = 64;         // its down splits
// Region at the start of every workspace that holds the tagged words of the
// one-launch decode layer: the per-block epochs, then 64-bit (value, tag)
// words only.  Its place and size do not depend on the call, so no other
// kernel ever writes into it.
constexpr size_t kLayerRegionBytes = size_t(8) << 20;
constexpr size_t kLayerEpochBytes = sizeof(uint32_t) * kMaxLayerGrid;
// Split-reduction accumulators and counters of the one-launch kernels, at
// fixed places in that region (after the epochs): they are zero between calls
// whatever the call's shape.  Gate/up tiles: 128 values each; output tiles:
// 64 values each; one 64-byte line per counter.
constexpr int kMaxAccTiles = 2048;
constexpr int kMaxOutTiles = 512;
constexpr size_t kAccGluOff = kLayerEpochBytes;
constexpr size_t kAccOutOff = kAccGluOff + sizeof(uint64_t) * 128 * kMaxAccTiles;
constexpr size_t kCntGluOff = kAccOutOff + sizeof(uint64_t) * 64 * kMaxOutTiles;
constexpr size_t kCntOutOff = kCntGluOff + 64 * (size_t)kMaxAccTiles;
constexpr size_t kTaggedOff = kCntOutOff + 64 * (size_t)kMaxOutTiles;
constexpr int kCntStride = 16;  // u32 words per counter line
// Sticky count of timed-out waits: the last line of the region, at the
// same place for every call (read by moe_workspace_timeouts).
constexpr size_t kErrOff = kLayerRegionBytes - kAlign;
// Epochs of the matrix-core router, one per 16-token tile, at a fixed place
// below that line: every call advances all of them in step, so the tagged
// partial logits of a call carry one epoch, above every older word's.
constexpr int kMaxRouteTiles = 4096;  // 65536 tokens
constexpr size_t kRouteEpochOff = kErrOff - sizeof(uint32_t) * kMaxRouteTiles;
static_assert(kRouteEpochOff % kAlign == 0, "aligned");
// and its tagged partial logits [kRouteParts][tokens][E], below them: a
// launch routes at most kRouteTagBytes / (8 kRouteParts E) tokens (longer
// calls are routed in windows of that many)
constexpr int kRouteParts = 4;
constexpr size_t kRouteTagBytes = size_t(4) << 20;
constexpr size_t kRouteTagOff = kRouteEpochOff - kRouteTagBytes;
// The row router's tagged logits [T][E] (calls of at most kRowTagTokens
// tokens) and its per-block epochs [kRowEpochs], below them; the one-launch
// layer's tagged words end below kRowTagOff.
constexpr int kRowTagTokens = 15;
constexpr int kRowEpochs = 4096;
constexpr size_t kRowEpochOff = kRouteTagOff - sizeof(uint32_t) * kRowEpochs;
constexpr size_t kRowTagOff = kRowEpochOff - sizeof(uint64_t) * kRowTagTokens * kMaxE;
static_assert(kRowTagOff % kAlign == 0, "aligned");

__host__ __device__ inline size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of the sections of one 4-bit GLU expert blob (D model width,
// F hidden width): gate.codes, up.codes, down.codes, gate.meta, up.meta,
// down.meta, each 256-byte aligned.
struct BlobLayout {
  size_t gate_codes, up_codes, down_codes, gate_meta, up_meta, down_meta, total;
};

__host__ __device__ inline BlobLayout blob_layout(int D, int F) {
  BlobLayout L;
  const size_t cb = (size_t)F * D / 2;        // 4-bit codes of [F, D] or [D, F]
  const size_t mb = (size_t)(D / kGroup) * F * 4;
  const size_t mbd = (size_t)(F / kGroup) * D * 4;
  size_t off = 0;
  L.gate_codes = off; off = align_up(off + cb);
  L.up_codes = off;   off = align_up(off + cb);
  L.down_codes = off; off = align_up(off + cb);
  L.gate_meta = off;  off = align_up(off + mb);
  L.up_meta = off;    off = align_up(off + mb);
  L.down_meta = off;  off = align_up(off + mbd);
  L.total = off;
  return L;
}

// Launch-shape knobs (moe_set_tuning).
struct Tuning {
  int glu_ks = 0;      // 0: chosen from the problem size
  int down_ks = 0;
  int fused = 1;       // one-launch expert phase for decode when it fits
  int fused_ksg = 0;   // its gate/up and down splits (0: chosen)
  int fused_ksd = 0;
  int prefill_min_t = 8;   // tokens per call from which the grouped matrix-core path runs
                           // (measured: equal at 8, 8 % faster at 12 than the few-token path)
  int route_mfma = 1;      // router of 16 or more tokens on the matrix cores
  int layer = 1;       // one launch for the whole decode layer when it fits (0: off)
  int layer_ksg = 0;   // its gate/up and down splits (0: chosen)
  int layer_ksd = 0;
  int layer_order = 1;
  int layer_select = 1;  // measured: 17.0 against 17.5 us per decode step
  int layer_log_copies = 16;
  int layer_sel_copies = 16;
  int layer_sel_stride = 0;  // words between selection lines; 0: packed
  int block_fused = 1;       // residual block: norms inside the one-launch decode layer
  int mid = 0;               // batched decode: each distinct expert read once for its tokens
                             // (measured slower than the per-token kernels: off)
  int mid_min_t = 2;         // from this many tokens per call
  int mid_max_t = 7;         // up to this many (and below prefill_min_t)
  int mid_ksg = 0;           // its gate/up and down splits (0: chosen)
  int mid_ksd = 0;
  int mid_kss = 0;           // its shared-expert gate/up split (0: chosen)
};
Tuning &tuning();

// Workspace carve-up for one call.  Every region is 256-byte aligned.
struct Workspace {
  uint8_t *layer;      // the fixed region of the one-launch decode layer
  uint32_t *xp;        // x as dot2 pairs [T][D/2]
  float *xs;           // x group sums [T][D/64]
  float *logits;       // [T][E]
  int32_t *ids;        // [T][k]
  const void **slot_blob;  // [T][k]
  float *gates;        // [T][k]
  float *h;            // GLU output, one float per hidden unit
  float *hs;           // h group sums, one float per 64 hidden units
  float *part;         // split-reduction partials
  uint32_t *counters;  // last-block-done counters (zero between calls)
  float *dpart;        // output-split partials of the one-launch expert phase
  uint32_t *fcounters; // its counters (zero between calls)
  uint32_t *err;       // sticky count of timed-out waits
  int32_t *perm_counts, *perm_offsets, *perm, *perm_inv, *perm_items, *perm_n_items;
  int2 *perm_info;               // per work-list item: its expert's (count, offset)
  const void **perm_iblob;       // per work-list item: its expert's blob
  uint16_t *hplanes;   // prefill: hidden activations as three bf16 planes
  float *hsum;         // prefill: 64-unit sums of the hidden activations
  float *y, *ys;       // prefill: routed outputs per pair, shared outputs per token
  uint64_t *mgacc;     // batched decode: gate/up split sums [units / 64][2][64]
  uint64_t *mdacc;     // batched decode: output split sums [T][D]
  size_t total;
};

struct Dims {
  int T, k, E, D, F, Fs;
};

Workspace carve_workspace(void *base, const Dims &d);
// Argument checks of moe_layer_forward (everything but the workspace); on
// success *d holds the call's sizes.
moe_status layer_forward_args(const void *x, int x_dtype, int T, const moe_qmat *router, int k,
                              const moe_bank *routed, const moe_bank *shared, moe_pool *pool,
                              int layer, const void *out, int out_dtype, Dims *d);
size_t workspace_bytes(const Dims &d);

// Host-side launchers (return hipError_t of the launch).
struct RouteLaunch {
  const void *x; int f16x; int T, D, E, k;
  const uint8_t *codes; const uint32_t *meta;
  const float *logit_bias;
  float *logits; int32_t *ids; float *gates;
  uint32_t *xp; float *xs; uint32_t *counters;
  const void *const *table;           // routed bank (for slot_blob) or null
  const void **slot_blob;             // [T][k] blob of each selected expert, or null
  // words cleared for the next kernel: zero[0, zero_words) and every
  // zero2_stride-th word of zero2, zero2_count of them
  uint32_t *zero; int zero_words;
  uint32_t *zero2; int zero2_count, zero2_stride;
  // 16 or more tokens (matrix-core router): tagged partial logits
  // [kRouteParts][T][E] and the epochs [kMaxRouteTiles], in the fixed
  // region (zero-filled once)
  uint64_t *rtag; uint32_t *rep;
  // at most kRowTagTokens tokens (row router): tagged logits [T][E] and the
  // per-block epochs [kRowEpochs] in the fixed region (zero-filled once);
  // null: the last block of a token group selects (counter)
  uint64_t *rowtag; uint32_t *rowep; uint32_t *err;
  // fewer than 16 tokens, streamed experts: the ids also go to pinned host
  // memory (device-readable addresses), then host_flag[t] = host_epoch per
  // token, so that the host reads them without a copy; null otherwise
  int32_t *host_ids; uint32_t *host_flag; uint32_t host_epoch;
};
hipError_t launch_route(const RouteLaunch &a, hipStream_t s);
// x pairs and 64-column sums for the expert kernels without routing
// Residual block around the layer (block_norm.hip): pre-norm RMSNorm of x
// into the layer's 16-bit input u, post-norm RMSNorm of the layer's fp32
// output y added to x.  D <= kBlockMaxD.
constexpr int kBlockMaxD = 8192;
struct BlockTail {
  size_t u_off, y_off, yt_off, cnt_off, total;
};
BlockTail block_tail(size_t layer_bytes, int T, int D);
hipError_t launch_block_pre(const void *x, int f16x, int T, int D, const float *w, float eps,
                            uint16_t *u, hipStream_t s);
hipError_t launch_block_post(const float *y, const void *x, int f16x, int T, int D,
                             const float *w, float eps, void *out, int out_dtype, hipStream_t s);

hipError_t launch_prep_x(const void *x, int f16x, int T, int D, uint32_t *xp, float *xs,
                         hipStream_t s);

struct ExpertLaunch {
  int f16x; int T, k, D, E;           // E: experts in the routed bank (ids range)
  const uint32_t *xp; const float *xs;
  const int32_t *ids;                 // [T][k] or null (expert 0)
  const void *const *slot_blob;       // [T][k] blob per slot (from the router) or null
  const float *gates;                 // [T][k] (combine mode)
  const void *const *rblobs; int F;   // routed bank
  const void *const *sblobs; int Fs;  // shared bank or null (Fs = 0)
  float *h; float *hs; float *part; uint32_t *counters;
  // outputs: y [T*k][D] (per-slot mode) or out [T][D] (combine mode)
  float *y; void *out; int out_dtype;
  int glu_first, glu_count;           // GLU block range: routed tiles first, then shared
  int glu_ks;                         // reduction split of the GLU (0: from glu_count)
};
// Batched-decode expert phase (expert_mid.hip): gate/up and down kernels in
// which every distinct selected expert, and the shared expert, is read once
// for all tokens that use it.  T <= kMaxMidT and T k <= 64; ids, gates, xp, xs
// from the router kernel; resident routed bank (rblobs).
struct MidLaunch {
  ExpertLaunch a;
  uint64_t *gacc, *dacc;    // fixed-point split sums, zero between calls:
                            // [units / 64][2][64] and [T][D] (workspace)
  uint32_t *err;
  uint32_t *gcnt, *dcnt;    // tile counters, zero between calls: [n_tiles], [D / 64]
  int KSg, KSs, KSd;        // gate/up splits of the routed and the shared tiles; down splits
  int n_tiles, n_blocks;    // gate/up tiles (routed, then shared) and blocks
};
void plan_mid(MidLaunch *m);
hipError_t launch_mid(const MidLaunch &m, hipStream_t s);
// One-launch expert phase (gate/up + down + combine) for a few tokens.
constexpr int kFlagCopies = 16;  // replicas of each slot-ready flag (one 128-byte line each)
struct FusedLaunch {
  ExpertLaunch a;           // needs slot_blob (resident experts)
  int KSg, KSd, n_gtiles;   // KSd = KSdr + KSds
  int KSdr, KSds;           // down splits of the routed / shared units
  int tile_begin, tile_end; // gate/up tiles of this launch (routed tiles, then shared)
  int do_down;              // this launch also runs the down projection and combine
  // slot counters and flags: zeroed by the router kernel launched just before
  uint32_t *slot_cnt, *slot_flag, *err;
  // split reductions: accumulators and counters that are zero between calls
  uint64_t *gacc, *dacc;
  uint32_t *gcnt, *dcnt;
};
int fused_grid(const FusedLaunch &f);
int fused_max_g(const FusedLaunch &f);
int fused_max_u(const FusedLaunch &f);
hipError_t fused_capacity(const FusedLaunch &f, int *cap);
hipError_t launch_fused(const FusedLaunch &f, hipStream_t s);

int pick_ks(int blocks, int reduce_len, int min_ks, int override_ks);
int glu_min_ks(int D);
int glu_blocks(const ExpertLaunch &a);
hipError_t launch_glu(const ExpertLaunch &a, hipStream_t s);
hipError_t launch_down(const ExpertLaunch &a, bool combine, hipStream_t s);
hipError_t launch_combine(const float *y, const float *gates, const float *ys, int T, int k,
                          int D, void *out, int out_dtype, hipStream_t s);
// Grouped (permuted) expert phase of a prefill chunk on the matrix cores.
struct PrefillLaunch {
  int f16x, T, k, E, D, F, Fs;
  const int32_t *counts, *offsets, *perm, *inv;
  const int32_t *items, *n_items;    // work list: expert | row chunk << 16, longest first
  const int2 *item_info;              // per item: its expert's (count, offset)
  const void *const *item_blob;       // per item: its expert's blob
  const float *gates;
  const void *const *rblobs, *const *sblobs;
  const uint32_t *xp; const float *xs;
  uint16_t *hp; size_t plane;         // h as three bf16 planes of `plane` elements
  float *hsum, *y, *ys;                // ys: sks partial sums of the shared expert, [sks][T][D]
  int sks;                            // splits of the shared down projection over its hidden groups
  void *out; int out_dtype;
  int max_items;                      // work-list entries the grids cover (set by the launcher)
  // a batch of a streamed call (null otherwise): expert -> blob in its slot,
  // null for the experts of other batches, whose items are skipped
  const void *const *batch_blob;
  int skip_combine;                   // gate/up and down only (the combine runs apart)
};
constexpr int kMaxSharedSplits = 4;
hipError_t launch_prefill_experts(const PrefillLaunch &p, hipStream_t s);
hipError_t launch_prefill_combine(const PrefillLaunch &p, hipStream_t s);

// The whole decode layer in one launch (router, top-k, experts, combine).
struct LayerLaunch {
  int f16x, T, k, E, D, F, Fs;
  const void *x;
  const uint8_t *rcodes; const uint32_t *rmeta; const float *logit_bias;
  const void *const *rblobs;          // routed bank [E]
  const void *const *sblobs;          // shared bank (expert 0) or null
  int KSg, n_gtiles;
  int KSdr, KSds;                     // down splits of the routed / shared units
  int NR;                             // router + routed blocks (the shared blocks follow)
  int blk0, grid_full;                // this launch covers blocks [blk0, blk0 + grid)
  int order;                          // dispatch order: 0 router, routed, shared; 1 router, shared, routed
  int select;                         // 0: router blocks rank and publish the selection; 1: routed blocks rank the logits
  int log_copies;                     // copies of the logits (select 1)
  // streamed experts (two launches): the blob of rank r of token t in the
  // pool's slots, given_blob[t][r]; null otherwise
  const void *const *given_blob;
  size_t table_off;                   // LDS byte offset of the blob table
  uint32_t *bep;                      // per-block epochs [kMaxLayerGrid]
  uint64_t *rlog;                     // [log_copies][T][E] tagged logits
  uint64_t *sel;                      // [T][sel_copies] lines of [2][lid] tagged ids, gates
  int sel_copies, lid, sel_stride;    // sel_stride: words from one line to the next
  uint64_t *hg, *hu;                  // [T*k*F + T*Fs] tagged gelu(gate) and up
  uint64_t *gacc, *dacc;              // split-reduction accumulators (zero between calls)
  uint32_t *gcnt, *dcnt;              // and their counters
  uint32_t *err;
  int32_t *ids_out; float *gates_out; // optional
  void *out; int out_dtype;
  // streamed experts in two launches of this kernel (router and shared
  // blocks, then the routed blocks): the router blocks also store each
  // selected expert as (id, host_epoch) into host_sel [T][k] (pinned host
  // memory); the routed blocks take the selection and gates from the
  // selection lines as usual and the blob of rank r from given_blob[t][r]
  uint64_t *host_sel; uint32_t host_epoch;
  int two;                            // that variant of the kernel (set before planning)
  int dw4;                            // every wave of a block takes down units (16 per block)
  // the residual block fused around the layer (w_pre non-null; one launch,
  // resident experts): x is the residual stream, normalised (w_pre) by every
  // role into the layer's input (also stored to u_out [T][D] if non-null);
  // each output element goes to ybuf [T][D] as a tagged word and is
  // counted in ocnt [T] (zero between calls); a router block per token
  // polls the count, then writes out = x + the post-norm (w_post) of the row
  const float *w_pre, *w_post;
  float eps;
  uint64_t *ybuf;
  uint32_t *ocnt;
  uint16_t *u_out;
};
int layer_m(const LayerLaunch &L);
int layer_routed_blocks(const LayerLaunch &L);
int layer_router_blocks(const LayerLaunch &L);
int layer_grid(const LayerLaunch &L);
size_t layer_smem(const LayerLaunch &L);
size_t layer_table_off(const LayerLaunch &L);
hipError_t layer_capacity(const LayerLaunch &L, int *cap);
int layer_shared_blocks(const LayerLaunch &L);
hipError_t launch_layer(const LayerLaunch &L, hipStream_t s);
// blocks [first, first + n) of the dispatch order L.order (0 or 1), two-launch variant
hipError_t launch_layer_ordered(LayerLaunch L, int first, int n, hipStream_t s);
// blocks [blk0, blk0 + n) of the grid only (streamed experts: shared blocks
// first, then the rest once the pool has the selected experts)
hipError_t launch_layer_range(LayerLaunch L, int blk0, int n, hipStream_t s);

// items (optional, [E * ceil(T k / chunk_rows)]): the grouped kernels' work
// list, expert | chunk << 16, experts by count (most first, ties by index);
// n_items: its length; info, iblob (optional, with blobs: the bank's blob
// table): each item's expert's (count, offset) and blob, so that a block
// reads everything about its item at once
hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *items,
                          int32_t *n_items, int chunk_rows, hipStream_t s, int2 *info = nullptr,
                          const void **iblob = nullptr, const void *const *blobs = nullptr);

}  // namespace moe
