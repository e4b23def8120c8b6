/*
 * moe.h -- C ABI of libmoe: the routed int4 Mixture-of-Experts FFN layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the one the pages walk through per transformer layer and
 * token (es.news.hada.io, "Proceso de generacion de tokens"; yodev.dev,
 * "Por que funciona: el A4B del nombre"; imasters.com.br, "O truque"):
 * an 8-bit router scores the experts from resident weights, the top 8 of 128
 * are selected, the selected 4-bit experts (MLX affine, group 64) run as GLU
 * blocks, and their gate-weighted outputs are combined with a resident shared
 * expert.  Prefill works on chunks of up to 128 tokens so that an expert
 * fetched once serves several rows (es.news.hada.io, same section).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers marked "device" are HBM addresses (hipMalloc / torch tensors);
 * "host" pointers are ordinary process memory.  The caller owns every buffer
 * passed in; the library keeps no pointer past the call except inside a pool
 * (moe_pool_create).  Calls are asynchronous on `stream` (a hipStream_t; NULL
 * is the default stream) unless stated otherwise.  Arguments are validated
 * before anything is launched: a negative status means nothing was enqueued,
 * except for a moe_layer_forward with a pool, which plans its slots after
 * routing: there MOE_E_POOL (an expert id outside the pool's range) or
 * MOE_E_HIP can come after work was enqueued, and the call's outputs are
 * undefined.  MOE_E_HIP reports a HIP runtime error from a launch or copy;
 * after one, zero-fill the workspace again before reusing it.  Device faults
 * surface at the caller's next synchronisation.  No call aborts and no C++
 * exception crosses this boundary.  Results are bitwise reproducible: every
 * reduction has a fixed order and no floating-point atomics are used (where
 * blocks add partial sums they add fixed-point integers, whose sum does not
 * depend on the order of arrival).
 *
 * Quantised matrix storage (W[rows, cols], w = scale * q + bias per 64
 * consecutive columns of a row; codes unsigned, bits in {4, 8}):
 *   codes: 16-byte chunks of 128/bits consecutive columns of one row; chunk
 *          (r, cc) at byte (cc * rows + r) * 16; the code of the j-th column
 *          of a chunk at bits [bits*j, bits*j+bits) of the little-endian chunk.
 *   meta:  u32 [cols/64][rows]; bits 0-15 fp16 scale, bits 16-31 fp16 bias.
 * Expert blob (4-bit GLU expert, model width D, hidden width F): sections
 *   gate.codes [F,D] | up.codes [F,D] | down.codes [D,F] | gate.meta |
 *   up.meta | down.meta, each 256-byte aligned; moe_blob_bytes gives the size
 *   (3,345,408 bytes at D = 2816, F = 704: the pages' "3.36 MB" per expert,
 *   hndistilled.com, "Enfoque tecnico").
 * Expert FFN: y = (gelu_tanh(x Wg^T) * (x Wu^T)) Wd^T, fp32 accumulation.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_E_INVALID (-1)     /* bad argument: null pointer, shape, dtype, k   */
#define MOE_E_UNSUPPORTED (-2) /* valid but not implemented (e.g. bits = 2)     */
#define MOE_E_HIP (-3)         /* a HIP runtime call failed                     */
#define MOE_E_WORKSPACE (-4)   /* ws_bytes smaller than moe_workspace_bytes()   */
#define MOE_E_POOL (-5)        /* expert pool misuse or copy failure            */

#define MOE_F16 1
#define MOE_BF16 2
#define MOE_F32 3

/* One affine-quantised matrix (layout above).  Router: rows = E, cols = D,
 * bits = 8 (es.news.hada.io, "Estructura de ejecucion...": 8-bit router). */
typedef struct moe_qmat {
  const void *codes; /* device, rows*cols*bits/8 bytes, 16-byte aligned */
  const void *meta;  /* device, (cols/64)*rows u32 words */
  int32_t rows, cols, bits;
} moe_qmat;

/* A bank of E GLU experts of shape (D, F), one blob per expert. */
typedef struct moe_bank {
  const void *const *blobs; /* DEVICE array [E] of device blob pointers (256-B aligned) */
  int32_t E, D, F;
} moe_bank;

typedef struct moe_pool moe_pool;

typedef struct moe_pool_stats {
  uint64_t lookups;     /* expert uses served (tokens * k)          */
  uint64_t hits;        /* uses already resident in an HBM slot     */
  uint64_t misses;      /* uses copied host -> HBM                  */
  uint64_t evictions;   /* resident experts replaced                */
  uint64_t bytes_h2d;   /* bytes copied host -> HBM                 */
} moe_pool_stats;

/* Size of one expert blob in bytes. */
size_t moe_blob_bytes(int32_t D, int32_t F);

/* Scratch bytes `ws` must hold for calls with these sizes (F_shared = 0: no
 * shared expert).  The same workspace serves moe_route, moe_expert_ffn and
 * moe_layer_forward at or below these sizes.  It must be zero-filled before
 * its first use; every call leaves its synchronisation counters at zero and
 * its hand-off words tagged with a call counter, so one workspace serves calls
 * of any shape in any order.  Two calls that overlap in time must not share a
 * workspace. */
size_t moe_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t D, int32_t F,
                           int32_t F_shared);

/* Number of device-side errors in calls on `ws` since it was last
 * zero-filled: bounded waits that timed out, and partial sums outside the
 * range of the fixed-point split reductions.  The one-launch kernels hand
 * data between blocks that must all be resident; a wait that gives up (after
 * about a second) counts here and lets the kernel finish with undefined
 * results instead of hanging.  The split reductions add partials as 64-bit
 * fixed-point integers (sums below 2^27 in magnitude in the decode layer
 * kernel, 2^31 in the expert phase); a partial that could take a sum out of
 * that range, or is not finite, counts here too.  A nonzero count means the
 * outputs of those calls are undefined and the workspace must be zero-filled
 * again before further use.
 *   ws      device workspace (as passed to the other calls), ws_bytes its size
 *   count   host; receives the count
 * Blocks the host: the word is copied after the work queued on `stream`. */
moe_status moe_workspace_timeouts(const void *ws, size_t ws_bytes, uint32_t *count,
                                  void *stream);

/* Router and selection (es.news.hada.io, "Proceso de generacion de tokens":
 * top-8 expert IDs per layer; stork.ai blog, "Por que la mayor parte...":
 * 8 of 128 experts).  logits[t,e] = x[t] . Wr[e] + logit_bias[e] (fp32);
 * ids[t, 0..k) are the k largest logits, largest first, equal logits to the
 * lower index; gates[t, :] = softmax of the selected logits.
 *   x         device [T, D] fp16 or bf16 (x_dtype MOE_F16 / MOE_BF16), 16-byte
 *             aligned (every call that takes x requires this)
 *   router    8-bit matrix [E, D], D % 64 == 0, 1 <= E <= 1024
 *   logit_bias device [E] fp32 or NULL;  1 <= k <= min(E, 64)
 *   ids       device [T, k] int32;  gates device [T, k] fp32
 *   logits    device [T, E] fp32 or NULL
 *   ws        device scratch of moe_workspace_bytes(T, k, E, D, 64, 0) bytes */
moe_status moe_route(const void *x, int32_t x_dtype, int32_t T, const moe_qmat *router,
                     const float *logit_bias, int32_t k, int32_t *ids, float *gates,
                     float *logits, void *ws, size_t ws_bytes, void *stream);

/* Expert FFN of every (token, slot) pair: y[t, j, :] = FFN_{ids[t,j]}(x[t]),
 * the selected experts' FFNs of the pages (es.news.hada.io, "Proceso de
 * generacion de tokens"), stored as MLX-style 4-bit affine weights in groups
 * of 64 (es.news.hada.io, "Estructura de ejecucion para reducir memoria"):
 * gate and up dequantised and applied to x, gelu_tanh(gate) * up, then down.
 *   bank      experts of shape (D, F); D, F multiples of 64
 *   ids       device [T, k] int32 in [0, E), or NULL: every row uses expert 0
 *             and k must be 1 (the shared expert)
 *   y         device [T, k, D] fp32
 *   ws        device scratch of moe_workspace_bytes(T, k, E, D, F, 0) bytes */
moe_status moe_expert_ffn(const void *x, int32_t x_dtype, int32_t T, const moe_bank *bank,
                          const int32_t *ids, int32_t k, float *y, void *ws, size_t ws_bytes,
                          void *stream);

/* Combine (es.news.hada.io, "Proceso de generacion de tokens": the shared and
 * routed outputs are combined): out[t] = y_shared[t] + sum_j gates[t,j] y[t,j],
 * summed in j order in double precision and rounded once (to fp32, then to
 * out_dtype).  y device [T,k,D] fp32; gates device [T,k] fp32;
 * y_shared device [T,D] fp32 or NULL; out device [T,D] of out_dtype
 * (MOE_F32, MOE_BF16 or MOE_F16, round to nearest even). */
moe_status moe_combine(const float *y, const float *gates, const float *y_shared, int32_t T,
                       int32_t k, int32_t D, void *out, int32_t out_dtype, void *stream);

/* Token -> expert permutation of a prefill chunk (chunks of up to 128 tokens
 * let one fetched expert serve several rows: es.news.hada.io, "Proceso de
 * generacion de tokens").  counts[e] = pairs routed to e; offsets = exclusive
 * prefix sum (E + 1 entries); perm[p] = flat index t*k + j of the p-th pair in
 * (expert, flat index) order; inv[t*k + j] = its position.  All device int32;
 * T * k <= 65536. */
moe_status moe_permute(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv, void *stream);

/* The whole layer: route, run the selected experts and the shared expert,
 * combine.  out device [T, D] (out_dtype); ids_out / gates_out device [T, k]
 * or NULL.  shared may be NULL (no shared expert) or a bank with E = 1.
 * pool == NULL: `routed` holds all E experts resident in HBM.  pool != NULL:
 * `routed` may be NULL; the experts of layer `layer` are served from the
 * pool's HBM slots, missing ones copied from pinned host memory on the
 * pool's side stream while the shared expert runs; this call then blocks the
 * host once, until the selected ids have arrived in the pool's pinned host
 * memory (written there by the routing kernels; the pages' CPU fetch plan:
 * es.news.hada.io, "Proceso de generacion de tokens").  A pooled call with
 * more (token, slot) pairs than the pool has slots (a prefill chunk, a
 * batch of tokens) runs its distinct experts in batches of at most `slots`,
 * in first-use order: each batch's misses are fetched (after the previous
 * batch's kernels, whose slots it may reuse) and the grouped kernels run
 * that batch's experts; the shared expert runs with the first batch and the
 * combine after the last, so one expert fetched once serves all of the
 * call's rows that chose it (es.news.hada.io, same section).  The output is
 * bitwise the resident grouped path's.  Consecutive calls with one pool go
 * on one stream (the pool's host-side buffers are reused once the previous
 * call's kernels are done, which it checks). */
moe_status moe_layer_forward(const void *x, int32_t x_dtype, int32_t T, const moe_qmat *router,
                             const float *logit_bias, int32_t k, const moe_bank *routed,
                             const moe_bank *shared, moe_pool *pool, int32_t layer, void *out,
                             int32_t out_dtype, int32_t *ids_out, float *gates_out, void *ws,
                             size_t ws_bytes, void *stream);

/* The residual block around the layer (the pages list the normalisation and
 * residual work of a block among what a production engine fuses around the
 * experts, without defining it: es.news.hada.io, "Alcance de implementacion y
 * registro experimental"; the reading taken is a Gemma-style RMSNorm on both
 * sides of the layer):
 *   u   = x / sqrt(mean_d(x^2) + eps) * (1 + w_pre), rounded to x_dtype
 *         (round to nearest even): the layer's input
 *   y   = moe_layer_forward(u) in fp32
 *   out = x + y / sqrt(mean_d(y^2) + eps) * (1 + w_post), in out_dtype
 * Arguments as moe_layer_forward, and:
 *   w_pre, w_post  device [D] fp32, 16-byte aligned;  eps >= 0;  D <= 8192
 *   out       device [T, D], 16-byte aligned; may be x itself when
 *             out_dtype == x_dtype (the residual stream updated in place); no
 *             other overlap with x
 *   u_out     device [T, D] of x_dtype, 16-byte aligned, or NULL: receives u
 *   ws        device scratch of moe_block_workspace_bytes(T, k, E, D, F,
 *             F_shared) bytes, zero-filled before its first use (the
 *             layer's workspace, then u, y and per-token counters)
 * Errors: MOE_E_INVALID for a bad argument or overlap, MOE_E_WORKSPACE for a
 * short workspace, else as moe_layer_forward. */
moe_status moe_block_forward(const void *x, int32_t x_dtype, int32_t T, const float *w_pre,
                             const float *w_post, float eps, const moe_qmat *router,
                             const float *logit_bias, int32_t k, const moe_bank *routed,
                             const moe_bank *shared, moe_pool *pool, int32_t layer, void *out,
                             int32_t out_dtype, void *u_out, int32_t *ids_out, float *gates_out,
                             void *ws, size_t ws_bytes, void *stream);
size_t moe_block_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t D, int32_t F,
                                 int32_t F_shared);

/* Expert store: every layer's expert blobs in one file on local storage,
 * blob (layer l, expert e) at byte offset (l * E + e) * moe_store_stride(D, F)
 * (the blob's size rounded up to 4096 bytes, zero padded), read on demand
 * with bounded-parallel pread rather than mmap: the pages' SSD tier
 * (hndistilled.com, "Enfoque tecnico (MoE + transmision desde SSD)";
 * yodev.dev, "Por que pread y no mmap"). */
typedef struct moe_store moe_store;

typedef struct moe_store_stats {
  uint64_t blobs;      /* expert blobs read                                  */
  uint64_t bytes;      /* blob bytes read (without the padding)              */
  uint64_t ns;         /* wall time spent in reads                           */
  uint64_t errors;     /* reads that failed                                  */
  uint64_t last_errno; /* errno of the last failure (0: none)                */
  uint64_t bounced;    /* 1: direct reads go through bounce buffers (the
                          destinations refused direct I/O)                   */
} moe_store_stats;

#define MOE_STORE_DIRECT 1 /* O_DIRECT: bypass the page cache (buffered if refused) */
#define MOE_STORE_MMAP 2   /* for comparison: map the file and copy out of it      */

size_t moe_store_stride(int32_t D, int32_t F);

/* Opens the file at `path` (host path) holding n_layers * E blobs of shape
 * (D, F).  flags: 0 (buffered pread), MOE_STORE_DIRECT or MOE_STORE_MMAP.
 * threads (1..64): reads in flight at once (the queue depth).  The store owns
 * its file descriptor and reader threads.  MOE_E_INVALID for bad arguments,
 * a missing file or one shorter than the blobs need. */
moe_status moe_store_open(moe_store **store, const char *path, int32_t n_layers, int32_t E,
                          int32_t D, int32_t F, int32_t flags, int32_t threads);

/* Reads blobs (layer, experts[i]), i < n, into host buffers dst[i] (HOST array
 * of n pointers; each buffer at least moe_store_stride bytes and, with direct
 * I/O, 4096-byte aligned: page-locked memory from hipHostMalloc is), split
 * into pieces of chunk_bytes (rounded up to 4096; 0: whole blobs) that the
 * reader threads fetch in parallel.  Blocks until done.  MOE_E_POOL if a read
 * fails. */
moe_status moe_store_read(moe_store *store, int32_t layer, const int32_t *experts, int32_t n,
                          void *const *dst, size_t chunk_bytes);
moe_status moe_store_get_stats(const moe_store *store, moe_store_stats *stats);
moe_status moe_store_close(moe_store *store);

/* HBM expert slot pool whose misses come from a store instead of pinned host
 * blobs: a call's missing experts are read by the store's threads into the
 * pool's page-locked staging buffers (one per slot) and copied into the HBM
 * slots on the side stream, while the shared expert runs.  Everything else
 * as moe_pool_create (layers and shapes from the store; the store must
 * outlive the pool).  chunk_bytes as in moe_store_read. */
moe_status moe_pool_create_store(moe_pool **pool, int32_t slots, moe_store *store,
                                 size_t chunk_bytes);

/* moe_layer_forward with every expert resident (no pool), for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The caller passes inputs
 * and outputs as for moe_layer_forward; the workspace is a fixed 48 MiB
 * device array inside the library (one per GPU, held until the process
 * ends), so nothing is allocated, by the library or by the caller.
 *   Calls whose moe_workspace_bytes(T, k, E, D, F, F_shared) exceeds 48 MiB
 *   return MOE_E_WORKSPACE and enqueue nothing (the Gemma-4-26B-A4B-shaped
 *   layer fits up to 128 tokens per call: 40.1 MiB).
 *   The first call on a device enqueues a zero-fill of the array on `stream`
 *   before its own kernels; every call leaves the array ready for the next.
 *   All calls on one GPU share the array: calls that overlap in time on one
 *   GPU (different streams or host threads without ordering) race and their
 *   outputs are undefined.  Errors as for moe_layer_forward; after MOE_E_HIP
 *   the next call on the device clears the array again. */
moe_status moe_layer_forward_noalloc(const void *x, int32_t x_dtype, int32_t T,
                                     const moe_qmat *router, const float *logit_bias, int32_t k,
                                     const moe_bank *routed, const moe_bank *shared, void *out,
                                     int32_t out_dtype, int32_t *ids_out, float *gates_out,
                                     void *stream);

/* HBM expert slot pool (per layer `slots` blobs in HBM; least-frequently-used
 * replacement: stork.ai blog, "Mas inteligente que tu RAM"; 16 slots per
 * layer: hndistilled.com, "Enfoque tecnico").  host_blobs is a HOST array of
 * n_layers * E pointers to page-locked host memory (hipHostMalloc), blob of
 * layer l, expert e at [l * E + e]; the blobs must outlive the pool.  The
 * pool owns its slots, pointer tables, side stream and events.  Requires
 * slots >= k of every forward call.  Single host thread. */
moe_status moe_pool_create(moe_pool **pool, int32_t n_layers, int32_t slots, int32_t E,
                           int32_t D, int32_t F, const void *const *host_blobs);
moe_status moe_pool_destroy(moe_pool *pool);
moe_status moe_pool_get_stats(const moe_pool *pool, moe_pool_stats *stats);
moe_status moe_pool_reset_stats(moe_pool *pool);

/* Host-only replay of the pool's replacement policy, for tests without a GPU:
 * ids host [n_tokens, k]; events host [n_tokens, k, 4] receives (expert,
 * slot, hit 0/1, evicted expert or -1) in ids order. */
moe_status moe_lfu_replay(int32_t slots, int32_t E, int32_t k, int32_t n_tokens,
                          const int32_t *ids, int32_t *events);

/* Replacement policy of a pool's slots: 0 least frequently used (the pages'
 * choice: stork.ai blog, "Mas inteligente que tu RAM"; the default), 1 least
 * recently used (victim: the resident expert the call does not need that was
 * used longest ago, ties to the lowest slot), for comparison (the pages weigh
 * other cache policies against LFU: hndistilled.com, "Enfoque tecnico").
 * Applies to the pool's later calls.  MOE_E_INVALID for another value. */
moe_status moe_pool_set_policy(moe_pool *pool, int32_t policy);

/* Test hook for the failure path of a pool's fetches: the pool lets `after`
 * more host -> HBM copies through and then reports the next one as failed
 * (once; -1 clears the hook).  The call that meets the failure returns
 * MOE_E_HIP after invalidating every slot it may have written, so that the
 * next call needing any of those experts fetches it again; as after any
 * MOE_E_HIP, zero-fill the workspace again before reusing it. */
moe_status moe_pool_fail_copy(moe_pool *pool, int32_t after);

/* moe_lfu_replay for either policy (0 LFU, 1 LRU). */
moe_status moe_cache_replay(int32_t policy, int32_t slots, int32_t E, int32_t k,
                            int32_t n_tokens, const int32_t *ids, int32_t *events);

/* Timing probe for measurement tools: while set, every moe_layer_forward
 * records events[2i] (a hipEvent_t) on its stream just before its expert
 * phase -- all work after routing: the one-launch expert kernel for decode,
 * the grouped matrix-core kernels for prefill -- and events[2i + 1] just
 * after it, i cycling through 0..n_pairs-1.  events: HOST array of 2*n_pairs
 * event handles owned by the caller; NULL / 0 turns the probe off.
 * Process-wide, single host thread. */
moe_status moe_set_profile_events(void *const *events, int32_t n_pairs);

/* Tuning knobs of the launch shapes; returns MOE_E_INVALID for an unknown
 * key or value.  Process-wide.  Every setting gives results within the same
 * parity bounds; the defaults are the measured fastest.  Keys (default):
 *   layer (1)            decode of up to 4 tokens in one launch of the layer
 *                        kernel; 0: off
 *   layer_ksg, layer_ksd (0)  its gate/up and down splits; 0: the widest
 *                        whose grid stays resident
 *   layer_order (1)      dispatch the shared expert's blocks before the routed
 *   layer_select (1)     the routed blocks rank the logits themselves; 0: the
 *                        router blocks rank and publish the selection
 *   block_fused (1)      moe_block_forward: both norms inside the one-launch
 *                        layer kernel; 0: separate row kernels
 *   layer_sel_copies (16), layer_log_copies (16), layer_sel_stride (0)
 *                        copies and spacing of the published selection
 *   fused (1)            the one-launch expert phase when the layer kernel
 *                        is off; fused_ksg, fused_ksd (0) its splits
 *   mid (0)              1: mid_min_t (2) to mid_max_t (7) tokens per
 *                        call, resident experts, when the layer kernel does
 *                        not take the call: kernels that read each distinct
 *                        selected expert and the shared expert once for all
 *                        tokens that use it (measured slower than the
 *                        per-token kernels, so off); mid_ksg, mid_kss,
 *                        mid_ksd (0) their routed, shared and down splits
 *   glu_ks, down_ks (0)  reduction splits of the few-token kernels
 *   prefill_min_t (8)    tokens per call from which the grouped matrix-core
 *                        kernels run
 *   route_mfma (1)       router of 16 or more tokens on the matrix cores */
moe_status moe_set_tuning(const char *key, int32_t value);

/* Measurement helper, not a step of the method: reads `bytes` of device
 * memory at `buf` once (16-byte aligned, a multiple of 16 bytes) with
 * streaming 16-byte loads over `blocks` workgroups of 256 threads, and writes
 * one uint32 per workgroup into sink (device [blocks]).  Its duration on a
 * buffer much larger than the 256 MB Infinity Cache measures the rate at
 * which the chip streams reads from HBM, the practical ceiling that the
 * benchmark also reports the kernels' achieved bytes per second against.
 * MOE_E_INVALID for a bad argument; asynchronous on `stream`. */
moe_status moe_read_probe(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks,
                          void *stream);

/* Static text for a status code. */
const char *moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
