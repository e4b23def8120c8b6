// Token -> expert permutation of a prefill chunk.
//
// Prefill runs in chunks of up to 128 tokens so that one fetched expert
// serves all of its rows in the chunk (es.news.hada.io, "Proceso de generacion
// de tokens").  The (token, slot) pairs are grouped by expert: a histogram
// (integer LDS atomics, order-free), an exclusive scan, then a stable
// placement in which wave 0 walks the pairs 64 at a time and ranks equal
// experts inside the wave with ballots, so equal experts keep token order and
// the result is the same on every run.  The expert ids are read from memory
// once, by all threads, and kept in LDS (up to kStageIds pairs).  When every
// chunk of 64 pairs has a wave of its own, the chunks are placed in parallel:
// a chunk's pairs of expert e follow the pairs of e in the earlier chunks
// (counted per chunk, summed in chunk order), which is the same placement.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kStageIds = 8192;  // pairs whose ids the walk reads from LDS
constexpr int kChunkHist = 8192; // chunk x expert counts for the parallel placement

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t *__restrict__ ids, int n,
                                                       int E, int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ inv,
                                                       int32_t *__restrict__ items,
                                                       int32_t *__restrict__ n_items,
                                                       int chunk_rows, int2 *__restrict__ info,
                                                       const void **__restrict__ iblob,
                                                       const void *const *__restrict__ blobs) {
  extern __shared__ int sm[];
  __shared__ int s_bkt[kMaxE], s_bst[kMaxE];
  int *cnt = sm, *fill = sm + E, *sid = sm + 2 * E;
  const bool staged = n <= kStageIds;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = ids[i];
    if (staged) sid[i] = e;
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < 64) {
    const int per = (E + 63) / 64, base = lane * per;
    int s = 0;
    for (int j = 0; j < per; ++j)
      if (base + j < E) s += cnt[base + j];
    int incl = s;
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int excl = incl - s;
    for (int j = 0; j < per; ++j) {
      if (base + j < E) {
        fill[base + j] = excl;
        offsets[base + j] = excl;
        counts[base + j] = cnt[base + j];
        excl += cnt[base + j];
      }
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  // work list of the grouped kernels: (expert, chunk of chunk_rows rows)
  // items, experts in buckets of chunk_rows / 2 rows, the fullest first, so
  // that the longest blocks start first and no block is spent on an empty
  // chunk.  All experts of a bucket have the same number of chunks; the
  // order inside a bucket is whatever the LDS atomics give: every item is
  // computed on its own, so the results do not depend on it.
  if (items) {
    const int half = (chunk_rows + 1) / 2;
    const int nb = (n + half - 1) / half + 1;  // buckets 0 .. ceil(max count / half)
    auto chunks = [&](int b) { return (b * half + chunk_rows - 1) / chunk_rows; };
    if (nb <= kMaxE) {
      for (int i = tid; i < nb; i += blockDim.x) s_bkt[i] = 0, s_bst[i] = 0;
      __syncthreads();
      for (int e = tid; e < E; e += blockDim.x) atomicAdd(&s_bkt[(cnt[e] + half - 1) / half], 1);
      __syncthreads();
      if (tid < 64) {  // first item of each bucket, fullest first (one wave scan)
        const int per = (nb + 63) / 64, base = lane * per;
        int sum = 0;
        for (int j = 0; j < per; ++j) {
          const int b = nb - 1 - (base + j);
          if (b >= 0) sum += s_bkt[b] * chunks(b);
        }
        int incl = sum;
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(incl, off, 64);
          if (lane >= off) incl += v;
        }
        int at = incl - sum;
        for (int j = 0; j < per; ++j) {
          const int b = nb - 1 - (base + j);
          if (b >= 0) {
            s_bst[b] = at;
            at += s_bkt[b] * chunks(b);
            s_bkt[b] = 0;  // now the bucket's fill count
          }
        }
        if (lane == 63) *n_items = incl;
      }
      __syncthreads();
      for (int e = tid; e < E; e += blockDim.x) {
        const int b = (cnt[e] + half - 1) / half, nc = chunks(b);
        if (nc == 0) continue;
        const int at = s_bst[b] + atomicAdd(&s_bkt[b], 1) * nc;
        const void *bl = info ? blobs[e] : nullptr;
        for (int yc = 0; yc < nc; ++yc) {
          items[at + yc] = e | (yc << 16);
          if (info) info[at + yc] = make_int2(cnt[e], fill[e]), iblob[at + yc] = bl;
        }
      }
    } else if (tid < 64) {  // too many buckets: experts in index order
      const int per = (E + 63) / 64, base = lane * per;
      int sum = 0;
      for (int j = 0; j < per; ++j)
        if (base + j < E) sum += (cnt[base + j] + chunk_rows - 1) / chunk_rows;
      int incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      int at = incl - sum;
      for (int j = 0; j < per; ++j) {
        if (base + j < E) {
          const int e = base + j, nc = (cnt[e] + chunk_rows - 1) / chunk_rows;
          const void *bl = info && nc ? blobs[e] : nullptr;
          for (int yc = 0; yc < nc; ++yc) {
            items[at + yc] = e | (yc << 16);
            if (info) info[at + yc] = make_int2(cnt[e], fill[e]), iblob[at + yc] = bl;
          }
          at += nc;
        }
      }
      if (lane == 63) *n_items = incl;
    }
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int nch = (n + 63) / 64;
  if (staged && nch <= 16 && nch * E <= kChunkHist) {  // 16 waves
    // one wave per chunk of 64 pairs: ranks inside the chunk by ballots, the
    // chunk's count of each of its experts, then (per expert, over the
    // chunks in order) the pairs of that expert in earlier chunks
    int *hist = sid + n;  // [nch][E]
    for (int i = tid; i < nch * E; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const int c = tid >> 6, i = 64 * c + lane;
    int e = -1, rank = 0, cnt_e = 0;
    if (c < nch) {
      e = i < n ? sid[i] : -1;
      const bool valid = e >= 0 && e < E;
      unsigned long long mask = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bal = __ballot(valid && bit);
        mask &= bit ? bal : ~bal;
      }
      if (valid) {
        rank = __popcll(mask & ((1ull << lane) - 1ull));
        cnt_e = __popcll(mask);
        if (rank == 0) hist[c * E + e] = cnt_e;
      } else {
        e = -1;
      }
    }
    __syncthreads();
    // exclusive prefix over the chunks, per expert, from the expert's offset
    for (int x = tid; x < E; x += blockDim.x) {
      int run = fill[x];
      for (int cc = 0; cc < nch; ++cc) {
        const int v = hist[cc * E + x];
        hist[cc * E + x] = run;
        run += v;
      }
    }
    __syncthreads();
    if (c < nch && i < n) {
      if (e >= 0) {
        const int pos = hist[c * E + e] + rank;
        perm[pos] = i;
        inv[i] = pos;
      } else {
        inv[i] = -1;
      }
    }
    return;
  }
  if (tid >= 64) return;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int e = i < n ? (staged ? sid[i] : ids[i]) : -1;
    const bool valid = e >= 0 && e < E;
    unsigned long long mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long bal = __ballot(valid && bit);
      mask &= bit ? bal : ~bal;
    }
    int rank = 0;
    if (valid) {
      rank = __popcll(mask & ((1ull << lane) - 1ull));
      const int pos = fill[e] + rank;
      perm[pos] = i;
      inv[i] = pos;
    } else if (i < n) {
      inv[i] = -1;
    }
    if (valid && rank == 0) fill[e] += __popcll(mask);
  }
}

}  // namespace

hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *items,
                          int32_t *n_items, int chunk_rows, hipStream_t s, int2 *info,
                          const void **iblob, const void *const *blobs) {
  if (E > kMaxE || (items && (!n_items || chunk_rows < 1))) return hipErrorInvalidValue;
  if (info && (!items || !iblob || !blobs)) return hipErrorInvalidValue;
  const int n = T * k;
  const int nch = (n + 63) / 64;
  const bool par = n <= kStageIds && nch <= 16 && nch * E <= kChunkHist;  // as the kernel decides
  const size_t smem =
      sizeof(int) * (2 * (size_t)E + (n <= kStageIds ? n : 0) + (par ? (size_t)nch * E : 0));
  if (smem > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), smem, s, ids, n, E, counts, offsets,
                     perm, inv, items, n_items, chunk_rows, info, iblob, blobs);
  return hipGetLastError();
}

}  // namespace moe
