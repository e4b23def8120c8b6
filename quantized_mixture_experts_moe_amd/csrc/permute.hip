// Token -> expert permutation of a prefill chunk.
//
// Prefill runs in chunks of up to 128 tokens so that one fetched expert
// serves all of its rows in the chunk (es.news.hada.io, "Proceso de generacion
// de tokens").  The (token, slot) pairs are grouped by expert: a histogram
// (integer LDS atomics, order-free), an exclusive scan, then a stable
// placement in which wave 0 walks the pairs 64 at a time and ranks equal
// experts inside the wave with ballots, so equal experts keep token order and
// the result is the same on every run.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t *__restrict__ ids, int n,
                                                       int E, int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ inv) {
  extern __shared__ int sm[];
  int *cnt = sm, *fill = sm + E;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = ids[i];
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
  if (tid >= 64) return;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int e = i < n ? ids[i] : -1;
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
                          int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), sizeof(int) * 2 * E, s, ids, T * k, E,
                     counts, offsets, perm, inv);
  return hipGetLastError();
}

}  // namespace moe
