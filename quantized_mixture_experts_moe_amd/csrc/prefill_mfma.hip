// Grouped expert FFN for prefill chunks on the matrix cores.
//
// Prompts are processed in chunks of up to 128 tokens so that one expert
// brought in once serves all of its rows in the chunk (es.news.hada.io,
// "Proceso de generacion de tokens").  After the token -> expert permutation
// each expert's rows form a contiguous group; a group with c rows multiplies
// a c x D activation block by the expert's 4-bit weights, a real (if skinny)
// matrix product, so these kernels use v_mfma_f32_16x16x32_{bf16,f16}.
//
// The work streams weights (about 430 MB per 128-token chunk against 17
// GFLOP).  Weights are read the way HBM likes them: one 16-byte chunk per
// lane, 64 consecutive rows per wave instruction (1 KB contiguous).  Each
// block stages one column group at a time in LDS (double buffered) and the
// waves read their matrix operands from there; every wave keeps the loads of
// the next kP groups in flight in a register ring, all issued
// unconditionally, so each wait covers exactly the group it needs.
//
// gate/up (glu_mfma_kernel): block = (expert, 64 hidden rows, 32 group rows);
//   per group the block stages gate and up codes (2 chunks x 64 rows each),
//   their scale/bias words and the activation pairs of its 32 rows.  Wave w
//   computes hidden rows 16w..16w+15.  B operand: 4-bit codes OR-ed into the
//   mantissa of 128.0 (bf16; 1024.0 for fp16), exact, in the column order
//   (m, m+4) of a code word; A operand: the activation pairs the router
//   kernel wrote in that same order.  One fp32 accumulator per 64-column
//   group; the affine terms fold per group as s * acc + (b - 128 s) * sum(x).
//   h = gelu(gate) * up is written as three bf16 planes (hi + mid + lo, 24
//   bits) and 64-unit sums.
// down (down_mfma_kernel): block = (expert, 256 output rows, 16 group rows);
//   per hidden group the block stages the down codes, their scale/bias words
//   and the three planes of h (once for its 256 rows: wave w computes output
//   rows 64w..64w+63).  B operand: codes as bf16 1 + q/16 (a nibble in the
//   mantissa of 1.0, exact), pairs (q_m, q_{m+4}); A operand: the planes in
//   the same pair order, three products per step; per group the fold is
//   16 s * sum h (1 + q/16) + (b - 16 s) * sum h.  The small offset (1, not
//   128) keeps the fp32 sums close to exact although h has a large mean.
// combine (combine_prefill_kernel): out[t] = y_shared[t] + sum_j gate y[inv].
#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRows = kPrefillRows;  // group rows per block (one or two 16-row tiles)
static_assert(kRows == 32, "one or two 16-row tiles");

// XCD-grouped block order.  Workgroups go to the 8 XCDs round robin (block b
// to XCD b % 8), and each XCD has its own L2.  Blocks that read the same
// weights (the row chunks of one weight slice) or the same activations (the
// tiles of one work-list item) are given indices that are equal mod 8 and
// close together, so the second reader finds the bytes in its XCD's L2
// instead of fetching them again.  A part of the grid covers n_slices
// slices of `per` blocks each: slice i lives on one XCD, slices alternate
// over the XCDs in a serpentine (0..7, 7..0, ...) so that a list sorted
// longest first spreads evenly.  Its block count is a multiple of 8, so the
// next part keeps the same XCD for the same index mod 8.
constexpr int kXcd = 8;
__host__ __device__ inline int grouped_blocks(int n_slices, int per) {
  return (n_slices + kXcd - 1) / kXcd * kXcd * per;
}
// block r of the part -> (slice, sub-block); slice may be >= n_slices (padding)
__device__ __forceinline__ void grouped_index(int r, int per, int *slice, int *sub) {
  const int x = r % kXcd, q = r / kXcd, i = q / per;
  *sub = q - i * per;
  *slice = i * kXcd + ((i & 1) ? kXcd - 1 - x : x);
}

template <bool F16>
__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 8 codes of one word -> (offset + q) pairs (q_m, q_{m+4}), m = 0..3
__device__ __forceinline__ u32x4_t unpack_magic(uint32_t w, uint32_t magic) {
  u32x4_t r;
  r.x = (w & 0x000F000Fu) | magic;
  r.y = ((w >> 4) & 0x000F000Fu) | magic;
  r.z = ((w >> 8) & 0x000F000Fu) | magic;
  r.w = ((w >> 12) & 0x000F000Fu) | magic;
  return r;
}

struct Group {
  const uint8_t *blob;
  int count, off, F;  // rows, first row in the pair order, hidden width
  bool shared;
};

__device__ __forceinline__ Group group_of(const PrefillLaunch &p, int g_idx) {
  Group g;
  if (g_idx < p.E) {
    g.count = p.counts[g_idx];
    g.off = p.offsets[g_idx];
    g.F = p.F;
    g.blob = (const uint8_t *)p.rblobs[g_idx];
    g.shared = false;
  } else {
    g.count = p.T;
    g.off = p.T * p.k;
    g.F = p.Fs;
    g.blob = (const uint8_t *)p.sblobs[0];
    g.shared = true;
  }
  return g;
}

// token of pair row r (absolute row index: routed rows first, then shared)
__device__ __forceinline__ int token_of(const PrefillLaunch &p, const Group &g, int r) {
  return g.shared ? r - p.T * p.k : p.perm[r] / p.k;
}

// hidden-activation planes and sums of row r
__device__ __forceinline__ size_t hrow_off(const PrefillLaunch &p, int r) {
  return r < p.T * p.k ? (size_t)r * p.F : (size_t)p.T * p.k * p.F + (size_t)(r - p.T * p.k) * p.Fs;
}

// Direct global -> LDS loads (no registers): lane i's `size` bytes land at
// dst + i * size; dst must be the same for the whole wave.
__device__ __forceinline__ void dma16(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                   (void __attribute__((address_space(3))) *)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                   (void __attribute__((address_space(3))) *)dst, 4, 0, 0);
}
// Wait until at most n of this wave's vector-memory operations are
// outstanding (they complete in order), then meet the other waves: the
// staged data of every wave is then in LDS.  No fence: the loads in flight
// for later stages stay in flight.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // compiler barriers: no LDS access moves across the wait and the barrier
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte slot of (row t, vector v of 8) in a staged [32 rows][8 vectors]
// tile: rows rotate their vectors so that 16 rows read at one v spread over
// the banks
__device__ __forceinline__ int xslot(int t, int v) { return t * 8 + (v ^ (t & 7)); }

// ---------------------------------------------------------------- gate/up
constexpr int kRg = 4;  // LDS stages of the gate/up ring (kRg - 1 groups in flight)

struct GluBuf {
  u32x4_t w[4][64];        // (matrix, half): gate lo/hi chunk, up lo/hi; row = lane
  uint32_t m[2][64];       // gate meta (staged by waves 0, 2), up meta (waves 1, 3)
  u32x4_t x[kRows * 8];    // activation pairs of the 32 rows, xslot order
};
// h of the tile [row][hidden col], in the first stage's buffer once the ring
// is drained (so that four blocks fit in a CU's LDS)
static_assert(sizeof(float) * kRows * 65 <= sizeof(GluBuf), "h fits in one stage");

template <bool F16X, int NM>
__device__ __forceinline__ void glu_body(const PrefillLaunch &p, const Group &g, int nt, int m0,
                                         int nrow, const int *s_tok, const float *s_xs,
                                         GluBuf &b0, GluBuf &b1, GluBuf &b2, GluBuf &b3) {
  // one LDS object per stage, so that a read of one stage does not wait for
  // the loads in flight into the others
  auto buf = [&](int s) -> GluBuf & { return s == 0 ? b0 : s == 1 ? b1 : s == 2 ? b2 : b3; };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = p.D, G = D / 64, F = g.F;
  const int col = lane & 15, kb = lane >> 4;
  const BlobLayout L = blob_layout(D, F);
  // this wave stages, per group: one code piece (matrix wave / 2, half
  // wave % 2; row = lane), the scale/bias words of matrix wave % 2 (waves 2
  // and 3 write the same words as waves 0 and 1: loads are issued
  // unconditionally, so the waits stay exact), and the activation pairs of
  // rows 8 wave .. 8 wave + 7 (lane p: row t = 8 wave + p / 8, vector
  // (p % 8) ^ (t & 7), so that it lands in its xslot)
  const u32x4_t *wsrc = (const u32x4_t *)(g.blob + ((wave >> 1) ? L.up_codes : L.gate_codes)) +
                        (size_t)(wave & 1) * F + nt * 64 + lane;
  const uint32_t *msrc =
      (const uint32_t *)(g.blob + ((wave & 1) ? L.up_meta : L.gate_meta)) + nt * 64 + lane;
  const int xt = 8 * wave + (lane >> 3), xv = (lane & 7) ^ (xt & 7);
  const u32x4_t *xsrc = (const u32x4_t *)(p.xp + (size_t)s_tok[xt] * (D / 2)) + xv;
  auto issue = [&](GluBuf &B, int gi) {
    gi = min(gi, G - 1);  // past the end: a repeat of the last group, folded with weight 0
    dma16(wsrc + (size_t)(2 * gi) * F, &B.w[wave][0]);
    dma4(msrc + (size_t)gi * F, &B.m[wave & 1][0]);  // waves 2, 3: the same words again
    dma16(xsrc + gi * 8, &B.x[64 * wave]);
  };
  const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);

  f32x4_t tg[NM], tu[NM];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
    tg[mt] = f32x4_t{0, 0, 0, 0};
    tu[mt] = f32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int s = 0; s < kRg - 1; ++s) issue(buf(s), s);
  for (int g0 = 0; g0 < G; g0 += kRg) {
#pragma unroll
    for (int s = 0; s < kRg; ++s) {
      const int gi = g0 + s;
      // this group's stage is in (3 loads per stage per wave; kRg - 2 later
      // stages may stay in flight), and every wave is done with group gi - 1
      stage_barrier<3 * (kRg - 2)>();
      issue(buf((s + kRg - 1) % kRg), gi + kRg - 1);
      const GluBuf &B = buf(s);
      const bool live = gi < G;
      f32x4_t ag[NM], au[NM];
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        ag[mt] = f32x4_t{0, 0, 0, 0};
        au[mt] = f32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4_t bg = unpack_magic(((const uint32_t *)&B.w[half][wave * 16 + col])[kb], magic);
        const u32x4_t bu = unpack_magic(((const uint32_t *)&B.w[2 + half][wave * 16 + col])[kb], magic);
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
          const u32x4_t a = B.x[xslot(mt * 16 + col, half * 4 + kb)];
          ag[mt] = mfma<F16X>(a, bg, ag[mt]);
          au[mt] = mfma<F16X>(a, bu, au[mt]);
        }
      }
      const uint32_t mg = B.m[0][wave * 16 + col], mu = B.m[1][wave * 16 + col];
      const float sg = live ? f16_to_f32(mg) : 0.0f, bgv = live ? f16_to_f32(mg >> 16) : 0.0f;
      const float su = live ? f16_to_f32(mu) : 0.0f, buv = live ? f16_to_f32(mu >> 16) : 0.0f;
      const float cg = fmaf(-Magic<F16X>::offset, sg, bgv);
      const float cu = fmaf(-Magic<F16X>::offset, su, buv);
      const int gx = min(gi, G - 1);
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xsv = s_xs[(mt * 16 + kb * 4 + i) * G + gx];
          tg[mt][i] = fmaf(sg, ag[mt][i], fmaf(cg, xsv, tg[mt][i]));
          tu[mt][i] = fmaf(su, au[mt][i], fmaf(cu, xsv, tu[mt][i]));
        }
      }
    }
  }
  // the stages past the end are still landing in LDS: let them finish (and
  // every wave is past its last read of the ring)
  stage_barrier<0>();
  float (*s_h)[65] = reinterpret_cast<float (*)[65]>(&b0);
  // h into LDS [row][hidden col of the tile]
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s_h[mt * 16 + kb * 4 + i][wave * 16 + col] = gelu_tanh(tg[mt][i]) * tu[mt][i];
  }
  __syncthreads();
  // three bf16 planes (in the pair order (h[8v + m], h[8v + m + 4]) of the
  // down kernel's code pairs) and the 64-unit sum of every valid row
  for (int idx = threadIdx.x; idx < nrow * 64; idx += 256) {
    const int m = idx >> 6, c = idx & 63;
    const float h = s_h[m][c];
    const uint32_t hi = f32_to_bf16(h);
    const float r1 = h - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16(r1);
    const uint32_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    const int u = c & 7, pos = (c & ~7) | (u < 4 ? 2 * u : 2 * (u - 4) + 1);
    const size_t o = hrow_off(p, g.off + m0 + m) + (size_t)nt * 64 + pos;
    p.hp[o] = (uint16_t)hi;
    p.hp[p.plane + o] = (uint16_t)mid;
    p.hp[2 * p.plane + o] = (uint16_t)lo;
  }
  if (threadIdx.x < nrow) {
    const int m = threadIdx.x;
    float s = 0.0f;
    for (int c = 0; c < 64; ++c) s += s_h[m][c];
    p.hsum[hrow_off(p, g.off + m0 + m) / 64 + nt] = s;
  }
}

template <bool F16X>
__global__ __launch_bounds__(256, 4) void glu_mfma_kernel(PrefillLaunch p) {
  extern __shared__ float s_dyn[];  // [kRows][G] 64-column sums of x
  __shared__ int s_tok[kRows];
  __shared__ GluBuf b0, b1, b2, b3;
  static_assert(kRg == 4, "one LDS object per stage");
  // blocks, longest first so that they do not form the tail: the shared
  // expert's (every row chunk of it has rows), then the work list's items
  // (expert by count, most rows first, and row chunk) x tiles; the blocks
  // past the list's end return at once
  const int NT = p.F / 64, NTs = p.sblobs ? p.Fs / 64 : 0;
  const int mch = (p.T + kRows - 1) / kRows;
  const int bid = blockIdx.x, nsh = NTs ? grouped_blocks(NTs, mch) : 0;
  int g_idx, nt, yc;
  Group rg{};
  if (bid < nsh) {
    // the shared expert: hidden tile nt's row chunks on one XCD
    g_idx = p.E;
    grouped_index(bid, mch, &nt, &yc);
    if (nt >= NTs) return;
  } else {
    g_idx = -1;
    // a work-list item's hidden tiles on one XCD
    int item;
    grouped_index(bid - nsh, NT, &item, &nt);
    if (item >= p.max_items) return;
    // the item, its expert's count, offset and blob, and the list's length
    // in one round trip (every index here is inside the arrays)
    const int n_it = *p.n_items, it = p.items[item];
    const int2 inf = p.item_info[item];
    const void *bl = p.item_blob[item];
    if (item >= n_it) return;
    if (p.batch_blob) {  // a batch of a streamed call: only its experts, from their slots
      bl = p.batch_blob[it & 0xFFFF];
      if (!bl) return;
    }
    yc = it >> 16;
    rg.count = inf.x, rg.off = inf.y, rg.F = p.F, rg.blob = (const uint8_t *)bl, rg.shared = false;
  }
  const Group g = g_idx < 0 ? rg : group_of(p, g_idx);
  const int m0 = yc * kRows;
  if (g.count <= m0) return;
  const int nrow = min(kRows, g.count - m0);
  const int G = p.D / 64;
  for (int i = threadIdx.x; i < kRows; i += 256) {
    const int m = min(i, nrow - 1);
    s_tok[i] = token_of(p, g, g.off + m0 + m);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRows * G; i += 256) {
    const int m = i / G, gg = i - m * G;
    s_dyn[i] = p.xs[(size_t)s_tok[m] * G + gg];
  }
  __syncthreads();
  if (nrow <= 16)
    glu_body<F16X, 1>(p, g, nt, m0, nrow, s_tok, s_dyn, b0, b1, b2, b3);
  else
    glu_body<F16X, 2>(p, g, nt, m0, nrow, s_tok, s_dyn, b0, b1, b2, b3);
}

// ---------------------------------------------------------------- down
constexpr int kRd = 2;    // LDS stages of the down ring (kRd - 1 groups in flight)
constexpr int kDT = 4;    // 16-row output tiles per wave (a block covers 256 output rows)
constexpr int kDRows = 16;  // group rows per down block (one matrix tile)

struct DownBuf {
  u32x4_t pl[3][kDRows * 8];  // planes of h (pair order) for the 16 rows, xslot order
  u32x4_t w[2][4 * 64];       // down codes, chunks 2gi and 2gi + 1; row = 64 wave + lane
  uint32_t m[4 * 64];         // scale/bias words of the 256 rows
};

__device__ __forceinline__ void down_body(const PrefillLaunch &p, const Group &g, int nb, int m0,
                                          int nrow, int gbeg, int GH, float *dst, int row0,
                                          const int *s_row, const float *s_hs, DownBuf &b0,
                                          DownBuf &b1) {
  // one LDS object per stage, so that a read of one stage does not wait for
  // the loads in flight into the others
  auto buf = [&](int s) -> DownBuf & { return s == 0 ? b0 : b1; };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // hidden groups gbeg .. gbeg + GH - 1 of the expert; s_hs holds their h
  // sums, [row][group - gbeg]
  const int D = p.D, F = g.F;
  const int col = lane & 15, kb = lane >> 4;
  const BlobLayout L = blob_layout(D, F);
  // this wave stages, per hidden group: plane wave % 3 of the 16 rows (two
  // loads of 8 rows; wave 3 loads plane 0 again, onto the same words, so
  // that every wave issues the same loads and the waits stay exact; lane p:
  // row t = 8 j + p / 8, vector (p % 8) ^ (t & 7), so that it lands in its
  // xslot), the two code chunks and the scale/bias word of output row
  // 64 wave + lane
  const int pq = wave % 3;
  const int xv = (lane & 7) ^ ((lane >> 3) & 7);
  const size_t plane_v = p.plane / 8;  // plane size in 16-byte vectors
  const u32x4_t *hsrc0 = (const u32x4_t *)(p.hp + hrow_off(p, s_row[lane >> 3])) + pq * plane_v + xv;
  const u32x4_t *hsrc1 =
      (const u32x4_t *)(p.hp + hrow_off(p, s_row[8 + (lane >> 3)])) + pq * plane_v + xv;
  const int wrow = min(nb * 256 + wave * 64 + lane, D - 1);
  const u32x4_t *wsrc = (const u32x4_t *)(g.blob + L.down_codes) + wrow;
  const uint32_t *msrc = (const uint32_t *)(g.blob + L.down_meta) + wrow;
  auto issue = [&](DownBuf &B, int gi) {
    gi = gbeg + min(gi, GH - 1);  // past the end: a repeat of the last group, folded with weight 0
    dma16(hsrc0 + gi * 8, &B.pl[pq][0]);
    dma16(hsrc1 + gi * 8, &B.pl[pq][64]);
    dma16(wsrc + (size_t)(2 * gi) * D, &B.w[0][64 * wave]);
    dma16(wsrc + (size_t)(2 * gi + 1) * D, &B.w[1][64 * wave]);
    dma4(msrc + (size_t)gi * D, &B.m[64 * wave]);
  };
  const uint32_t umagic = opaque_vgpr(0x3F803F80u);  // bf16 1.0 pairs

  // each group's fold is added in double: the rows' sums reach about 5e4
  // (the folds of a few groups already about 3e4), where adding the folds in
  // fp32 rounds at several ulps of the result over the expert's groups
  double t[kDT][4];
#pragma unroll
  for (int j = 0; j < kDT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) t[j][i] = 0.0;
#pragma unroll
  for (int s = 0; s < kRd - 1; ++s) issue(buf(s), s);
  for (int g0 = 0; g0 < GH; g0 += kRd) {
#pragma unroll
    for (int s = 0; s < kRd; ++s) {
      const int gi = g0 + s;
      // this group's stage is in (5 loads per stage per wave; kRd - 2 later
      // stages may stay in flight), and every wave is done with group gi - 1
      stage_barrier<5 * (kRd - 2)>();
      issue(buf((s + kRd - 1) % kRd), gi + kRd - 1);
      const DownBuf &B = buf(s);
      const bool live = gi < GH;
      const int gx = gbeg + min(gi, GH - 1);
      // the planes of the block's rows, shared by the wave's kDT output tiles
      u32x4_t a_in[2][3];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int q = 0; q < 3; ++q) a_in[half][q] = B.pl[q][xslot(col, half * 4 + kb)];
      float hs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[i] = s_hs[(kb * 4 + i) * GH + (gx - gbeg)];
#pragma unroll
      for (int j = 0; j < kDT; ++j) {
        // output tile j of this wave: rows 64 wave + 16 j + col
        const int r = wave * 64 + j * 16 + col;
        f32x4_t a = f32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x4_t b = code_pairs_unit(((const uint32_t *)&B.w[half][r])[kb], umagic);
          a = mfma<false>(a_in[half][0], b, a);
          a = mfma<false>(a_in[half][1], b, a);
          a = mfma<false>(a_in[half][2], b, a);
        }
        // sum h (1 + q/16) = sum h + sum h q / 16: fold s q + b per group
        const uint32_t mw = B.m[r];
        const float sd = live ? f16_to_f32(mw) : 0.0f, bd = live ? f16_to_f32(mw >> 16) : 0.0f;
        const float s16 = 16.0f * sd, c16 = fmaf(-16.0f, sd, bd);
#pragma unroll
        for (int i = 0; i < 4; ++i) t[j][i] += (double)fmaf(s16, a[i], c16 * hs[i]);
      }
    }
  }
  // the stages past the end are still landing in LDS: let them finish
  stage_barrier<0>();
  // the lane's column and row block, computed again rather than held
  // through the loop (at five blocks per CU the two would be spilled)
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const int col2 = ln & 15, kb2 = ln >> 4;
#pragma unroll
  for (int j = 0; j < kDT; ++j) {
    const int n = nb * 256 + wave * 64 + j * 16 + col2;  // output row of this lane's column
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = kb2 * 4 + i;
      if (m < nrow && n < D) dst[(size_t)(row0 + m0 + m) * D + n] = (float)t[j][i];
    }
  }
}

__global__ __launch_bounds__(256, 5) void down_mfma_kernel(PrefillLaunch p) {
  __shared__ int s_row[kDRows];
  // h sums of the block's own hidden groups, [row][group], sized at launch
  // (static LDS of 30.8 KB plus these: five blocks per CU)
  extern __shared__ float s_hs[];
  __shared__ DownBuf b0, b1;
  static_assert(kRd == 2, "one LDS object per stage");
  static_assert(kRows == 2 * kDRows, "two down row chunks per work-list item");
  // blocks: the shared expert's first, its hidden groups split sks ways (as
  // many groups per block as a routed expert has), then the work list's
  // items x their two 16-row halves x 256 output rows (the second half of
  // an item with 16 rows or fewer returns at once)
  const int D = p.D, NB = (D + 255) / 256;
  const int mch = (p.T + kDRows - 1) / kDRows;
  const int nsh = p.sblobs ? grouped_blocks(p.sks * NB, mch) : 0;
  const int bid = blockIdx.x;
  int g_idx, nb, yc, ks = 0;
  Group rg{};
  if (bid < nsh) {
    // the shared expert: the row chunks of weight slice (ks, nb) on one XCD
    g_idx = p.E;
    int w;
    grouped_index(bid, mch, &w, &yc);
    if (w >= p.sks * NB) return;
    ks = w / NB;
    nb = w - ks * NB;
  } else {
    g_idx = -1;
    // a work-list item's halves and output tiles on one XCD (the halves
    // read the same weights, the tiles the same hidden values)
    int item, rr;
    grouped_index(bid - nsh, 2 * NB, &item, &rr);
    if (item >= p.max_items) return;
    const int half = rr / NB;
    nb = rr - half * NB;
    // the item, its expert's count, offset and blob, and the list's length
    // in one round trip (every index here is inside the arrays)
    const int n_it = *p.n_items, it = p.items[item];
    const int2 inf = p.item_info[item];
    const void *bl = p.item_blob[item];
    if (item >= n_it) return;
    if (p.batch_blob) {
      bl = p.batch_blob[it & 0xFFFF];
      if (!bl) return;
    }
    yc = 2 * (it >> 16) + half;
    rg.count = inf.x, rg.off = inf.y, rg.F = p.F, rg.blob = (const uint8_t *)bl, rg.shared = false;
  }
  const Group g = g_idx < 0 ? rg : group_of(p, g_idx);
  const int m0 = yc * kDRows;
  if (g.count <= m0) return;
  const int nrow = min(kDRows, g.count - m0);
  const int GH = g.F / 64;
  const int gbeg = g.shared ? ks * GH / p.sks : 0, gend = g.shared ? (ks + 1) * GH / p.sks : GH;
  // routed rows into y (at their pair row), shared rows into partial ks of ys
  float *dst = g.shared ? p.ys + (size_t)ks * p.T * D : p.y;
  const int row0 = g.shared ? 0 : g.off;
  for (int i = threadIdx.x; i < kDRows; i += 256) s_row[i] = g.off + m0 + min(i, nrow - 1);
  __syncthreads();
  const int GL = gend - gbeg;
  for (int i = threadIdx.x; i < kDRows * GL; i += 256) {
    const int m = i / GL, gg = i - m * GL;
    s_hs[i] = p.hsum[hrow_off(p, s_row[m]) / 64 + gbeg + gg];
  }
  __syncthreads();
  down_body(p, g, nb, m0, nrow, gbeg, GL, dst, row0, s_row, s_hs, b0, b1);
}

// four consecutive outputs per thread (16-byte loads of y), the k routed
// rows in fixed j order after the shared expert's partial sums.  The rows'
// positions and gates are read first and every row's load is issued before
// the sums (KB rows per batch), so a thread waits for two round trips per
// batch instead of two per row.
template <int KB>
__global__ void combine_prefill_kernel(PrefillLaunch p) {
  const size_t total = (size_t)p.T * p.D, total4 = total / 4;
  const int D4 = p.D / 4, k = p.k;
  const bool aligned = ((uintptr_t)p.out & 15) == 0;  // else element by element
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total4;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / D4, d = (i - t * D4) * 4;
    // summed in double and rounded once: the outputs reach about 1e5, where
    // one fp32 rounding per added row would already cost several ulps (a
    // product of two floats is exact in double)
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    if (p.sblobs) {
      float4 v[kMaxSharedSplits];
#pragma unroll
      for (int ks = 0; ks < kMaxSharedSplits; ++ks)
        if (ks < p.sks) v[ks] = *(const float4 *)(p.ys + (size_t)ks * total + t * p.D + d);
#pragma unroll
      for (int ks = 0; ks < kMaxSharedSplits; ++ks)
        if (ks < p.sks) s[0] += v[ks].x, s[1] += v[ks].y, s[2] += v[ks].z, s[3] += v[ks].w;
    }
    for (int j0 = 0; j0 < k; j0 += KB) {
      int row[KB];
      float gt[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int jj = min(j0 + j, k - 1);
        row[j] = p.inv[t * k + jj];
        gt[j] = p.gates[t * k + jj];
      }
      float4 v[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) v[j] = *(const float4 *)(p.y + (size_t)row[j] * p.D + d);
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (j0 + j < k) {
          const double g = gt[j];
          s[0] = fma(g, (double)v[j].x, s[0]), s[1] = fma(g, (double)v[j].y, s[1]);
          s[2] = fma(g, (double)v[j].z, s[2]), s[3] = fma(g, (double)v[j].w, s[3]);
        }
      }
    }
    const float4 sf = make_float4((float)s[0], (float)s[1], (float)s[2], (float)s[3]);
    const size_t o = t * p.D + d;
    if (!aligned) {
      const float v[4] = {sf.x, sf.y, sf.z, sf.w};
      for (int u = 0; u < 4; ++u) {
        if (p.out_dtype == MOE_F32)
          ((float *)p.out)[o + u] = v[u];
        else if (p.out_dtype == MOE_BF16)
          ((uint16_t *)p.out)[o + u] = (uint16_t)f32_to_bf16(v[u]);
        else
          ((uint16_t *)p.out)[o + u] = (uint16_t)f32_to_f16(v[u]);
      }
    } else if (p.out_dtype == MOE_F32) {
      *(float4 *)((float *)p.out + o) = sf;
    } else {
      const bool bf = p.out_dtype == MOE_BF16;
      const uint32_t c0 = bf ? f32_to_bf16(sf.x) : f32_to_f16(sf.x);
      const uint32_t c1 = bf ? f32_to_bf16(sf.y) : f32_to_f16(sf.y);
      const uint32_t c2 = bf ? f32_to_bf16(sf.z) : f32_to_f16(sf.z);
      const uint32_t c3 = bf ? f32_to_bf16(sf.w) : f32_to_f16(sf.w);
      *(uint2 *)((uint16_t *)p.out + o) = make_uint2(c0 | (c1 << 16), c2 | (c3 << 16));
    }
  }
}

}  // namespace

hipError_t launch_prefill_experts(const PrefillLaunch &p, hipStream_t s) {
  if (p.D / 64 > kMaxDGroups || p.F / 64 > kMaxHGroups || p.Fs / 64 > kMaxHGroups)
    return hipErrorInvalidValue;
  if (p.sblobs && (p.sks < 1 || p.sks > kMaxSharedSplits)) return hipErrorInvalidValue;
  const int mchunks = (p.T + kRows - 1) / kRows;
  // routed blocks: the work list has at most one partial chunk per expert
  const int max_items = std::min(p.E * mchunks, p.E + (p.T * p.k + kRows - 1) / kRows);
  PrefillLaunch q = p;
  q.max_items = max_items;
  dim3 g1(grouped_blocks(max_items, p.F / 64) +
          (p.sblobs ? grouped_blocks(p.Fs / 64, mchunks) : 0));
  const size_t smem = sizeof(float) * kRows * (p.D / 64);
  if (p.f16x)
    hipLaunchKernelGGL(glu_mfma_kernel<true>, g1, dim3(256), smem, s, q);
  else
    hipLaunchKernelGGL(glu_mfma_kernel<false>, g1, dim3(256), smem, s, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb4 = (p.D + 255) / 256;  // 256 output rows per down block
  const int mch16 = (p.T + 15) / 16;  // 16-row chunks of the shared expert
  dim3 g2(grouped_blocks(max_items, 2 * nb4) + (p.sblobs ? grouped_blocks(p.sks * nb4, mch16) : 0));
  // h sums of a block's hidden groups: all of a routed expert's, or the
  // largest of the shared expert's sks slices
  const int gl = std::max(p.F / 64, p.sblobs ? (p.Fs / 64 + p.sks - 1) / p.sks : 0);
  hipLaunchKernelGGL(down_mfma_kernel, g2, dim3(256), sizeof(float) * kDRows * gl, s, q);
  e = hipGetLastError();
  if (e != hipSuccess || p.skip_combine) return e;
  return launch_prefill_combine(p, s);
}

hipError_t launch_prefill_combine(const PrefillLaunch &p, hipStream_t s) {
  PrefillLaunch q = p;
  const size_t total = (size_t)p.T * p.D / 4;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(combine_prefill_kernel<8>, dim3(blocks), dim3(256), 0, s, q);
  return hipGetLastError();
}

}  // namespace moe
