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
// down (down_mfma_kernel): block = (expert, 256 output rows, 32 group rows);
//   per hidden group the block stages the down codes, their scale/bias words
//   and the three planes of h (once for its 256 rows: wave w computes output
//   rows 64w..64w+63).  B operand: exact codes (byte spread,
//   v_cvt_f32_ubyte, packed to bf16); A operand: the planes, three products
//   per step, so no offset or rounding of h enters the fp32 accumulation.
// combine (combine_prefill_kernel): out[t] = y_shared[t] + sum_j gate y[inv].
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRows = 32;  // group rows per block (one or two 16-row tiles)

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

// 8 codes of one word -> exact bf16 values in natural column order
__device__ __forceinline__ u32x4_t unpack_exact_bf16(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
  u32x4_t r;
  // integers 0..15 are exact in bf16: the top half of their fp32 pattern
  r.x = (__float_as_uint((float)(ev & 0xFFu)) >> 16) | (__float_as_uint((float)(od & 0xFFu)) & 0xFFFF0000u);
  r.y = (__float_as_uint((float)((ev >> 8) & 0xFFu)) >> 16) |
        (__float_as_uint((float)((od >> 8) & 0xFFu)) & 0xFFFF0000u);
  r.z = (__float_as_uint((float)((ev >> 16) & 0xFFu)) >> 16) |
        (__float_as_uint((float)((od >> 16) & 0xFFu)) & 0xFFFF0000u);
  r.w = (__float_as_uint((float)(ev >> 24)) >> 16) | (__float_as_uint((float)(od >> 24)) & 0xFFFF0000u);
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

// 16-byte slot of (row t, vector v of 8) in a staged [32 rows][8 vectors]
// tile: rows rotate their vectors so that 16 rows read at one v spread over
// the banks
__device__ __forceinline__ int xslot(int t, int v) { return t * 8 + (v ^ (t & 7)); }

// ---------------------------------------------------------------- gate/up
constexpr int kPg = 4;  // groups in flight per wave

struct GluBuf {
  u32x4_t w[4][64];        // (matrix, half): gate lo/hi chunk, up lo/hi; row = lane
  uint32_t m[4][64];       // gate meta, up meta (rows 2, 3: unused copies)
  u32x4_t x[kRows * 8];    // activation pairs of the 32 rows, xslot order
};

struct GluSlot {
  u32x4_t w, x;
  uint32_t m;
};

template <bool F16X, int NM>
__device__ __forceinline__ void glu_body(const PrefillLaunch &p, const Group &g, int nt, int m0,
                                         int nrow, const int *s_tok, const float *s_xs,
                                         GluBuf (&buf)[2], float (*s_h)[65]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = p.D, G = D / 64, F = g.F;
  const int col = lane & 15, kb = lane >> 4;
  const BlobLayout L = blob_layout(D, F);
  // this wave's loads: weight piece (matrix wave/2, half wave%2), meta of
  // matrix wave%2, activation pairs of rows 8 wave .. 8 wave + 7
  const gptr<u32x4_t> wsrc = as_global(
      (const u32x4_t *)(g.blob + ((wave >> 1) ? L.up_codes : L.gate_codes)) + (size_t)(wave & 1) * F +
      nt * 64 + lane);
  const gptr<uint32_t> msrc =
      as_global((const uint32_t *)(g.blob + ((wave & 1) ? L.up_meta : L.gate_meta)) + nt * 64 + lane);
  const int xt = 8 * wave + (lane >> 3), xv = lane & 7;
  const gptr<u32x4_t> xsrc =
      as_global((const u32x4_t *)(p.xp + (size_t)s_tok[xt] * (D / 2)) + xv);
  auto issue = [&](GluSlot &S, int gi) {
    gi = min(gi, G - 1);  // past the end: a repeat of the last group, folded with weight 0
    S.w = wsrc[(size_t)(2 * gi) * F];
    S.m = msrc[(size_t)gi * F];
    S.x = xsrc[gi * 8];
  };
  const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);

  f32x4_t tg[NM], tu[NM];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
    tg[mt] = f32x4_t{0, 0, 0, 0};
    tu[mt] = f32x4_t{0, 0, 0, 0};
  }
  GluSlot ring[kPg];
#pragma unroll
  for (int s = 0; s < kPg; ++s) issue(ring[s], s);
  for (int g0 = 0; g0 < G; g0 += kPg) {
#pragma unroll
    for (int s = 0; s < kPg; ++s) {
      const int gi = g0 + s;
      GluBuf &B = buf[s & 1];
      B.w[wave][lane] = ring[s].w;
      B.m[wave][lane] = ring[s].m;
      B.x[xslot(xt, xv)] = ring[s].x;
      issue(ring[s], gi + kPg);
      __syncthreads();
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
  // h into LDS [row][hidden col of the tile]
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s_h[mt * 16 + kb * 4 + i][wave * 16 + col] = gelu_tanh(tg[mt][i]) * tu[mt][i];
  }
  __syncthreads();
  // three bf16 planes and the 64-unit sum of every valid row
  for (int idx = threadIdx.x; idx < nrow * 64; idx += 256) {
    const int m = idx >> 6, c = idx & 63;
    const float h = s_h[m][c];
    const uint32_t hi = f32_to_bf16(h);
    const float r1 = h - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16(r1);
    const uint32_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    const size_t o = hrow_off(p, g.off + m0 + m) + (size_t)nt * 64 + c;
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
__global__ __launch_bounds__(256) void glu_mfma_kernel(PrefillLaunch p) {
  extern __shared__ float s_dyn[];  // [kRows][G] 64-column sums of x
  __shared__ int s_tok[kRows];
  __shared__ GluBuf buf[2];
  __shared__ float s_h[kRows][65];
  const int NT = p.F / 64;
  const int bid = blockIdx.x;
  const int g_idx = bid < p.E * NT ? bid / NT : p.E;
  const int nt = bid < p.E * NT ? bid - g_idx * NT : bid - p.E * NT;
  const Group g = group_of(p, g_idx);
  const int m0 = blockIdx.y * kRows;
  if (g.count <= m0 || (g.shared && !p.sblobs)) return;
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
    glu_body<F16X, 1>(p, g, nt, m0, nrow, s_tok, s_dyn, buf, s_h);
  else
    glu_body<F16X, 2>(p, g, nt, m0, nrow, s_tok, s_dyn, buf, s_h);
}

// ---------------------------------------------------------------- down
constexpr int kPd = 2;   // hidden groups in flight per wave
constexpr int kDT = 4;   // 16-row output tiles per wave (a block covers 256 output rows)

struct DownBuf {
  u32x4_t pl[3][kRows * 8];   // planes of h for the 32 rows, 64 units, xslot order
  u32x4_t w[2][4 * 64];       // down codes, chunks 2gi and 2gi + 1; row = 64 wave + lane
  uint32_t m[4 * 64];         // scale/bias words of the 256 rows
};

struct DownSlot {
  u32x4_t pl[3];  // plane q of rows 8 wave .. 8 wave + 7
  u32x4_t w[2];   // chunks 2gi, 2gi + 1 of output row 64 wave + lane
  uint32_t m;     // its scale/bias word
};

template <int NM>
__device__ __forceinline__ void down_body(const PrefillLaunch &p, const Group &g, int nb, int m0,
                                          int nrow, const int *s_row, const float *s_hs,
                                          DownBuf (&buf)[2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = p.D, F = g.F, GH = F / 64;
  const int col = lane & 15, kb = lane >> 4;
  const BlobLayout L = blob_layout(D, F);
  const int xt = 8 * wave + (lane >> 3), xv = lane & 7;
  const gptr<u32x4_t> hsrc = as_global((const u32x4_t *)(p.hp + hrow_off(p, s_row[xt])) + xv);
  const size_t plane_v = p.plane / 8;  // plane size in 16-byte vectors
  const int wrow = min(nb * 256 + wave * 64 + lane, D - 1);  // output row this lane loads
  const gptr<u32x4_t> wsrc = as_global((const u32x4_t *)(g.blob + L.down_codes) + wrow);
  const gptr<uint32_t> msrc = as_global((const uint32_t *)(g.blob + L.down_meta) + wrow);
  auto issue = [&](DownSlot &S, int gi) {
    gi = min(gi, GH - 1);  // past the end: a repeat of the last group, folded with weight 0
#pragma unroll
    for (int q = 0; q < 3; ++q) S.pl[q] = hsrc[q * plane_v + gi * 8];
    S.w[0] = wsrc[(size_t)(2 * gi) * D];
    S.w[1] = wsrc[(size_t)(2 * gi + 1) * D];
    S.m = msrc[(size_t)gi * D];
  };

  f32x4_t t[NM][kDT];
#pragma unroll
  for (int mt = 0; mt < NM; ++mt)
#pragma unroll
    for (int j = 0; j < kDT; ++j) t[mt][j] = f32x4_t{0, 0, 0, 0};
  DownSlot ring[kPd];
#pragma unroll
  for (int s = 0; s < kPd; ++s) issue(ring[s], s);
  for (int g0 = 0; g0 < GH; g0 += kPd) {
#pragma unroll
    for (int s = 0; s < kPd; ++s) {
      const int gi = g0 + s;
      DownBuf &B = buf[(gi) & 1];
#pragma unroll
      for (int q = 0; q < 3; ++q) B.pl[q][xslot(xt, xv)] = ring[s].pl[q];
      B.w[0][wave * 64 + lane] = ring[s].w[0];
      B.w[1][wave * 64 + lane] = ring[s].w[1];
      B.m[wave * 64 + lane] = ring[s].m;
      issue(ring[s], gi + kPd);
      __syncthreads();
      const bool live = gi < GH;
      const int gx = min(gi, GH - 1);
#pragma unroll
      for (int j = 0; j < kDT; ++j) {
        // output tile j of this wave: rows 64 wave + 16 j + col
        const int r = wave * 64 + j * 16 + col;
        f32x4_t a[NM];
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) a[mt] = f32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x4_t b = unpack_exact_bf16(((const uint32_t *)&B.w[half][r])[kb]);
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
            const int sl = xslot(mt * 16 + col, half * 4 + kb);
            a[mt] = mfma<false>(B.pl[0][sl], b, a[mt]);
            a[mt] = mfma<false>(B.pl[1][sl], b, a[mt]);
            a[mt] = mfma<false>(B.pl[2][sl], b, a[mt]);
          }
        }
        const uint32_t mw = B.m[r];
        const float sd = live ? f16_to_f32(mw) : 0.0f, bd = live ? f16_to_f32(mw >> 16) : 0.0f;
#pragma unroll
        for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            t[mt][j][i] = fmaf(sd, a[mt][i], fmaf(bd, s_hs[(mt * 16 + kb * 4 + i) * GH + gx], t[mt][j][i]));
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kDT; ++j) {
    const int n = nb * 256 + wave * 64 + j * 16 + col;  // output row of this lane's column
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + kb * 4 + i;
        if (m < nrow && n < D) {
          const int rr = g.off + m0 + m;
          float *dst = rr < p.T * p.k ? p.y + (size_t)rr * D : p.ys + (size_t)(rr - p.T * p.k) * D;
          dst[n] = t[mt][j][i];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void down_mfma_kernel(PrefillLaunch p) {
  __shared__ int s_row[kRows];
  __shared__ float s_hs[kRows * kMaxHGroups];
  __shared__ DownBuf buf[2];
  const int D = p.D, NB = (D + 255) / 256;
  const int bid = blockIdx.x;
  const int g_idx = bid < p.E * NB ? bid / NB : p.E;
  const int nb = bid < p.E * NB ? bid - g_idx * NB : bid - p.E * NB;
  const Group g = group_of(p, g_idx);
  const int m0 = blockIdx.y * kRows;
  if (g.count <= m0 || (g.shared && !p.sblobs)) return;
  const int nrow = min(kRows, g.count - m0);
  const int GH = g.F / 64;
  for (int i = threadIdx.x; i < kRows; i += 256) s_row[i] = g.off + m0 + min(i, nrow - 1);
  __syncthreads();
  for (int i = threadIdx.x; i < kRows * GH; i += 256) {
    const int m = i / GH, gg = i - m * GH;
    s_hs[i] = p.hsum[hrow_off(p, s_row[m]) / 64 + gg];
  }
  __syncthreads();
  if (nrow <= 16)
    down_body<1>(p, g, nb, m0, nrow, s_row, s_hs, buf);
  else
    down_body<2>(p, g, nb, m0, nrow, s_row, s_hs, buf);
}

__global__ void combine_prefill_kernel(PrefillLaunch p) {
  const size_t total = (size_t)p.T * p.D;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t t = i / p.D, d = i - t * p.D;
    float s = p.sblobs ? p.ys[i] : 0.0f;
    for (int j = 0; j < p.k; ++j)
      s = fmaf(p.gates[t * p.k + j], p.y[(size_t)p.inv[t * p.k + j] * p.D + d], s);
    if (p.out_dtype == MOE_F32)
      ((float *)p.out)[i] = s;
    else if (p.out_dtype == MOE_BF16)
      ((uint16_t *)p.out)[i] = (uint16_t)f32_to_bf16(s);
    else
      ((uint16_t *)p.out)[i] = (uint16_t)f32_to_f16(s);
  }
}

}  // namespace

hipError_t launch_prefill_experts(const PrefillLaunch &p, hipStream_t s) {
  if (p.D / 64 > kMaxDGroups || p.F / 64 > kMaxHGroups || p.Fs / 64 > kMaxHGroups)
    return hipErrorInvalidValue;
  const int mchunks = (p.T + kRows - 1) / kRows;
  dim3 g1(p.E * (p.F / 64) + (p.sblobs ? p.Fs / 64 : 0), mchunks);
  const size_t smem = sizeof(float) * kRows * (p.D / 64);
  if (p.f16x)
    hipLaunchKernelGGL(glu_mfma_kernel<true>, g1, dim3(256), smem, s, p);
  else
    hipLaunchKernelGGL(glu_mfma_kernel<false>, g1, dim3(256), smem, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb4 = (p.D + 255) / 256;  // 256 output rows per down block
  dim3 g2(p.E * nb4 + (p.sblobs ? nb4 : 0), mchunks);
  hipLaunchKernelGGL(down_mfma_kernel, g2, dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)p.T * p.D;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(combine_prefill_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
