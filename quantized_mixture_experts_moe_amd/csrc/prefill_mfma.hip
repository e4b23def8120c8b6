// Grouped expert FFN for prefill chunks on the matrix cores.
//
// Prompts are processed in chunks of up to 128 tokens so that one expert
// brought in once serves all of its rows in the chunk (es.news.hada.io,
// "Proceso de generacion de tokens").  After the token -> expert permutation
// each expert's rows form a contiguous group; a group with c rows multiplies
// a c x D activation block by the expert's 4-bit weights, a real (if skinny)
// matrix product, so these kernels use v_mfma_f32_16x16x32_{bf16,f16}.
//
// gate/up (glu_mfma_kernel): block = (expert, 64 hidden rows, 64 group rows).
//   B operand: 4-bit codes OR-ed into the mantissa of 128.0 (bf16; 1024.0 for
//   fp16), exact, in the column order (m, m+4) of a code word; A operand: the
//   activation pairs the router kernel wrote in that same order.  One fp32
//   accumulator per 64-column group; the affine terms fold per group as
//   s * acc + (b - 128 s) * sum(x).
// down (down_mfma_kernel): block = (expert, 64 output rows, 64 group rows).
//   B operand: exact codes (byte spread, v_cvt_f32_ubyte, packed to bf16);
//   A operand: the hidden activations split into three bf16 planes
//   (h = hi + mid + lo to 24 bits), three products per step, so no large
//   offset or rounding of h enters the fp32 accumulation.
// combine (combine_prefill_kernel): out[t] = y_shared[t] + sum_j gate y[inv].
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;  // group rows per block

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

template <bool F16X>
__global__ __launch_bounds__(256) void glu_mfma_kernel(PrefillLaunch p) {
  __shared__ int s_tok[kRows];
  __shared__ float s_xs[kRows][kMaxDGroups];
  __shared__ float s_h[kRows][65];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NT = p.F / 64;
  const int bid = blockIdx.x;
  const int g_idx = bid < p.E * NT ? bid / NT : p.E;
  const int nt = bid < p.E * NT ? bid - g_idx * NT : bid - p.E * NT;
  const Group g = group_of(p, g_idx);
  const int m0 = blockIdx.y * kRows;
  if (g.count <= m0 || (g.shared && !p.sblobs)) return;
  const int nrow = min(kRows, g.count - m0);
  const int nM = (nrow + 15) / 16;
  const int D = p.D, G = D / 64, F = g.F;

  for (int i = threadIdx.x; i < kRows; i += 256) {
    const int m = min(i, nrow - 1);
    s_tok[i] = token_of(p, g, g.off + m0 + m);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kRows * G; i += 256) {
    const int m = i / G, gg = i - m * G;
    s_xs[m][gg] = p.xs[(size_t)s_tok[m] * G + gg];
  }
  __syncthreads();

  const int col = lane & 15, kb = lane >> 4;
  const int n = nt * 64 + wave * 16 + col;  // hidden row of this lane's B column
  const BlobLayout L = blob_layout(D, F);
  const gptr<uint32_t> gc = as_global((const uint32_t *)(g.blob + L.gate_codes) + (size_t)n * 4 + kb);
  const gptr<uint32_t> uc = as_global((const uint32_t *)(g.blob + L.up_codes) + (size_t)n * 4 + kb);
  const gptr<uint32_t> gm = as_global((const uint32_t *)(g.blob + L.gate_meta) + n);
  const gptr<uint32_t> um = as_global((const uint32_t *)(g.blob + L.up_meta) + n);
  const uint32_t magic = opaque_vgpr(Magic<F16X>::bits);
  const uint32_t *xrow[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) xrow[mt] = p.xp + (size_t)s_tok[mt * 16 + col] * (D / 2) + kb * 4;

  f32x4_t tg[4], tu[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    tg[mt] = f32x4_t{0, 0, 0, 0};
    tu[mt] = f32x4_t{0, 0, 0, 0};
  }
  // codes of group gi: chunk 2gi and 2gi + 1 for gate and up; prefetched one group ahead
  uint32_t cw[4], nw[4], cm[2], nm[2];
  auto load_group = [&](uint32_t(&w)[4], uint32_t(&m)[2], int gi) {
    const size_t c0 = (size_t)(2 * gi) * F * 4;
    w[0] = gc[c0];
    w[1] = gc[c0 + (size_t)F * 4];
    w[2] = uc[c0];
    w[3] = uc[c0 + (size_t)F * 4];
    m[0] = gm[(size_t)gi * F];
    m[1] = um[(size_t)gi * F];
  };
  load_group(cw, cm, 0);
  for (int gi = 0; gi < G; ++gi) {
    if (gi + 1 < G) load_group(nw, nm, gi + 1);
    f32x4_t ag[4], au[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      ag[mt] = f32x4_t{0, 0, 0, 0};
      au[mt] = f32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4_t bg = unpack_magic(cw[half], magic);
      const u32x4_t bu = unpack_magic(cw[2 + half], magic);
      const int c = 2 * gi + half;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < nM) {
          const u32x4_t a = *(const u32x4_t *)(xrow[mt] + c * 16);
          ag[mt] = mfma<F16X>(a, bg, ag[mt]);
          au[mt] = mfma<F16X>(a, bu, au[mt]);
        }
      }
    }
    const float sg = f16_to_f32(cm[0]), bgv = f16_to_f32(cm[0] >> 16);
    const float su = f16_to_f32(cm[1]), buv = f16_to_f32(cm[1] >> 16);
    const float cg = fmaf(-Magic<F16X>::offset, sg, bgv), cu = fmaf(-Magic<F16X>::offset, su, buv);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < nM) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xsv = s_xs[mt * 16 + kb * 4 + i][gi];
          tg[mt][i] = fmaf(sg, ag[mt][i], fmaf(cg, xsv, tg[mt][i]));
          tu[mt][i] = fmaf(su, au[mt][i], fmaf(cu, xsv, tu[mt][i]));
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) cw[q] = nw[q];
    cm[0] = nm[0];
    cm[1] = nm[1];
  }
  // h into LDS [row][hidden col of the tile]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < nM) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_h[mt * 16 + kb * 4 + i][wave * 16 + col] = gelu_tanh(tg[mt][i]) * tu[mt][i];
    }
  }
  __syncthreads();
  // three bf16 planes and the 64-unit sum of every valid row
  for (int idx = threadIdx.x; idx < nrow * 64; idx += 256) {
    const int m = idx >> 6, c = idx & 63;
    const int r = g.off + m0 + m;
    const float h = s_h[m][c];
    const uint32_t hi = f32_to_bf16(h);
    const float r1 = h - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16(r1);
    const uint32_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    const size_t o = hrow_off(p, r) + (size_t)nt * 64 + c;
    p.hp[o] = (uint16_t)hi;
    p.hp[p.plane + o] = (uint16_t)mid;
    p.hp[2 * p.plane + o] = (uint16_t)lo;
  }
  if (threadIdx.x < nrow) {
    const int m = threadIdx.x;
    float s = 0.0f;
    for (int c = 0; c < 64; ++c) s += s_h[m][c];
    const int r = g.off + m0 + m;
    p.hsum[hrow_off(p, r) / 64 + nt] = s;
  }
}

__global__ __launch_bounds__(256) void down_mfma_kernel(PrefillLaunch p) {
  __shared__ int s_row[kRows];
  __shared__ float s_hs[kRows][kMaxHGroups];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = p.D, NB = D / 64;
  const int bid = blockIdx.x;
  const int g_idx = bid < p.E * NB ? bid / NB : p.E;
  const int nb = bid < p.E * NB ? bid - g_idx * NB : bid - p.E * NB;
  const Group g = group_of(p, g_idx);
  const int m0 = blockIdx.y * kRows;
  if (g.count <= m0 || (g.shared && !p.sblobs)) return;
  const int nrow = min(kRows, g.count - m0);
  const int nM = (nrow + 15) / 16;
  const int F = g.F, GH = F / 64;

  for (int i = threadIdx.x; i < kRows; i += 256) s_row[i] = g.off + m0 + min(i, nrow - 1);
  __syncthreads();
  for (int i = threadIdx.x; i < kRows * GH; i += 256) {
    const int m = i / GH, gg = i - m * GH;
    s_hs[m][gg] = p.hsum[hrow_off(p, s_row[m]) / 64 + gg];
  }
  __syncthreads();

  const int col = lane & 15, kb = lane >> 4;
  const int n = nb * 64 + wave * 16 + col;  // output row of this lane's B column
  const BlobLayout L = blob_layout(D, F);
  const gptr<uint32_t> dc = as_global((const uint32_t *)(g.blob + L.down_codes) + (size_t)n * 4 + kb);
  const gptr<uint32_t> dm = as_global((const uint32_t *)(g.blob + L.down_meta) + n);
  const uint16_t *arow[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) arow[mt] = p.hp + hrow_off(p, s_row[mt * 16 + col]) + kb * 8;

  f32x4_t t[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) t[mt] = f32x4_t{0, 0, 0, 0};
  uint32_t cw[2], nw[2], cm, nm;
  auto load_group = [&](uint32_t(&w)[2], uint32_t &m, int gi) {
    const size_t c0 = (size_t)(2 * gi) * D * 4;
    w[0] = dc[c0];
    w[1] = dc[c0 + (size_t)D * 4];
    m = dm[(size_t)gi * D];
  };
  load_group(cw, cm, 0);
  for (int gi = 0; gi < GH; ++gi) {
    if (gi + 1 < GH) load_group(nw, nm, gi + 1);
    f32x4_t a[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a[mt] = f32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4_t b = unpack_exact_bf16(cw[half]);
      const int c = 2 * gi + half;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < nM) {
          const uint16_t *ap = arow[mt] + c * 32;
          a[mt] = mfma<false>(*(const u32x4_t *)ap, b, a[mt]);
          a[mt] = mfma<false>(*(const u32x4_t *)(ap + p.plane), b, a[mt]);
          a[mt] = mfma<false>(*(const u32x4_t *)(ap + 2 * p.plane), b, a[mt]);
        }
      }
    }
    const float sd = f16_to_f32(cm), bd = f16_to_f32(cm >> 16);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < nM) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          t[mt][i] = fmaf(sd, a[mt][i], fmaf(bd, s_hs[mt * 16 + kb * 4 + i][gi], t[mt][i]));
      }
    }
    cw[0] = nw[0];
    cw[1] = nw[1];
    cm = nm;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < nM) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + kb * 4 + i;
        if (m < nrow) {
          const int r = g.off + m0 + m;
          float *dst = r < p.T * p.k ? p.y + (size_t)r * D : p.ys + (size_t)(r - p.T * p.k) * D;
          dst[n] = t[mt][i];
        }
      }
    }
  }
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
  if (p.f16x)
    hipLaunchKernelGGL(glu_mfma_kernel<true>, g1, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(glu_mfma_kernel<false>, g1, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(p.E * (p.D / 64) + (p.sblobs ? p.D / 64 : 0), mchunks);
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
