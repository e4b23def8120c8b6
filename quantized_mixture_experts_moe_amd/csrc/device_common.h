// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __uint_as_float((bits & 0xFFFFu) << 16);
}
// Round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two-element dot product with fp32 accumulation: v_dot2c_f32_{bf16,f16}.
template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <>
__device__ __forceinline__ float dot2<false>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
template <>
__device__ __forceinline__ float dot2<true>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                c, false);
}

// Global-address-space views: loads through them are global_load (not flat).
template <class T>
using gptr = const __attribute__((address_space(1))) T *;
template <class T>
__device__ __forceinline__ gptr<T> as_global(const T *p) {
  return (gptr<T>)(p);
}

// A register holding v with its value hidden from the optimiser, so that the
// mask-and-insert of the code unpacking stays one v_and_or_b32 (gfx9 VOP3
// takes no literal operand).
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// 4-bit codes to a pair of 16-bit floats without a conversion instruction:
// OR-ing a nibble into the mantissa of 128.0 (bf16 0x4300) gives 128 + q
// exactly; for fp16 the base is 1024.0 (0x6400).  Word w holds the codes of 8
// consecutive columns, nibble i = column i; (w >> 4m) & 0x000F000F selects
// columns m and m + 4, so the activation pairs are (x[m], x[m + 4]).
template <bool F16>
struct Magic;
template <>
struct Magic<false> {
  static constexpr uint32_t bits = 0x43004300u;
  static constexpr float offset = 128.0f;
};
template <>
struct Magic<true> {
  static constexpr uint32_t bits = 0x64006400u;
  static constexpr float offset = 1024.0f;
};

// sum over the 32 columns of one 16-byte chunk of (offset + q) * x, with the
// activation pairs xw[i * 4 + m] = (x[8i + m], x[8i + m + 4]).
template <bool F16>
__device__ __forceinline__ float dot_chunk(const u32x4 q, const uint32_t *xw, float acc,
                                           uint32_t magic) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t qp = ((w[i] >> (4 * m)) & 0x000F000Fu) | magic;
      acc = dot2<F16>(xw[i * 4 + m], qp, acc);
    }
  }
  return acc;
}

// Same with the activation split as hi + lo bf16 halves: xw[i*8 + m] are the
// hi pairs, xw[i*8 + 4 + m] the lo pairs of word i.
__device__ __forceinline__ float dot_chunk_hilo(const u32x4 q, const uint32_t *xw, float acc,
                                                uint32_t magic) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t qp = ((w[i] >> (4 * m)) & 0x000F000Fu) | magic;
      acc = dot2<false>(xw[i * 8 + m], qp, acc);
      acc = dot2<false>(xw[i * 8 + 4 + m], qp, acc);
    }
  }
  return acc;
}

// Matrix-core product v_mfma_f32_16x16x32_{bf16,f16}: D = A B + C with
// A[row l % 16][k 8 (l / 16) + j], B[k 8 (l / 16) + j][col l % 16] (8 16-bit
// values per lane in 4 registers, value j in half j % 2 of register j / 2)
// and D[row 4 (l / 16) + i][col l % 16] in register i.
typedef __bf16 mma_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mma_f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <bool F16>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mma_f16x8, a),
                                                  __builtin_bit_cast(mma_f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mma_bf16x8, a),
                                                   __builtin_bit_cast(mma_bf16x8, b), c, 0, 0,
                                                   0);
}

// The 8 codes of one word as 16-bit pairs (offset + q_m, offset + q_{m+4}),
// m = 0..3 (magic 0x43004300: bf16 128 + q; 0x64006400: fp16 1024 + q).
__device__ __forceinline__ u32x4 code_pairs(uint32_t w, uint32_t magic) {
  u32x4 r;
  r.x = (w & 0x000F000Fu) | magic;
  r.y = ((w >> 4) & 0x000F000Fu) | magic;
  r.z = ((w >> 8) & 0x000F000Fu) | magic;
  r.w = ((w >> 12) & 0x000F000Fu) | magic;
  return r;
}
// The same pairs as bf16 1 + q / 16 (the nibble in mantissa bits 3..6 of
// 1.0): a small offset, for products whose other factor has a large mean.
__device__ __forceinline__ u32x4 code_pairs_unit(uint32_t w, uint32_t magic) {
  u32x4 r;
  r.x = ((w << 3) & 0x00780078u) | magic;
  r.y = ((w >> 1) & 0x00780078u) | magic;
  r.z = ((w >> 5) & 0x00780078u) | magic;
  r.w = ((w >> 9) & 0x00780078u) | magic;
  return r;
}

// View of global memory through the constant address space: wave-uniform
// loads through it become scalar loads into SGPRs.  Only for data written by
// an earlier kernel (the scalar cache does not see stores of the same kernel).
template <class T>
using const_ptr = const __attribute__((address_space(4))) T *;
template <class T>
__device__ __forceinline__ const_ptr<T> as_const(const T *p) {
  return (const_ptr<T>)(p);
}

// Copy N wave-uniform words into registers (scalar loads).
template <int N>
__device__ __forceinline__ void load_uniform(const uint32_t *src, uint32_t (&dst)[N]) {
  const_ptr<uint32_t> p = as_const(src);
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = p[i];
}

// Device-coherent handoff between blocks without a full-cache fence: the
// producer writes with device-scope stores (they bypass the XCD-private L2),
// waits for them to complete, then bumps a counter with a device-scope atomic;
// a consumer that sees the count reads with device-scope loads.
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t *p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// all outstanding memory operations of this wave have completed
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Sum over 64 codes (two chunks) of q * h with fp32 products: the codes are
// spread to bytes and converted exactly (v_cvt_f32_ubyte*), h is fp32 and
// wave-uniform.  Word i of chunk c holds columns 8i..8i+7 of the chunk.
__device__ __forceinline__ float dot_group_f32(const u32x4 q0, const u32x4 q1, const float *h) {
  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ev = w[i] & 0x0F0F0F0Fu;         // columns 8i, 8i+2, 8i+4, 8i+6
    const uint32_t od = (w[i] >> 4) & 0x0F0F0F0Fu;  // columns 8i+1, 8i+3, 8i+5, 8i+7
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc = fmaf((float)((ev >> (8 * b)) & 0xFFu), h[8 * i + 2 * b], acc);
      acc = fmaf((float)((od >> (8 * b)) & 0xFFu), h[8 * i + 2 * b + 1], acc);
    }
  }
  return acc;
}

// Deterministic reduction over the splits of a tile (wave-wide, R rows of 64
// values).  Each split adds its partials, rounded to multiples of 2^-32, into
// 64-bit integer accumulators with device-scope atomics; integer addition
// gives the same sum in any arrival order, so results are bitwise
// reproducible.  After its adds have completed, each split bumps the tile's
// counter; the split that arrives last reads the sums into out[] (returns
// true) and puts the accumulators and the counter back to zero, so they are
// zero between calls.  The rounding is 2^-33 per partial; sums must stay
// below 2^31 in magnitude, and a partial that could break that bumps *err.
__device__ __forceinline__ long long to_fixed32(float v) {
  return __double2ll_rn((double)v * 4294967296.0);
}
__device__ __forceinline__ float from_fixed32(long long a) {
  return (float)((double)a * (1.0 / 4294967296.0));
}
template <int R>
__device__ __forceinline__ bool split_reduce_fixed(uint64_t *acc, uint32_t *counter, int nsplits,
                                                   const float (&v)[R], float (&out)[R],
                                                   uint32_t *err) {
  const int lane = threadIdx.x & 63;
  // a partial outside |v| < 2^31 / nsplits (or not finite) could wrap the
  // sum: counted as an error of the call
  bool range_ok = true;
#pragma unroll
  for (int r = 0; r < R; ++r) range_ok = range_ok && fabsf(v[r]) * (float)nsplits < 2147483648.0f;
  if (!range_ok) add_dev(err, 1u);
#pragma unroll
  for (int r = 0; r < R; ++r)
    __hip_atomic_fetch_add(acc + r * 64 + lane, (uint64_t)to_fixed32(v[r]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  wait_all_memory();
  uint32_t old = 0;
  if (lane == 0) old = add_dev(counter, 1u);
  old = __shfl(old, 0, 64);
  if (old != (uint32_t)(nsplits - 1)) return false;
#pragma unroll
  for (int r = 0; r < R; ++r) out[r] = from_fixed32((long long)ld_dev(acc + r * 64 + lane));
  wait_all_memory();
#pragma unroll
  for (int r = 0; r < R; ++r) st_dev(acc + r * 64 + lane, (uint64_t)0);
  if (lane == 0) st_dev(counter, 0u);
  return true;
}

template <int N>
__device__ __forceinline__ void load_uniform_f(const float *src, float (&dst)[N]) {
  const_ptr<float> p = as_const(src);
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = p[i];
}

// Wave-wide reductions through DPP row operations (no LDS round trips).  The
// combination order is fixed, so results are bitwise reproducible; every lane
// receives lane 63's total.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v, float identity) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, identity),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v, int identity) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xF, false);
}
// quad_perm xor 1, xor 2; row_half_mirror; row_mirror; row_bcast15; row_bcast31
#define MOE_DPP_REDUCE(T, v, op, id, dpp)                 \
  v = op(v, dpp<0xB1>(v, id));                            \
  v = op(v, dpp<0x4E>(v, id));                            \
  v = op(v, dpp<0x141>(v, id));                           \
  v = op(v, dpp<0x140>(v, id));                           \
  v = op(v, dpp<0x142, 0xA>(v, id));                      \
  v = op(v, dpp<0x143, 0xC>(v, id));

__device__ __forceinline__ float f_add(float a, float b) { return a + b; }
__device__ __forceinline__ int i_min(int a, int b) { return a < b ? a : b; }

__device__ __forceinline__ float wave_sum(float v) {
  MOE_DPP_REDUCE(float, v, f_add, 0.0f, dpp_f32)
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// ---------------------------------------------------------------- RMSNorm of the residual block
// Every kernel that normalises a row sums its squares in one fixed order, so
// fused and separate paths give the same bits: the row is read as chunks of
// 8 columns; thread t of 256 squares and adds chunks t, t + 256, ... in
// column order (fmaf from 0); each wave of 64 threads sums its lanes with
// wave_sum; the four wave sums are added in wave order.  The normalised
// value is (v * inv) * (1 + w) with inv = 1 / sqrt(sum / D + eps).
constexpr int kNormThreads = 256;
__device__ __forceinline__ float sumsq8(const float (&v)[8], float acc) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc = fmaf(v[m], v[m], acc);
  return acc;
}
__device__ __forceinline__ float norm_inv(float sumsq, int D, float eps) {
  return 1.0f / sqrtf(sumsq / (float)D + eps);
}
__device__ __forceinline__ float norm_scale(float v, float inv, float w) {
  return v * inv * (1.0f + w);
}
// The sum by one wave standing in for the 256 threads: lane l plays threads
// l, l + 64, l + 128, l + 192.  load(c, v) reads chunk c into v[8].
template <class Load>
__device__ __forceinline__ float row_sumsq_wave(int nch, Load load) {
  const int lane = threadIdx.x & 63;
  float tot = 0.0f;
#pragma unroll
  for (int s = 0; s < kNormThreads / 64; ++s) {
    float p = 0.0f;
    for (int c = s * 64 + lane; c < nch; c += kNormThreads) {
      float v[8];
      load(c, v);
      p = sumsq8(v, p);
    }
    tot += wave_sum(p);
  }
  return tot;
}
// The sum by a block of 256 threads, from each thread's own partial (chunks
// t, t + 256, ...).  red4: 4 floats of LDS, read back after a barrier.
__device__ __forceinline__ float row_sumsq_block(float p, float *red4) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float w = wave_sum(p);
  if (lane == 0) red4[wave] = w;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int s = 0; s < kNormThreads / 64; ++s) tot += red4[s];
  return tot;
}
template <bool F16X>
__device__ __forceinline__ float act_to_f32(uint32_t bits) {
  return F16X ? f16_to_f32(bits) : bf16_to_f32(bits);
}
template <bool F16X>
__device__ __forceinline__ uint32_t f32_to_act(float v) {
  return F16X ? f32_to_f16(v) : f32_to_bf16(v);
}
// the 8 values of a chunk of 16-bit activations (column order)
template <bool F16X>
__device__ __forceinline__ void unpack8(const u32x4 q, float (&v)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    v[2 * m] = act_to_f32<F16X>(w[m] & 0xFFFFu);
    v[2 * m + 1] = act_to_f32<F16X>(w[m] >> 16);
  }
}
// u of a chunk: the normalised values rounded to the activation type
template <bool F16X>
__device__ __forceinline__ u32x4 norm_chunk(const u32x4 q, float inv, const float4 w0,
                                            const float4 w1) {
  float v[8];
  unpack8<F16X>(q, v);
  const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f32_to_act<F16X>(norm_scale(v[m], inv, w[m]));
  return u32x4{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
               o[6] | (o[7] << 16)};
}

__device__ __forceinline__ float wave_max(float v) {
  MOE_DPP_REDUCE(float, v, fmaxf, -INFINITY, dpp_f32)
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ int wave_min(int v) {
  MOE_DPP_REDUCE(int, v, i_min, 0x7FFFFFFF, dpp_i32)
  return __builtin_amdgcn_readlane(v, 63);
}

// Sum of 64 values of which each of 8 consecutive lanes (8q .. 8q + 7) holds
// the in-order sum of 8: the lanes combine through DPP as
// ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7)); all 8 lanes receive the
// total.  The 64-column activation sums of the 4-bit kernels use this order
// everywhere, so every path gets the same bits.
__device__ __forceinline__ float sum8_lanes(float v) {
  v = v + dpp_f32<0xB1>(v, 0.0f);   // quad_perm [1, 0, 3, 2]
  v = v + dpp_f32<0x4E>(v, 0.0f);   // quad_perm [2, 3, 0, 1]
  v = v + dpp_f32<0x141>(v, 0.0f);  // row_half_mirror
  return v;
}

// Order-preserving map of a float to an unsigned key (larger float, larger
// key); -0 maps like +0, so equal floats get equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int u_max(int a, int b) {
  return (int)((uint32_t)a > (uint32_t)b ? (uint32_t)a : (uint32_t)b);
}
// wave-wide maximum of unsigned values (every lane receives it)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  int v = (int)x;
  MOE_DPP_REDUCE(int, v, u_max, 0, dpp_i32)
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Top-k of one token's logits held by one wave, by k rounds of a wave-wide
// maximum: v[j] is the logit of expert lane + 64 j (-inf or skipped beyond
// E).  Round r takes the largest remaining order-preserving key, the lowest
// expert index among equal keys, so the result is the descending order with
// ties to the lower index.  Lane r < k receives the r-th expert's id and
// logit; no LDS and no barrier.
template <int NV>
__device__ __forceinline__ void topk_rounds(const float (&v)[NV], int E, int k, int32_t *id_out,
                                            float *val_out) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) key[j] = lane + 64 * j < E ? order_key(v[j]) : 0u;  // 0: below all
  int32_t my_id = 0;
  uint32_t my_key = 0u;
  for (int r = 0; r < k; ++r) {
    uint32_t m = key[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) m = m > key[j] ? m : key[j];
    m = wave_max_u32(m);
    int win = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint64_t b = __ballot(key[j] == m);
      if (!found && b) {
        win = 64 * j + (int)__builtin_ctzll(b);
        found = true;
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (win == lane + 64 * j) key[j] = 0u;
    if (lane == r) {
      my_id = win;
      my_key = m;
    }
  }
  *id_out = my_id;
  *val_out = key_value(my_key);
}

// Top-k of one token's logits held by one wave, v[j] = logit of expert
// lane + 64 j (-inf beyond E): larger first, equal logits to the lower index
// (topk_rounds; the -inf entries rank last and k <= E never reaches them).
// Lane r < k receives the r-th id and its softmax gate over the k selected
// logits: max = the rank-0 logit, exp of the differences, a DPP wave sum, a
// division -- every selection in the library uses this arithmetic, so they
// all give the same bits.  xch is unused (kept for the callers' layout).
template <int NV>
__device__ __forceinline__ void topk_regs(float (&v)[NV], int k, uint2 *xch, int32_t *id_out,
                                          float *gate_out) {
  (void)xch;
  const int lane = threadIdx.x & 63;
  int32_t myi;
  float myv;
  topk_rounds(v, 64 * NV, k, &myi, &myv);
  if (lane >= k) myv = 0.0f;
  const float m0 =
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, myv), 0));
  const float z = lane < k ? expf(myv - m0) : 0.0f;
  const float sum = wave_sum(z);
  *id_out = lane < k ? myi : 0;
  *gate_out = z / sum;
}

__device__ __forceinline__ float gelu_tanh(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

}  // namespace moe
