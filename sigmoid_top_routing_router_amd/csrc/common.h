// Device helpers shared by the gfx950 kernels of the MoE layer.
//
// Wave64 reductions use DPP row operations inside each 16-lane row and
// v_readlane across the four rows, so a reduction result is wave-uniform
// (lives in a scalar register).  All reductions must be called with every
// lane of the wave active.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- keys
// Order-preserving map of an fp32 value to uint32: a > b  <=>  key(a) > key(b)
// for finite values.  -0 is folded onto +0 first, so both get the same key.
__device__ __forceinline__ uint32_t f32_order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
  return __uint_as_float(u);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
// Order-preserving 16-bit key of a bf16 pattern (-0 folded onto +0).
// 16-bit order-preserving key of a bfloat16 value b (low 16 bits): zero and
// positive b map to 0x8000 + |b|, negative b to 0x8000 - |b|, so -0 and +0
// share 0x8000.
__device__ __forceinline__ uint32_t bf16_order_key(uint32_t b) {
  const uint32_t m = b & 0x7FFFu;
  return (b & 0x8000u) ? (0x8000u - m) : (0x8000u | m);
}
__device__ __forceinline__ uint32_t bf16_from_order_key(uint32_t k) {
  k &= 0xFFFFu;
  return (k & 0x8000u) ? (k & 0x7FFFu) : (0x8000u | (0x8000u - k));
}
// The keys of two bfloat16 values packed in one word (low and high half), with
// 16-bit packed integer operations: ~b + 1 for negative halves (0x7FFF - |b|
// + 1), b ^ 0x8000 for the others.
__device__ __forceinline__ uint32_t bf16_order_key2(uint32_t p) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
  const s16x2_t sgn = __builtin_bit_cast(s16x2_t, p) >> (short)15;  // 0 or -1 per half
  const uint32_t su = __builtin_bit_cast(uint32_t, sgn);
  const u16x2_t k = __builtin_bit_cast(u16x2_t, p ^ (su | 0x80008000u)) -
                    __builtin_bit_cast(u16x2_t, sgn);
  return __builtin_bit_cast(uint32_t, k);
}

// ---------------------------------------------------------------- DPP
// dpp_ctrl encodings (GCN/CDNA): quad_perm, row_half_mirror, row_mirror.
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadSwap1>(v));
  v = max(v, dpp_u32<kDppQuadSwap2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  uint32_t a = max(readlane_u32(v, 0), readlane_u32(v, 16));
  uint32_t b = max(readlane_u32(v, 32), readlane_u32(v, 48));
  return max(a, b);
}
// Maximum over each DPP row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadSwap1>(v));
  v = max(v, dpp_u32<kDppQuadSwap2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  return max(v, dpp_u32<kDppRowMirror>(v));
}
__device__ __forceinline__ float row16_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuadSwap1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuadSwap2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(v))));
}
__device__ __forceinline__ uint32_t row16_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppQuadSwap1>(v));
  v = min(v, dpp_u32<kDppQuadSwap2>(v));
  v = min(v, dpp_u32<kDppRowHalfMirror>(v));
  return min(v, dpp_u32<kDppRowMirror>(v));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppQuadSwap1>(v));
  v = min(v, dpp_u32<kDppQuadSwap2>(v));
  v = min(v, dpp_u32<kDppRowHalfMirror>(v));
  v = min(v, dpp_u32<kDppRowMirror>(v));
  uint32_t a = min(readlane_u32(v, 0), readlane_u32(v, 16));
  uint32_t b = min(readlane_u32(v, 32), readlane_u32(v, 48));
  return min(a, b);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Inclusive prefix sum over the wave (lane order) with DPP: row_shr 1, 2, 4,
// 8 inside each 16-lane row, then row_bcast15 (lane 15 of a row into the
// next row) and row_bcast31 (lane 31 into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_inclusive_sum_dpp_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

// Inclusive prefix sum over the wave (lane order), shuffle based.
__device__ __forceinline__ uint32_t wave_inclusive_sum_u32(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    uint32_t o = __shfl_up(v, s, kWave);
    if (l >= s) v += o;
  }
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------- routing
// Order key of a biased score z + b with b read as b + 0 (never -0): under
// round to nearest a sum is -0 only when both operands are -0, so no such
// score is -0 and the order-preserving map needs no test for it.
__device__ __forceinline__ uint32_t order_key_nonneg_zero(float v) {
  const uint32_t u = __float_as_uint(v);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// Mixture weight sigma(z) in fp32 (a few ulp); logits below -80, where e^-z
// nears the fp32 range, take the fp64 form.
__device__ __forceinline__ float sigmoid_weight(float z) {
  if (z < -80.0f) return (float)(1.0 / (1.0 + exp(-(double)z)));
  return 1.0f / (1.0f + expf(-z));
}
// Mean of the raw expert biases -q[e], e < E, in fp64 with the terms added
// in expert order ("Kolibri Pre-Training from Scratch" §7.1: the biases are
// centred after the quantile step).  q is in LDS; one thread calls this.
// The reads of 16 terms go ahead of their adds.
__device__ __forceinline__ double raw_bias_mean(const float* q, int E) {
  double acc = 0.0;
  int i = 0;
  for (; i + 16 <= E; i += 16) {
    float b[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) b[j] = q[i + j];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += (double)(-b[j]);
  }
  for (; i < E; ++i) acc += (double)(-q[i]);
  return acc / (double)E;
}
// Highest and lowest set-bit positions (as powers of two) of a nonzero
// finite float.
__device__ __forceinline__ void f32_bit_span(float f, int& top, int& low) {
  const uint32_t b = __float_as_uint(f);
  const int ef = (int)((b >> 23) & 0xFFu);
  const uint32_t m = b & 0x7FFFFFu;
  if (ef == 0) {  // subnormal: m * 2^-149
    top = 31 - __clz((int)m) - 149;
    low = __ffs((int)m) - 1 - 149;
  } else {
    const uint32_t sig = m | 0x800000u;
    top = ef - 127;
    low = ef - 150 + (__ffs((int)sig) - 1);
  }
}
// The same mean, formed by the whole block (BLOCK threads, all of them
// calling).  When every partial sum of the E terms is exact in fp64 (all the
// terms' set bits, and those of any sum of at most 2^9 of them, fit in 53
// bits: top + 10 - low <= 53), the sum does not depend on the order of the
// additions, so a tree over the block gives the bits of the sequential sum;
// otherwise one thread adds them in expert order.  Every partial starts
// from +0, so a zero total is +0 as in the sequential sum.
template <int BLOCK>
__device__ __forceinline__ double block_raw_bias_mean(const float* q, int E) {
  constexpr int W = BLOCK / 64;
  __shared__ double part_s[W];
  __shared__ int top_s[W], low_s[W];
  __shared__ double mean_s;
  double part = 0.0;
  int top = -100000, low = 100000;
  for (int i = (int)threadIdx.x; i < E; i += BLOCK) {
    const float v = -q[i];
    part += (double)v;
    if (v != 0.0f) {
      int t, l;
      f32_bit_span(v, t, l);
      top = max(top, t);
      low = min(low, l);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    part += __shfl_xor(part, o);
    top = max(top, __shfl_xor(top, o));
    low = min(low, __shfl_xor(low, o));
  }
  if ((threadIdx.x & 63) == 0) {
    part_s[threadIdx.x >> 6] = part;
    top_s[threadIdx.x >> 6] = top;
    low_s[threadIdx.x >> 6] = low;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    int t = -100000, l = 100000;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      sum += part_s[w];
      t = max(t, top_s[w]);
      l = min(l, low_s[w]);
    }
    const bool exact = t < -99999 || t + 10 - l <= 53;
    mean_s = exact ? sum / (double)E : raw_bias_mean(q, E);
  }
  __syncthreads();
  return mean_s;
}
// Grid-stride clear of n words (a buffer that later kernels accumulate into),
// ahead of a kernel's own work.
// BLOCK is the launch's block size (a constant, so that no load of the
// dispatch packet's block size stands in front of the kernel's own loads).
template <int BLOCK>
__device__ __forceinline__ void clear_words(uint32_t* __restrict__ p, int64_t n) {
  if (!p) return;
  const int64_t stride = (int64_t)gridDim.x * BLOCK;
  for (int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

// ---------------------------------------------------------------- MFMA types
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

}  // namespace moe
