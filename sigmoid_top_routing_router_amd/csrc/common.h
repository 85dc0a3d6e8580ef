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

// ---------------------------------------------------------------- MFMA types
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

}  // namespace moe
