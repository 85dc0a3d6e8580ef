// Weighted combine of the expert outputs and small utility kernels.
//
// "Kolibri Pre-Training from Scratch" §6.1: y_t = f_shared(x_t) +
// sum_{e in I_t} S_{t,e} f_e(x_t), with the unbiased, unnormalised sigmoid
// weights.  The routed expert outputs sit in expert-grouped order (row
// src_pos[t,k] holds f_{I_tk}(x_t)); each thread owns 8 consecutive columns
// of one token, issues the K gathered 16-byte loads at once (K is a
// compile-time constant, 1..8), accumulates in fp32 in the token's slot order
// on top of the shared expert's output and writes bf16 (round to nearest
// even).  Expert outputs are read once, so they are loaded non-temporally.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt16(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int K>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint16_t* __restrict__ sh, const uint16_t* __restrict__ Y,
    const float* __restrict__ S, const int32_t* __restrict__ src_pos, int64_t N, int d,
    uint16_t* __restrict__ y) {
  const int cpr = d / 8;  // 16-byte chunks per row
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * cpr) return;
  const int64_t t = i / cpr;
  const int c = (int)(i % cpr) * 8;
  // all K gathered rows in flight before any arithmetic
  float w[K];
  uint4 v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    w[k] = S[t * K + k];
    const int64_t p = src_pos[t * K + k];
    v[k] = load_nt16(Y + p * d + c);
  }
  float acc[8];
  if (sh) {
    bf16x8_to_f32(load_nt16(sh + t * d + c), acc);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float f[8];
    bf16x8_to_f32(v[k], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += w[k] * f[j];
  }
  uint4 o;
  o.x = f32_to_bf16_rne_bits(acc[0]) | (f32_to_bf16_rne_bits(acc[1]) << 16);
  o.y = f32_to_bf16_rne_bits(acc[2]) | (f32_to_bf16_rne_bits(acc[3]) << 16);
  o.z = f32_to_bf16_rne_bits(acc[4]) | (f32_to_bf16_rne_bits(acc[5]) << 16);
  o.w = f32_to_bf16_rne_bits(acc[6]) | (f32_to_bf16_rne_bits(acc[7]) << 16);
  *reinterpret_cast<uint4*>(y + t * d + c) = o;
}

hipError_t launch_combine(const uint16_t* sh, const uint16_t* Y, const float* S,
                          const int32_t* src_pos, int64_t N, int K, int d, uint16_t* y,
                          hipStream_t stream) {
  const int64_t total = N * (int64_t)(d / 8);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  switch (K) {
#define MOE_COMBINE_CASE(KK)                                                            \
    case KK:                                                                            \
      hipLaunchKernelGGL(combine_kernel<KK>, grid, block, 0, stream, sh, Y, S, src_pos, N, \
                         d, y);                                                         \
      break;
    MOE_COMBINE_CASE(1) MOE_COMBINE_CASE(2) MOE_COMBINE_CASE(3) MOE_COMBINE_CASE(4)
    MOE_COMBINE_CASE(5) MOE_COMBINE_CASE(6) MOE_COMBINE_CASE(7) MOE_COMBINE_CASE(8)
#undef MOE_COMBINE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v,
                                                       size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, value, n);
  return hipGetLastError();
}

}  // namespace moe
