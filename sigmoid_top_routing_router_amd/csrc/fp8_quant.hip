// FP8 (E4M3) quantisation of weights and activations.
//
// "Kolibri 1 im Detail", section on the FP8 path: linear weights are stored
// as E4M3 in 128 x 128 blocks with one fp32 scale per block; activations are
// quantised dynamically in groups of 1 x 128.  The pages fix the format but
// not the scale; here s = fp32(amax) / 448 (448 being the largest E4M3
// value), and each value becomes the E4M3 code of fp32(v / s) clamped to
// +-448, rounded to nearest even by the hardware conversion
// (v_cvt_pk_fp8_f32).  An all-zero group gets s = 0 and zero codes.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 values -> two E4M3 codes in the low 16 bits (first value low).
__device__ __forceinline__ uint32_t fp8x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float quant_input(float v, float s) {
  return fminf(fmaxf(v / s, -kE4M3Max), kE4M3Max);
}

// Inputs not aligned for 16-byte loads: one wave per (row, group of 128),
// lane l holds elements 2l, 2l+1.
__global__ __launch_bounds__(256) void quant_rows_wave_kernel(const uint16_t* __restrict__ X,
                                                              int64_t N, int C,
                                                              uint8_t* __restrict__ Q,
                                                              float* __restrict__ S) {
  const int groups = C / 128;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= N * groups) return;
  const int lane = lane_id();
  const int64_t n = wid / groups;
  const int g = (int)(wid % groups);
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(X + n * C + g * 128 + 2 * lane);
  const float a = bf16_to_f32((uint16_t)(pair & 0xFFFFu));
  const float b = bf16_to_f32((uint16_t)(pair >> 16));
  const uint32_t m = wave_max_u32(max(__float_as_uint(fabsf(a)), __float_as_uint(fabsf(b))));
  const float amax = __uint_as_float(m);
  const float s = amax / kE4M3Max;
  uint32_t codes = 0;
  if (amax != 0.0f) codes = fp8x2(quant_input(a, s), quant_input(b, s));
  *reinterpret_cast<uint16_t*>(Q + n * C + g * 128 + 2 * lane) = (uint16_t)codes;
  if (lane == 0) S[n * groups + g] = (amax != 0.0f) ? s : 0.0f;
}

// Eight bf16 (one 16-byte word) -> their eight E4M3 codes under scale s.
__device__ __forceinline__ uint2 quant8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c[i] = fp8x2(quant_input(bf16_to_f32(w[i] & 0xFFFFu), s), quant_input(bf16_to_f32(w[i] >> 16), s));
  return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

// |v| of the eight bf16 in v, widened to fp32 bits, maximum of them (the order
// of non-negative floats is the order of their bits).
__device__ __forceinline__ uint32_t abs_max8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] << 17 >> 1, w[i] & 0x7FFF0000u));
  return m;
}

// Rows are contiguous and C % 128 == 0, so the matrix is a run of 16-byte
// words in which every 16 consecutive words form one (row, group of 128).
// Each DPP row of 16 lanes takes one group: lane l holds elements 8l..8l+7 of
// it and stores their codes as one 8-byte word; the group's maximum is a
// 16-lane DPP reduction.  (Two or four words per thread measured no faster.)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void quant_rows_kernel(const u32x4_t* __restrict__ X,
                                                         int64_t words,
                                                         uint2* __restrict__ Q,
                                                         float* __restrict__ S) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // words % 16 == 0 and blocks start on 16-word boundaries: a DPP row is
  // wholly in range or wholly out of it
  if (w >= words) return;
  const u32x4_t t = __builtin_nontemporal_load(X + w);
  const uint4 v = make_uint4(t.x, t.y, t.z, t.w);
  const float amax = __uint_as_float(row16_max_u32(abs_max8(v)));
  const float s = amax / kE4M3Max;
  Q[w] = (amax != 0.0f) ? quant8(v, s) : make_uint2(0, 0);
  if ((threadIdx.x & 15) == 0) S[w >> 4] = (amax != 0.0f) ? s : 0.0f;
}

// One block of 256 threads per 128 x 128 tile of one matrix: thread t takes
// row t/2 of the tile, 64 columns.  VEC: C % 8 == 0 and W 16-byte aligned, so
// the 64 columns move as 16-byte loads (eight bf16) and 8-byte code stores;
// otherwise element by element.
template <bool VEC>
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint16_t* __restrict__ W,
                                                           int R, int C,
                                                           uint8_t* __restrict__ Q,
                                                           float* __restrict__ S) {
  __shared__ uint32_t wmax[4];
  const int nbr = (R + 127) / 128, nbc = (C + 127) / 128;
  const int64_t mat = blockIdx.z;
  const int br = blockIdx.y, bc = blockIdx.x;
  const uint16_t* Wm = W + mat * (int64_t)R * C;
  uint8_t* Qm = Q + mat * (int64_t)R * C;
  const int r = br * 128 + (threadIdx.x >> 1);
  const int c0 = bc * 128 + (threadIdx.x & 1) * 64;
  uint32_t m = 0;
  uint4 v[8];
  if (VEC) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = r < R && c0 + 8 * j < C;
      v[j] = in ? *reinterpret_cast<const uint4*>(Wm + (int64_t)r * C + c0 + 8 * j)
                : make_uint4(0, 0, 0, 0);
      m = max(m, abs_max8(v[j]));
    }
  } else if (r < R) {
    for (int j = 0; j < 64 && c0 + j < C; ++j)
      m = max(m, __float_as_uint(fabsf(bf16_to_f32(Wm[(int64_t)r * C + c0 + j]))));
  }
  m = wave_max_u32(m);
  if (lane_id() == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = __uint_as_float(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  const float s = amax / kE4M3Max;
  if (VEC) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!(r < R && c0 + 8 * j < C)) continue;
      *reinterpret_cast<uint2*>(Qm + (int64_t)r * C + c0 + 8 * j) =
          (amax != 0.0f) ? quant8(v[j], s) : make_uint2(0, 0);
    }
  } else if (r < R) {
    for (int j = 0; j < 64 && c0 + j < C; j += 2) {
      const float a = bf16_to_f32(Wm[(int64_t)r * C + c0 + j]);
      const bool two = c0 + j + 1 < C;
      const float b = two ? bf16_to_f32(Wm[(int64_t)r * C + c0 + j + 1]) : 0.0f;
      const uint32_t codes = (amax != 0.0f) ? fp8x2(quant_input(a, s), quant_input(b, s)) : 0u;
      Qm[(int64_t)r * C + c0 + j] = (uint8_t)(codes & 0xFFu);
      if (two) Qm[(int64_t)r * C + c0 + j + 1] = (uint8_t)(codes >> 8);
    }
  }
  if (threadIdx.x == 0) S[(mat * nbr + br) * nbc + bc] = (amax != 0.0f) ? s : 0.0f;
}

hipError_t launch_quant_rows(const uint16_t* X, int64_t N, int C, uint8_t* Q, float* S,
                             hipStream_t stream) {
  if (N <= 0 || C <= 0) return hipSuccess;
  if (C % 128 != 0) return hipErrorInvalidValue;
  const bool vec = (uintptr_t)X % 16 == 0 && (uintptr_t)Q % 8 == 0;
  // at most 2^30 16-byte words (16 GiB of x) per launch keeps the grid in range
  const int64_t rows_per = std::max<int64_t>(1, (int64_t(1) << 30) / (C / 8));
  for (int64_t r0 = 0; r0 < N; r0 += rows_per) {
    const int64_t n = std::min(rows_per, N - r0);
    const uint16_t* x = X + r0 * C;
    uint8_t* q = Q + r0 * C;
    float* sc = S + r0 * (C / 128);
    if (vec) {
      const int64_t words = n * C / 8;
      hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                         stream, reinterpret_cast<const u32x4_t*>(x), words,
                         reinterpret_cast<uint2*>(q), sc);
    } else {
      const int64_t waves = n * (C / 128);
      hipLaunchKernelGGL(quant_rows_wave_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                         stream, x, n, C, q, sc);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quant_blocks(const uint16_t* W, int64_t count, int R, int C, uint8_t* Q,
                               float* S, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 127) / 128), (unsigned)((R + 127) / 128), (unsigned)count);
  if (C % 8 == 0 && (uintptr_t)W % 16 == 0 && (uintptr_t)Q % 8 == 0)
    hipLaunchKernelGGL(quant_blocks_kernel<true>, grid, dim3(256), 0, stream, W, R, C, Q, S);
  else
    hipLaunchKernelGGL(quant_blocks_kernel<false>, grid, dim3(256), 0, stream, W, R, C, Q, S);
  return hipGetLastError();
}

}  // namespace moe
