// FP8 (E4M3) quantisation of weights and activations.
//
// "Kolibri 1 im Detail", section on the FP8 path: linear weights are stored
// as E4M3 in 128 x 128 blocks with one fp32 scale per block; activations are
// quantised dynamically in groups of 1 x 128.  The pages fix the format but
// not the scale; here s = fp32(amax) / 448 (448 being the largest E4M3
// value), and each value becomes the E4M3 code of fp32(v / s) clamped to
// +-448, rounded to nearest even by the hardware conversion
// (v_cvt_pk_fp8_f32).  An all-zero group gets s = 0 and zero codes.
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

// One wave per (row, group of 128): lane l holds elements 2l, 2l+1.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ X,
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
  // |v| as bits: the order of non-negative floats is the order of their bits
  const uint32_t m = wave_max_u32(max(__float_as_uint(fabsf(a)), __float_as_uint(fabsf(b))));
  const float amax = __uint_as_float(m);
  const float s = amax / kE4M3Max;
  uint32_t codes = 0;
  if (amax != 0.0f) codes = fp8x2(quant_input(a, s), quant_input(b, s));
  *reinterpret_cast<uint16_t*>(Q + n * C + g * 128 + 2 * lane) = (uint16_t)codes;
  if (lane == 0) S[n * groups + g] = (amax != 0.0f) ? s : 0.0f;
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
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max(w[i] << 17 >> 1, w[i] & 0x7FFF0000u));
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
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      uint32_t lo = 0, hi = 0;
      if (amax != 0.0f) {
        lo = fp8x2(quant_input(bf16_to_f32(w[0] & 0xFFFFu), s), quant_input(bf16_to_f32(w[0] >> 16), s)) |
             (fp8x2(quant_input(bf16_to_f32(w[1] & 0xFFFFu), s), quant_input(bf16_to_f32(w[1] >> 16), s)) << 16);
        hi = fp8x2(quant_input(bf16_to_f32(w[2] & 0xFFFFu), s), quant_input(bf16_to_f32(w[2] >> 16), s)) |
             (fp8x2(quant_input(bf16_to_f32(w[3] & 0xFFFFu), s), quant_input(bf16_to_f32(w[3] >> 16), s)) << 16);
      }
      *reinterpret_cast<uint2*>(Qm + (int64_t)r * C + c0 + 8 * j) = make_uint2(lo, hi);
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
  const int64_t waves = N * (C / 128);
  if (waves <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream,
                     X, N, C, Q, S);
  return hipGetLastError();
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
