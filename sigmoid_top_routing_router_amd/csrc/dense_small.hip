// Dense products of small batches: the router logits and the shared expert's
// projections for N <= 64 tokens ("Kolibri 1 im Detail", routing section:
// x W_r^T in fp32, the SwiGLU expert; FP8 section for the E4M3 variant).
//
// For such a batch each product only has to read its weight matrix once
// (router 2 MB, shared expert 7.9 MB at the Kolibri shape), but a 256 x 256
// tile grid gives it just a handful of blocks.  Here the work is split over
// 64-row blocks of the weight matrix and 256-wide chunks of k (split-K), so a
// product runs on 60-160 blocks, each reading 32 KB of weights straight into
// its MFMA operand registers:
//  * wave w of a block multiplies 16 weight rows with all tokens (16 per MFMA
//    block): bf16 v_mfma_f32_16x16x32_bf16, E4M3 v_mfma_f32_16x16x128_f8f6f4
//    whose product is scaled by s_W(block, kb) * s_x(token, kb) and added in
//    fp32; weights are the first operand, so lane l holds token (l & 15) and
//    four consecutive weight rows;
//  * all loads of a block are issued before its first multiply (one round
//    trip per block);
//  * each block writes fp32 partial sums [chunk][token][row]; a second kernel
//    adds the chunks in a fixed order (deterministic) and applies the
//    epilogue: router + offset (fp32), SiLU(g) * u in bf16 or quantised to
//    E4M3 per 1 x 128 group, or the bf16 down projection.
// The rows of the gate/up product are the hs gate rows followed by the hs up
// rows.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 64;  // weight rows per block (4 waves x 16)
constexpr int kChunkK = 256;       // k per block (split-K chunk)

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct DenseSmallArgs {
  const char* A;        // activations [N][kdim] (bf16 or E4M3 codes)
  const float* sa;      // E4M3: activation scales [N][kdim/128]
  int64_t N;
  int kdim;
  const char* B0;       // weight rows 0 .. R0-1, [R0][kdim]
  const char* B1;       // weight rows R0 .. R-1 (the up projection) or NULL
  const float* sb0;     // E4M3: block scales of B0 [R0/128][kdim/128]
  const float* sb1;     // E4M3: block scales of B1
  int R0, R;            // rows of B0, rows in all
  float* part;          // [chunks][N][R] fp32 partial sums
};

template <bool FP8, int NB>
__global__ __launch_bounds__(256) void dense_small_kernel(DenseSmallArgs a) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 128 : 32;   // k per MFMA
  constexpr int NKS = kChunkK / KSTEP;    // MFMA k-steps per chunk
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int fr = lane & 15, q = lane >> 4;
  const int r0 = blockIdx.x * kRowsPerBlock + wave * 16;  // first row of this wave
  if (r0 >= a.R) return;                                   // (no barriers below)
  const int kc = blockIdx.y;
  const int k0 = kc * kChunkK;
  const int nks = min(kChunkK, a.kdim - k0) / KSTEP;       // k-steps in this chunk

  // this lane's weight row (clamped; rows past R are computed, never stored)
  const int vr = min(r0 + fr, a.R - 1);
  const bool up = vr >= a.R0;
  const int rr = up ? vr - a.R0 : vr;
  const char* wrow = (up ? a.B1 : a.B0) + (int64_t)rr * a.kdim * EB;
  const int nkb = a.kdim / 128;
  // byte offset of this lane's fragment piece j in k-step s of the chunk
  auto off = [&](int s, int j) -> int64_t {
    return FP8 ? (int64_t)(k0 + s * 128) + 32 * q + 16 * j
               : ((int64_t)(k0 + s * 32) + 8 * q) * 2;
  };
  // every load is issued up front; k-steps past the chunk re-read k-step 0
  // and are multiplied by a zero activation fragment
  constexpr int NP = FP8 ? 2 : 1;  // 16-byte pieces per fragment
  u32x4_t W[NKS][NP];
  float sw[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int ss = s < nks ? s : 0;
#pragma unroll
    for (int j = 0; j < NP; ++j) W[s][j] = *reinterpret_cast<const u32x4_t*>(wrow + off(ss, j));
    if (FP8) sw[s] = (up ? a.sb1 : a.sb0)[(rr / 128) * nkb + (k0 / 128) + ss];
  }
  u32x4_t T[NB][NKS][NP];
  float st[NB][NKS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t t = min((int64_t)(nb * 16 + fr), a.N - 1);
    const char* trow = a.A + t * a.kdim * EB;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int ss = s < nks ? s : 0;
#pragma unroll
      for (int j = 0; j < NP; ++j) T[nb][s][j] = *reinterpret_cast<const u32x4_t*>(trow + off(ss, j));
      if (FP8) st[nb][s] = a.sa[t * nkb + (k0 / 128) + ss];
    }
  }

  // Straight-line multiplies (k-steps past the chunk use a zero activation
  // fragment), so the compiler keeps every load ahead of them.
  __builtin_amdgcn_sched_barrier(0);
  floatx4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const bool live = s < nks;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
        if (!live) T[nb][s][j] = u32x4_t{0u, 0u, 0u, 0u};
      if (FP8) {
        const i32x8_t wf = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(W[s][0], W[s][NP - 1], 0, 1, 2, 3, 4, 5, 6, 7));
        const i32x8_t tf = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(T[nb][s][0], T[nb][s][NP - 1], 0, 1, 2, 3, 4, 5, 6, 7));
        const floatx4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf, tf, floatx4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        const float fac = sw[s] * st[nb][s];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[nb][r] = fmaf(p[r], fac, acc[nb][r]);
      } else {
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, W[s][0]),
                                                          __builtin_bit_cast(bf16x8_t, T[nb][s][0]),
                                                          acc[nb], 0, 0, 0);
      }
    }
  }
  // lane (fr, q): token 16*nb + fr, rows r0 + 4q .. +3
  const int row = r0 + 4 * q;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t t = nb * 16 + fr;
    if (t >= a.N) continue;
    float* dst = a.part + ((int64_t)kc * a.N + t) * a.R + row;
    if (row + 3 < a.R && (a.R % 4) == 0) {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row + r < a.R) dst[r] = acc[nb][r];
    }
  }
}

enum FinalMode { kFinRouter = 0, kFinGateUp = 1, kFinDown = 2 };

// Sum of the chunks' partials in chunk order; four loads are issued ahead
// of their additions.
__device__ __forceinline__ float sum_chunks(const float* part, int chunks, int64_t N, int R,
                                            int64_t t, int r) {
  const int64_t stride = N * R;
  const float* p = part + t * R + r;
  float s = 0.0f;
  int c = 0;
  for (; c + 4 <= chunks; c += 4) {
    const float v0 = p[c * stride], v1 = p[(c + 1) * stride];
    const float v2 = p[(c + 2) * stride], v3 = p[(c + 3) * stride];
    s += v0;
    s += v1;
    s += v2;
    s += v3;
  }
  for (; c < chunks; ++c) s += p[c * stride];
  return s;
}

// One thread per output element (router, down, bf16 gate/up).
template <int MODE>
__global__ __launch_bounds__(256) void dense_small_finalize(const float* part, int chunks,
                                                            int64_t N, int R, int R0,
                                                            const float* offset, void* out,
                                                            int64_t ldo) {
  const int cols = (MODE == kFinGateUp) ? R0 : R;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * cols) return;
  const int64_t t = i / cols;
  const int c = (int)(i % cols);
  if (MODE == kFinRouter) {
    float z = sum_chunks(part, chunks, N, R, t, c);
    if (offset) z += offset[c];
    reinterpret_cast<float*>(out)[t * ldo + c] = z;
  } else if (MODE == kFinDown) {
    reinterpret_cast<uint16_t*>(out)[t * ldo + c] =
        (uint16_t)f32_to_bf16_rne_bits(sum_chunks(part, chunks, N, R, t, c));
  } else {
    const float g = sum_chunks(part, chunks, N, R, t, c);
    const float u = sum_chunks(part, chunks, N, R, t, R0 + c);
    const float h = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
    reinterpret_cast<uint16_t*>(out)[t * ldo + c] = (uint16_t)f32_to_bf16_rne_bits(h);
  }
}

// E4M3 gate/up: one wave per (token, 1 x 128 group of H); lane l takes the
// hidden columns 2l, 2l+1 of the group.  H is quantised from its fp32 value
// with s = amax / 448 as the tile engine's epilogue does.
__global__ __launch_bounds__(256) void dense_small_finalize_fp8(const float* part, int chunks,
                                                                int64_t N, int R, int R0,
                                                                uint8_t* Hq, float* Hs) {
  const int groups = R0 / 128;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= N * groups) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = wid / groups;
  const int g = (int)(wid % groups);
  float hb[2];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = g * 128 + 2 * lane + j;
    const float gg = sum_chunks(part, chunks, N, R, t, c);
    const float uu = sum_chunks(part, chunks, N, R, t, R0 + c);
    const float h = gg * __builtin_amdgcn_rcpf(1.0f + __expf(-gg)) * uu;
    hb[j] = h;
    m = max(m, __float_as_uint(fabsf(h)));
  }
  m = wave_max_u32(m);
  const float amax = __uint_as_float(m);
  const float sc = amax / 448.0f;
  uint32_t codes = 0;
  if (amax != 0.0f) {
    const float u0 = fminf(fmaxf(hb[0] / sc, -448.0f), 448.0f);
    const float u1 = fminf(fmaxf(hb[1] / sc, -448.0f), 448.0f);
    codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u0, u1, 0, false) & 0xFFFFu;
  }
  *reinterpret_cast<uint16_t*>(Hq + t * R0 + g * 128 + 2 * lane) = (uint16_t)codes;
  if (lane == 0) Hs[t * groups + g] = (amax != 0.0f) ? sc : 0.0f;
}

template <bool FP8>
hipError_t launch_products(const DenseSmallArgs& a, hipStream_t stream) {
  const int chunks = (a.kdim + kChunkK - 1) / kChunkK;
  const dim3 grid((unsigned)((a.R + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)chunks);
  const int nb = (int)((a.N + 15) / 16);
  switch (nb) {
    case 1: hipLaunchKernelGGL((dense_small_kernel<FP8, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((dense_small_kernel<FP8, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((dense_small_kernel<FP8, 3>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((dense_small_kernel<FP8, 4>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int chunks_of(int kdim) { return (kdim + kChunkK - 1) / kChunkK; }

}  // namespace

size_t dense_small_part_floats(int64_t N, int d, int E, int hs) {
  const size_t r = (size_t)chunks_of(d) * N * E;
  const size_t g = (size_t)chunks_of(d) * N * 2 * hs;
  const size_t dn = (size_t)chunks_of(hs) * N * d;
  return r > g ? (r > dn ? r : dn) : (g > dn ? g : dn);
}

hipError_t launch_router_dense_small(const uint16_t* x, const uint16_t* w_router,
                                     const float* offset, int64_t N, int d, int E, float* Z,
                                     float* part, hipStream_t stream) {
  if (N < 1 || N > kSmallBatch) return hipErrorInvalidValue;
  DenseSmallArgs a{};
  a.A = reinterpret_cast<const char*>(x); a.N = N; a.kdim = d;
  a.B0 = reinterpret_cast<const char*>(w_router); a.B1 = nullptr; a.R0 = E; a.R = E;
  a.part = part;
  hipError_t e = launch_products<false>(a, stream);
  if (e != hipSuccess) return e;
  const int64_t n = N * E;
  hipLaunchKernelGGL(dense_small_finalize<kFinRouter>, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, part, chunks_of(d), N, E, E, offset, (void*)Z,
                     (int64_t)E);
  return hipGetLastError();
}

hipError_t launch_shared_gateup_dense_small(const void* x, const float* xs, int64_t N, int d,
                                            const void* wg, const float* sg, const void* wu,
                                            const float* su, int hs, bool fp8, void* H,
                                            float* Hs, float* part, hipStream_t stream) {
  if (N < 1 || N > kSmallBatch) return hipErrorInvalidValue;
  DenseSmallArgs a{};
  a.A = reinterpret_cast<const char*>(x); a.sa = xs; a.N = N; a.kdim = d;
  a.B0 = reinterpret_cast<const char*>(wg); a.B1 = reinterpret_cast<const char*>(wu);
  a.sb0 = sg; a.sb1 = su; a.R0 = hs; a.R = 2 * hs; a.part = part;
  hipError_t e = fp8 ? launch_products<true>(a, stream) : launch_products<false>(a, stream);
  if (e != hipSuccess) return e;
  if (fp8) {
    const int64_t waves = N * (hs / 128);
    hipLaunchKernelGGL(dense_small_finalize_fp8, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, part, chunks_of(d), N, 2 * hs, hs, reinterpret_cast<uint8_t*>(H),
                       Hs);
  } else {
    const int64_t n = N * hs;
    hipLaunchKernelGGL(dense_small_finalize<kFinGateUp>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, stream, part, chunks_of(d), N, 2 * hs, hs, nullptr, H,
                       (int64_t)hs);
  }
  return hipGetLastError();
}

hipError_t launch_shared_down_dense_small(const void* H, const float* Hs, int64_t N, int d,
                                          const void* wd, const float* sd, int hs, bool fp8,
                                          uint16_t* Y, float* part, hipStream_t stream) {
  if (N < 1 || N > kSmallBatch) return hipErrorInvalidValue;
  DenseSmallArgs a{};
  a.A = reinterpret_cast<const char*>(H); a.sa = Hs; a.N = N; a.kdim = hs;
  a.B0 = reinterpret_cast<const char*>(wd); a.B1 = nullptr; a.sb0 = sd; a.sb1 = sd;
  a.R0 = d; a.R = d; a.part = part;
  hipError_t e = fp8 ? launch_products<true>(a, stream) : launch_products<false>(a, stream);
  if (e != hipSuccess) return e;
  const int64_t n = N * d;
  hipLaunchKernelGGL(dense_small_finalize<kFinDown>, dim3((unsigned)((n + 255) / 256)), dim3(256),
                     0, stream, part, chunks_of(hs), N, d, d, nullptr, (void*)Y, (int64_t)d);
  return hipGetLastError();
}

}  // namespace moe
