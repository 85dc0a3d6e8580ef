// Load-Error Injection: balance inside a microbatch through the gradient of
// the routing scores.
//
// "Kolibri Pre-Training from Scratch" §8: with the loads c_e of the
// microbatch B, f_e = c_e / (K|B|/E), rho = f - 1, xi = ||rho||_inf / tau, the
// gradient with respect to every score S_{t,e} receives
// lam * tanh(xi)/xi * rho_e (the factor is 1 at xi = 0), which stays below
// lam * tau in size.  The logits get the sum through S'(Z) = sigma(1 - sigma).
//
// lei_coef_kernel (one block): rho, xi and the factor in fp64, the per-expert
// injection rounded once to fp32.  lei_apply_kernel: one pass over [N,E]
// (16-byte accesses when E % 4 == 0): G' = G + inj_e in fp32, and
// dZ = G' * e / (1 + e)^2 with e = exp(-|z|), the form of sigma(1 - sigma)
// without cancellation for large |z|.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void lei_coef_kernel(const int32_t* __restrict__ counts,
                                                       int64_t N, int E, int K, double lam,
                                                       double tau, float* __restrict__ inj,
                                                       float* __restrict__ inj_out) {
  __shared__ double s_max[256];
  const double target = (double)K * (double)N / (double)E;
  double m = 0.0;
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    m = fmax(m, fabs((double)counts[e] / target - 1.0));
  s_max[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s_max[threadIdx.x] = fmax(s_max[threadIdx.x], s_max[threadIdx.x + w]);
    __syncthreads();
  }
  const double xi = s_max[0] / tau;
  const double scale = (xi == 0.0) ? 1.0 : tanh(xi) / xi;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const double rho = (double)counts[e] / target - 1.0;
    const float v = (float)(lam * scale * rho);
    inj[e] = v;
    if (inj_out) inj_out[e] = v;
  }
}

__device__ __forceinline__ float sigmoid_prime(float z) {
  const float e = expf(-fabsf(z));
  const float d = 1.0f + e;
  return e / (d * d);
}

template <bool VEC4>
__global__ __launch_bounds__(256) void lei_apply_kernel(
    const float* __restrict__ Z, const float* G, const float* __restrict__ inj, int64_t N,
    int E, float* Gout, float* __restrict__ dZ) {
  // G and Gout may be the same buffer (in-place update): every element is
  // read before it is written by the same thread.
  const int64_t total = N * (int64_t)E;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (VEC4) {
    const int64_t total4 = total / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += stride) {
      const int e = (int)((i * 4) % E);
      const float4 iv = *reinterpret_cast<const float4*>(inj + e);
      float4 g = G ? reinterpret_cast<const float4*>(G)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      g.x += iv.x; g.y += iv.y; g.z += iv.z; g.w += iv.w;
      if (Gout) reinterpret_cast<float4*>(Gout)[i] = g;
      if (dZ) {
        const float4 z = reinterpret_cast<const float4*>(Z)[i];
        float4 o;
        o.x = g.x * sigmoid_prime(z.x); o.y = g.y * sigmoid_prime(z.y);
        o.z = g.z * sigmoid_prime(z.z); o.w = g.w * sigmoid_prime(z.w);
        reinterpret_cast<float4*>(dZ)[i] = o;
      }
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
      const float g = (G ? G[i] : 0.0f) + inj[i % E];
      if (Gout) Gout[i] = g;
      if (dZ) dZ[i] = g * sigmoid_prime(Z[i]);
    }
  }
}

static bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hipError_t launch_lei(const float* Z, const int32_t* ids, const float* G, int64_t N, int E,
                      int K, float lam, float tau, float* Gout, float* dZ, float* inj_out,
                      int32_t* counts, float* inj, hipStream_t stream) {
  hipError_t err = launch_count(ids, N * (int64_t)K, E, counts, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(lei_coef_kernel, dim3(1), dim3(256), 0, stream, counts, N, E, K,
                     (double)lam, (double)tau, inj, inj_out);
  const bool vec = (E % 4) == 0 && al16(Z) && al16(G) && al16(Gout) && al16(dZ) && al16(inj);
  const int64_t work = vec ? N * (int64_t)E / 4 : N * (int64_t)E;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (vec)
    hipLaunchKernelGGL(lei_apply_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, Z, G,
                       inj, N, E, Gout, dZ);
  else
    hipLaunchKernelGGL(lei_apply_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, Z,
                       G, inj, N, E, Gout, dZ);
  return hipGetLastError();
}

}  // namespace moe
