// Routing diagnostics: expert loads, MaxVio, intervention rate, near-ties.
//
// "Kolibri Pre-Training from Scratch" §6.2: MaxVio = max_e c_e / (K T / E) - 1
// over the loads c_e of a batch.  §9: the intervention rate of the bias is the
// mean over tokens of 1 - |I^u_t ∩ I_t| / K, where I^u_t is the router's own
// top-K (no bias) and I_t the routed one; with a bias that has taken over the
// selection it approaches 1 - K/E.
//
// stats_kernel: one thread per token adds its K selections to the loads
// (integer atomics), counts how many of its routed experts are also among its
// unbiased top-K, and whether its margin is a near-tie; wave and block sums,
// then one 64-bit integer atomic per block and counter.  finalize_kernel (one
// block) reduces the loads to their maximum and minimum and forms the two
// rates in fp64.  All sums are integer, so every result is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int K>
__global__ __launch_bounds__(256) void route_stats_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ ids_u,
    const float* __restrict__ margin, int64_t N, int E, float tau,
    int32_t* __restrict__ counts, RouteStatsDev* __restrict__ st) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t overlap = 0, near = 0;
  if (t < N) {
    int32_t a[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      a[k] = ids[t * K + k];
      if ((uint32_t)a[k] < (uint32_t)E) atomicAdd(counts + a[k], 1);  // ids outside [0,E) are not counted
    }
    if (ids_u) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int32_t u = ids_u[t * K + j];
        bool hit = false;
#pragma unroll
        for (int k = 0; k < K; ++k) hit |= (a[k] == u);
        overlap += hit ? 1u : 0u;
      }
    }
    if (margin) near = (margin[t] < tau) ? 1u : 0u;
  }
  // block sums: wave sums by shuffles, then the four waves through LDS
  __shared__ uint32_t s_ov[4], s_nt[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t ov = wave_inclusive_sum_u32(overlap);
  uint32_t nt = wave_inclusive_sum_u32(near);
  if (lane == 63) { s_ov[w] = ov; s_nt[w] = nt; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t bo = (uint64_t)s_ov[0] + s_ov[1] + s_ov[2] + s_ov[3];
    const uint64_t bn = (uint64_t)s_nt[0] + s_nt[1] + s_nt[2] + s_nt[3];
    if (bo) atomicAdd(reinterpret_cast<unsigned long long*>(&st->overlap), (unsigned long long)bo);
    if (bn) atomicAdd(reinterpret_cast<unsigned long long*>(&st->near_ties), (unsigned long long)bn);
  }
}

__global__ __launch_bounds__(256) void route_stats_finalize_kernel(
    const int32_t* __restrict__ counts, int64_t N, int E, int K, int have_u,
    RouteStatsDev* __restrict__ st) {
  __shared__ int32_t s_max[4], s_min[4];
  int32_t mx = 0, mn = 0x7FFFFFFF;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int32_t c = counts[e];
    mx = max(mx, c);
    mn = min(mn, c);
  }
  // wave max/min of non-negative loads as unsigned
  mx = (int32_t)wave_max_u32((uint32_t)mx);
  mn = (int32_t)wave_min_u32((uint32_t)mn);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { s_max[w] = mx; s_min[w] = mn; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t M = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    const int32_t m = min(min(s_min[0], s_min[1]), min(s_min[2], s_min[3]));
    const double target = (double)K * (double)N / (double)E;
    st->max_load = M;
    st->min_load = m;
    st->max_vio = (double)M / target - 1.0;
    st->intervention_rate =
        have_u ? 1.0 - (double)st->overlap / ((double)N * (double)K) : __builtin_nan("");
  }
}

hipError_t launch_route_stats(const int32_t* ids, const int32_t* ids_u, const float* margin,
                              int64_t N, int E, int K, float tau, int32_t* counts,
                              RouteStatsDev* st, hipStream_t stream) {
  hipError_t err = launch_fill_u32(reinterpret_cast<uint32_t*>(counts), 0u, (size_t)E, stream);
  if (err != hipSuccess) return err;
  err = launch_fill_u32(reinterpret_cast<uint32_t*>(st), 0u, sizeof(RouteStatsDev) / 4, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)((N + 255) / 256)), block(256);
  switch (K) {
#define MOE_STATS_CASE(KK)                                                                 \
    case KK:                                                                               \
      hipLaunchKernelGGL(route_stats_kernel<KK>, grid, block, 0, stream, ids, ids_u, margin, \
                         N, E, tau, counts, st);                                           \
      break;
    MOE_STATS_CASE(1) MOE_STATS_CASE(2) MOE_STATS_CASE(3) MOE_STATS_CASE(4)
    MOE_STATS_CASE(5) MOE_STATS_CASE(6) MOE_STATS_CASE(7) MOE_STATS_CASE(8)
#undef MOE_STATS_CASE
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(route_stats_finalize_kernel, dim3(1), block, 0, stream, counts, N, E, K,
                     ids_u ? 1 : 0, st);
  return hipGetLastError();
}

}  // namespace moe
