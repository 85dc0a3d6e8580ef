// Bias-corrected top-K selection with unbiased sigmoid weights.
//
// "Kolibri Pre-Training from Scratch" §6.1 (routing equations): the bias is
// added to the logits for selection only, the mixture weights are the sigmoid
// of the unbiased logits and are not renormalised.  §7.1 gives the token bias
// alpha_t = -Q_K(Z_t + beta), i.e. minus the (K+1)-th largest biased score,
// which this kernel emits alongside the selection.
//
// One wave per token row (a wave walks rows with a grid stride and loads the
// next row while selecting the current one).  Lane l holds the experts l,
// l+64, ... (at most six for E <= 384) and turns each biased score into an
// order-preserving 32-bit key.  The selection order is key descending, then
// expert ascending (-0 and +0 share a key).  The row is read once from HBM.
//
// Full selection: K+1 rounds of a wave-wide max over the lanes' maxima give a
// lower bound L on the (K+1)-th largest key; the few entries with key >= L
// are compacted into LDS and ranked exactly (see the comments in the code).
//
// ALPHA_ONLY (the first pass of a bias update, which needs alpha alone): the
// value of the (K+1)-th largest key does not depend on how ties are ordered,
// so each lane sorts its keys and K+1 rounds pop the wave-wide maximum, with
// no ids.
#include "common.h"
#include "kernels.h"

namespace moe {

template <int NV, bool ALPHA_ONLY>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ Z, const float* __restrict__ beta, int64_t N, int E,
    int K, int32_t* __restrict__ ids, float* __restrict__ S,
    float* __restrict__ alpha, float* __restrict__ margin) {
  const int lane = lane_id();
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  // per wave: candidate composites of the current row (at most 64 * NV)
  __shared__ uint64_t cand[4][ALPHA_ONLY ? 1 : kWave * NV];
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;  // whole wave leaves together

  float bv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = lane + kWave * j;
    bv[j] = (beta && e < E) ? beta[e] : 0.0f;
  }
  // Rows are walked with a grid stride; the loads of the next row are issued
  // before the selection of the current one.
  float cur[NV], nxt[NV];
  auto load_row = [&](int64_t r, float* v) {
    const float* zr = Z + r * (int64_t)E;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = lane + kWave * j;
      v[j] = (e < E) ? zr[e] : 0.0f;
    }
  };
  load_row(row, cur);
  for (; row < N; row += nwaves) {
    const int64_t nrow = row + nwaves;
    if (nrow < N) load_row(nrow, nxt);

    uint32_t key[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = lane + kWave * j;
      key[j] = (e < E) ? f32_order_key(cur[j] + bv[j]) : 0u;  // 0: below every finite value
    }
    if (ALPHA_ONLY) {
#pragma unroll
      for (int i = 1; i < NV; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
          const uint32_t k0 = key[j - 1], k1 = key[j];
          key[j - 1] = max(k0, k1);
          key[j] = min(k0, k1);
        }
      }
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k <= MOE_KMAX_INTERNAL; ++k) {
        if (k > K) break;  // uniform
        m = wave_max_u32(key[0]);
        // one lane holding the maximum pops it (ties: the value is the same)
        const int win = __ffsll((unsigned long long)ballot(key[0] == m)) - 1;
        if (lane == win) {
#pragma unroll
          for (int j = 0; j + 1 < NV; ++j) key[j] = key[j + 1];
          key[NV - 1] = 0u;
        }
      }
      if (lane == 0) alpha[row] = -f32_from_order_key(m);
#pragma unroll
      for (int j = 0; j < NV; ++j) cur[j] = nxt[j];
      continue;
    }
    // Full selection.  (1) L = the (K+1)-th largest of the 64 lane maxima,
    // counted with multiplicity: the K+1 lanes popped hold K+1 distinct
    // entries >= L, so the row's (K+1)-th largest key is >= L and every entry
    // of the top K+1 is a candidate (key >= L).  (2) The candidates, usually
    // a handful, are compacted into LDS as 64-bit composites
    // (key << 32) | (2^32 - 1 - expert): distinct, and ordered exactly as
    // (key descending, expert ascending).  (3) Each candidate's rank is the
    // number of larger composites; ranks 0..K-1 are the selection in order,
    // ranks K-1 and K give the margin and alpha.
    uint32_t lm = key[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) lm = max(lm, key[j]);
    uint32_t L = 0u;
#pragma unroll
    for (int k = 0; k <= MOE_KMAX_INTERNAL; ++k) {
      if (k > K) break;  // uniform
      L = wave_max_u32(lm);
      const int win = __ffsll((unsigned long long)ballot(lm == L)) - 1;
      if (lane == win) lm = 0u;
    }
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) c += (key[j] >= L) ? 1u : 0u;
    // exclusive prefix of the per-lane counts (c <= 6), bit by bit
    uint32_t off = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const uint64_t m = ballot(((c >> b) & 1u) != 0u);
      off += (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
      total += (uint32_t)__popcll(m) << b;
    }
    uint64_t* cl = cand[threadIdx.x >> 6];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (key[j] >= L) {
        const uint32_t e = (uint32_t)(lane + kWave * j);
        cl[off++] = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - e);
      }
    }
    // the wave's own LDS writes are complete before its reads below
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint32_t key_k = 0u, key_k1 = 0u;
    for (uint32_t i = (uint32_t)lane; i < total; i += kWave) {
      const uint64_t ci = cl[i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < total; ++j) rank += (cl[j] > ci) ? 1u : 0u;
      if (rank < (uint32_t)K) {
        const uint32_t e = 0xFFFFFFFFu - (uint32_t)ci;
        if (ids) ids[row * K + rank] = (int32_t)e;
        if (S) {
          const float z = Z[row * (int64_t)E + e];
          S[row * K + rank] = (float)(1.0 / (1.0 + exp(-(double)z)));
        }
      }
      if (rank == (uint32_t)K - 1) key_k = (uint32_t)(ci >> 32);
      if (rank == (uint32_t)K) key_k1 = (uint32_t)(ci >> 32);
    }
    const uint64_t hk = ballot(key_k != 0u), hk1 = ballot(key_k1 != 0u);
    key_k = readlane_u32(key_k, __ffsll((unsigned long long)hk) - 1);
    key_k1 = readlane_u32(key_k1, __ffsll((unsigned long long)hk1) - 1);
    if (lane == 0) {
      const float vK = f32_from_order_key(key_k);
      const float vK1 = f32_from_order_key(key_k1);
      if (alpha) alpha[row] = -vK1;
      if (margin) margin[row] = vK - vK1;
    }
    // the next row's candidates overwrite this row's list
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NV; ++j) cur[j] = nxt[j];
  }
}

// ---------------------------------------------------------------- 16 lanes per row
// The same selection (same candidates, ranks and outputs) with a quarter wave
// per row, for E % 4 == 0 and a 16-byte aligned Z: lane g of a row's 16 lanes
// holds the experts 4g + 64j + c (c < 4, j < NC), read as float4, so one wave
// selects four rows at once and every cross-lane step is a 16-lane DPP row
// (the lane maxima, the K+1 pops that give L) or a ballot masked to the row.
// Rows past N (the last quad) re-read row N-1 and store nothing.  FULL: E is
// 64 * NC, so no lane holds a slot past E.  The next quad's rows load while
// this quad is selected.
//
// Keys: the bias is read once as beta + 0, which turns -0 into +0.  Under
// round to nearest a sum is -0 only when both operands are -0, so no biased
// score z + b is -0 and the order-preserving map needs no test for it (the
// two zeros share a key, as in f32_order_key).  The sigmoid weight
// is evaluated in fp32 (relative error a few ulp, within the 1e-6 of the
// weights); logits below -80, where e^-z nears the fp32 range, take the fp64
// form.
__device__ __forceinline__ uint32_t order_key_nonneg_zero(float v) {
  const uint32_t u = __float_as_uint(v);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float sigmoid_weight(float z) {
  if (z < -80.0f) return (float)(1.0 / (1.0 + exp(-(double)z)));
  return 1.0f / (1.0f + expf(-z));
}

template <int NC, bool FULL>
__global__ __launch_bounds__(256) void route_group_kernel(
    const float* __restrict__ Z, const float* __restrict__ beta, int64_t N, int E, int K,
    int32_t* __restrict__ ids, float* __restrict__ S, float* __restrict__ alpha,
    float* __restrict__ margin) {
  constexpr int NVL = 4 * NC;  // experts per lane
  const int lane = lane_id();
  const int g = lane & 15;     // lane within the row's 16
  const int grp = lane >> 4;   // row of the wave's quad
  const int wib = threadIdx.x >> 6;
  __shared__ uint64_t cand[4][4][16 * NVL];
  __shared__ uint32_t kk[4][4][2];
  const int64_t nquads = (N + 3) / 4;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t quad = (int64_t)blockIdx.x * 4 + wib;
  if (quad >= nquads) return;  // whole wave leaves together

  float bv[NVL];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * g + 64 * j + c;
      bv[4 * j + c] = (beta && (FULL || e < E)) ? beta[e] + 0.0f : 0.0f;
    }
  auto load_row = [&](int64_t q, float4 (&v)[NC]) {
    const int64_t r = min(q * 4 + grp, N - 1);
    const float* zr = Z + r * (int64_t)E;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int e0 = 4 * g + 64 * j;
      v[j] = (FULL || e0 < E) ? *reinterpret_cast<const float4*>(zr + e0)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  const uint64_t gmask = 0xFFFFull << (16 * grp);
  uint64_t* cl = cand[wib][grp];
  uint32_t* kl = kk[wib][grp];

  auto select = [&](int64_t q, const float4 (&cur)[NC]) {
    const int64_t row = q * 4 + grp;
    const bool row_ok = row < N;
    uint32_t key[NVL];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const float zc[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * g + 64 * j + c;
        key[4 * j + c] = (FULL || e < E) ? order_key_nonneg_zero(zc[c] + bv[4 * j + c]) : 0u;
      }
    }
    // (1) L = the (K+1)-th largest of the row's 16 lane maxima (with
    // multiplicity): every entry of the row's top K+1 has key >= L.
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < NVL; ++i) lm = max(lm, key[i]);
    uint32_t L = 0u;
#pragma unroll
    for (int k = 0; k <= MOE_KMAX_INTERNAL; ++k) {
      if (k > K) break;  // uniform
      L = row16_max_u32(lm);
      const int win = __ffsll((unsigned long long)(ballot(lm == L) & gmask)) - 1;
      if (lane == win) lm = 0u;
    }
    // (2) compact the candidates (key >= L) of the row into its LDS list as
    // composites (key << 32) | (2^32 - 1 - expert), in lane order
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < NVL; ++i) cnt += (key[i] >= L) ? 1u : 0u;
    uint32_t off = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {  // cnt <= 24
      const uint64_t m = ballot(((cnt >> b) & 1u) != 0u) & gmask;
      off += (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
      total += (uint32_t)__popcll(m) << b;
    }
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * j + c;
        if (key[i] >= L) {
          const uint32_t e = (uint32_t)(4 * g + 64 * j + c);
          cl[off++] = ((uint64_t)key[i] << 32) | (uint64_t)(0xFFFFFFFFu - e);
        }
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own list is written
    // (3) rank = number of larger composites
    for (uint32_t i = (uint32_t)g; i < total; i += 16) {
      const uint64_t ci = cl[i];
      uint32_t rank = 0;
#pragma unroll 4
      for (uint32_t j = 0; j < total; ++j) rank += (cl[j] > ci) ? 1u : 0u;
      if (row_ok && rank < (uint32_t)K) {
        const uint32_t e = 0xFFFFFFFFu - (uint32_t)ci;
        if (ids) ids[row * K + rank] = (int32_t)e;
        if (S) S[row * K + rank] = sigmoid_weight(Z[row * (int64_t)E + e]);
      }
      if (rank == (uint32_t)K - 1) kl[0] = (uint32_t)(ci >> 32);
      if (rank == (uint32_t)K) kl[1] = (uint32_t)(ci >> 32);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    if (g == 0 && row_ok) {
      const float vK = f32_from_order_key(kl[0]);
      const float vK1 = f32_from_order_key(kl[1]);
      if (alpha) alpha[row] = -vK1;
      if (margin) margin[row] = vK - vK1;
    }
    // the next quad's candidates overwrite this quad's lists
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  };

  float4 cur[NC], nxt[NC];
  load_row(quad, cur);
  for (; quad < nquads; quad += nwaves) {
    const int64_t nq = quad + nwaves;
    if (nq < nquads) load_row(nq, nxt);
    select(quad, cur);
#pragma unroll
    for (int j = 0; j < NC; ++j) cur[j] = nxt[j];
  }
}

// Blocks of 256 threads of one variant that the device holds at once
// (occupancy x compute units), queried once per variant and device.
// kind 0: one wave per row, 1: its keys-only variant, 2: 16 lanes per row.
static int64_t route_resident_blocks(int nv, int kind) {
  static int64_t cache[3][8][7] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 8) return 2048;
  int64_t& c = cache[kind][dev][nv];
  if (c) return c;
  const void* fn = nullptr;
  switch (nv) {
#define MOE_ROUTE_FN(V)                                                        \
    case V:                                                                    \
      fn = kind == 2 ? (const void*)route_group_kernel<V, false>               \
           : kind == 1 ? (const void*)route_topk_kernel<V, true>               \
                       : (const void*)route_topk_kernel<V, false>;             \
      break;
    MOE_ROUTE_FN(1) MOE_ROUTE_FN(2) MOE_ROUTE_FN(3) MOE_ROUTE_FN(4) MOE_ROUTE_FN(5) MOE_ROUTE_FN(6)
#undef MOE_ROUTE_FN
    default: return 2048;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      per_cu <= 0 || cus <= 0)
    return 2048;
  c = (int64_t)per_cu * cus;
  return c;
}

hipError_t launch_route(const float* Z, const float* beta, int64_t N, int E, int K,
                        int32_t* ids, float* S, float* alpha, float* margin,
                        hipStream_t stream) {
  const int nv = (E + kWave - 1) / kWave;
  // alpha alone: keys-only variant
  const bool alpha_only = ids == nullptr && S == nullptr && margin == nullptr && alpha != nullptr;
  const dim3 block(256);
  if (E % 4 == 0 && (uintptr_t)Z % 16 == 0) {
    // 16 lanes per row; the waves walk quads of rows with a grid stride
    int64_t blocks = ((N + 3) / 4 + 3) / 4;
    const int64_t cap = route_resident_blocks(nv, 2);
    if (blocks > cap) blocks = cap;
    const dim3 grid((unsigned)blocks);
    switch (nv) {
#define MOE_ROUTE_GROUP_CASE(V)                                                           \
      case V:                                                                             \
        if (E == 64 * V)                                                                  \
          hipLaunchKernelGGL((route_group_kernel<V, true>), grid, block, 0, stream, Z, beta, N, \
                             E, K, ids, S, alpha, margin);                                \
        else                                                                              \
          hipLaunchKernelGGL((route_group_kernel<V, false>), grid, block, 0, stream, Z, beta, \
                             N, E, K, ids, S, alpha, margin);                             \
        break;
      MOE_ROUTE_GROUP_CASE(1) MOE_ROUTE_GROUP_CASE(2) MOE_ROUTE_GROUP_CASE(3)
      MOE_ROUTE_GROUP_CASE(4) MOE_ROUTE_GROUP_CASE(5) MOE_ROUTE_GROUP_CASE(6)
#undef MOE_ROUTE_GROUP_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // The waves walk the rows with a grid stride; the grid is capped at what is
  // resident at once, so that no wave waits for a second round.
  int64_t blocks = (N + 3) / 4;
  const int64_t cap = route_resident_blocks(nv, alpha_only ? 1 : 0);
  if (blocks > cap) blocks = cap;
  const dim3 grid((unsigned)blocks);
  switch (nv) {
#define MOE_ROUTE_CASE(V)                                                                   \
    case V:                                                                                 \
      if (alpha_only)                                                                       \
        hipLaunchKernelGGL((route_topk_kernel<V, true>), grid, block, 0, stream, Z, beta, N, \
                           E, K, ids, S, alpha, margin);                                    \
      else                                                                                  \
        hipLaunchKernelGGL((route_topk_kernel<V, false>), grid, block, 0, stream, Z, beta,  \
                           N, E, K, ids, S, alpha, margin);                                 \
      break;
    MOE_ROUTE_CASE(1) MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(3)
    MOE_ROUTE_CASE(4) MOE_ROUTE_CASE(5) MOE_ROUTE_CASE(6)
#undef MOE_ROUTE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
