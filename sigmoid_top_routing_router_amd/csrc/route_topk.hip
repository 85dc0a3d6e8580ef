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
// l+64, ... (at most six for E <= 384), turns each biased score into an
// order-preserving 32-bit key
// and sorts its own few entries (key descending, expert ascending).  K+1
// rounds of a wave-wide max over the lanes' current heads then pick the
// winners in global order; ties between lanes go to the lower expert id
// through a second (rare) min-reduction.  The row is read once from HBM.
//
// ALPHA_ONLY (the first pass of a bias update, which needs alpha alone): the
// value of the (K+1)-th largest key does not depend on how ties are ordered,
// so only keys are sorted and popped, with no tie-break and no ids.
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
    uint32_t eid[NV];
    float zv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = lane + kWave * j;
      zv[j] = cur[j];
      key[j] = (e < E) ? f32_order_key(cur[j] + bv[j]) : 0u;  // 0: below every finite value
      eid[j] = (uint32_t)e;
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
    // Per-lane sort, key descending; equal keys keep ascending expert order
    // (insertion sort moves an entry only past strictly smaller keys).
#pragma unroll
    for (int i = 1; i < NV; ++i) {
#pragma unroll
      for (int j = i; j > 0; --j) {
        const bool sw = key[j] > key[j - 1];
        const uint32_t k0 = key[j - 1], k1 = key[j];
        const uint32_t e0 = eid[j - 1], e1 = eid[j];
        const float z0 = zv[j - 1], z1 = zv[j];
        key[j - 1] = sw ? k1 : k0; key[j] = sw ? k0 : k1;
        eid[j - 1] = sw ? e1 : e0; eid[j] = sw ? e0 : e1;
        zv[j - 1] = sw ? z1 : z0; zv[j] = sw ? z0 : z1;
      }
    }

    uint32_t key_k = 0u, key_k1 = 0u;  // keys of the K-th and (K+1)-th winners
    uint32_t my_id = 0;
    float my_z = 0.0f;
#pragma unroll
    for (int k = 0; k <= MOE_KMAX_INTERNAL; ++k) {
      if (k > K) break;  // uniform
      const uint32_t head = key[0];
      const uint32_t m = wave_max_u32(head);
      const uint64_t tied = ballot(head == m);
      int win;
      if (__popcll(tied) == 1) {
        win = __ffsll((unsigned long long)tied) - 1;
      } else {
        const uint32_t cand = (head == m) ? eid[0] : 0xFFFFFFFFu;
        const uint32_t best = wave_min_u32(cand);
        win = __ffsll((unsigned long long)ballot(head == m && eid[0] == best)) - 1;
      }
      const uint32_t wid = readlane_u32(eid[0], win);
      const float wz = __uint_as_float(readlane_u32(__float_as_uint(zv[0]), win));
      if (k == K - 1) key_k = m;
      if (k == K) key_k1 = m;
      if (lane == k) { my_id = wid; my_z = wz; }
      if (lane == win) {
#pragma unroll
        for (int j = 0; j + 1 < NV; ++j) { key[j] = key[j + 1]; eid[j] = eid[j + 1]; zv[j] = zv[j + 1]; }
        key[NV - 1] = 0u;
      }
    }

    if (lane < K) {
      if (ids) ids[row * K + lane] = (int32_t)my_id;
      if (S) S[row * K + lane] = (float)(1.0 / (1.0 + exp(-(double)my_z)));
    }
    if (lane == 0) {
      const float vK = f32_from_order_key(key_k);
      const float vK1 = f32_from_order_key(key_k1);
      if (alpha) alpha[row] = -vK1;
      if (margin) margin[row] = vK - vK1;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) cur[j] = nxt[j];
  }
}

// Blocks of 256 threads of one variant that the device holds at once
// (occupancy x compute units), queried once per variant and device.
static int64_t route_resident_blocks(int nv, bool alpha_only) {
  static int64_t cache[2][8][7] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 8) return 2048;
  int64_t& c = cache[alpha_only ? 1 : 0][dev][nv];
  if (c) return c;
  const void* fn = nullptr;
  switch (nv) {
#define MOE_ROUTE_FN(V) \
    case V: fn = alpha_only ? (const void*)route_topk_kernel<V, true> : (const void*)route_topk_kernel<V, false>; break;
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
  // The waves walk the rows with a grid stride; the grid is capped at what is
  // resident at once, so that no wave waits for a second round.
  int64_t blocks = (N + 3) / 4;
  const int64_t cap = route_resident_blocks(nv, alpha_only);
  if (blocks > cap) blocks = cap;
  const dim3 grid((unsigned)blocks), block(256);
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
