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
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace moe {

template <int NV, bool ALPHA_ONLY>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ Z, const float* __restrict__ beta, int64_t N, int E,
    int K, int32_t* __restrict__ ids, float* __restrict__ S,
    float* __restrict__ alpha, float* __restrict__ margin, uint32_t* __restrict__ zero,
    int64_t zero_n) {
  clear_words<256>(zero, zero_n);
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
// The same selection (same outputs) with a quarter wave per row, for E % 4 == 0
// and a 16-byte aligned Z: lane g of a row's 16 lanes holds the experts
// 4g + 64j + c (c < 4, j < NC), read as float4, so one wave selects four rows
// (a quad) at once and every cross-lane step is a 16-lane DPP row or a ballot
// masked to the row.  Rows past N (the last quad) re-read row N-1 and store
// nothing.  FULL: E is 64 * NC, so no lane holds a slot past E (other slots
// score -inf, below every finite score).
//
// Schedule: one quad of rows per wave and a block per four quads, with no
// loop; seven blocks per CU are resident (registers, at E = 384), so other
// waves' loads overlap a wave's selection.  The results (ids, the picks'
// unbiased logits, the K-th and (K+1)-th scores) are gathered in LDS and
// stored by the wave at its end; the lanes that rank a winning candidate read
// its unbiased logit back from memory (an L2 hit), and the weight is formed
// from it only at the store, where little else is live (the sigmoid's fp64
// branch needs many registers).  (A grid-stride loop that loads the next
// quad during the selection was no faster: the gather for the weights waits
// for every load in flight, the prefetch included.)
//
// The bias is read once as beta + 0, which turns -0 into +0.  Under round to
// nearest a sum is -0 only when both operands are -0, so no biased score is
// -0, and for finite scores the float order is the order of the keys (the two
// zeros compare equal, as they share a key).  The sigmoid weight is evaluated
// in fp32 (relative error a few ulp, within the 1e-6 of the weights); logits
// below -80, where e^-z nears the fp32 range, take the fp64 form.
//
// (1) L = the (K+1)-th largest of the row's 16 lane maxima (with
// multiplicity): every entry of the row's top K+1 is >= L.
// (2) The candidates (score >= L) are compacted into the row's LDS list as
// (score, expert) pairs, and each is ranked by the number of candidates
// before it in the selection order (score descending, expert ascending).  A
// row with more than kRouteCap candidates (many scores tied at or above L)
// sends its wave to (2'): K+1 rounds pop the row's largest (score, lowest
// expert), which gives the same ids in the same order, and the same K-th and
// (K+1)-th scores.
constexpr int kRouteCap = 64;
__host__ __device__ constexpr int qraw_cap(int nc) { return 64 * nc; }

//
// Centring on the fly (CENTRE, after an exact quantile update): the bias is
// beta_e = fp32(fp64(-qraw_e) - mean), the mean over all experts in fp64 in
// expert order, formed as eqb_centre_kernel forms it (block_raw_bias_mean,
// from the raw quantiles in LDS); every block computes it before it loads
// its rows, and block 0 stores the biases to beta_out.  This saves the
// one-block centring launch, which inside the layer waits for a free
// compute unit.
template <int NC, bool FULL, bool CENTRE>
__global__ __launch_bounds__(256) void route_group_kernel(
    const float* __restrict__ Z, const float* __restrict__ beta, int64_t N, int E, int K,
    int32_t* __restrict__ ids, float* __restrict__ S, float* __restrict__ alpha,
    float* __restrict__ margin, uint32_t* __restrict__ zero, int64_t zero_n,
    const float* __restrict__ qraw, float* __restrict__ beta_out) {
  clear_words<256>(zero, zero_n);
  constexpr int NVL = 4 * NC;  // experts per lane
  const int lane = lane_id();
  const int g = lane & 15;     // lane within the row's 16
  const int grp = lane >> 4;   // row of the wave's quad
  const int wib = threadIdx.x >> 6;
  __shared__ float4 sbeta[16 * NC];  // [j][g]: the bias of lane g's four experts of j
  __shared__ float cand_s[4][4][kRouteCap];     // candidate scores
  __shared__ uint32_t cand_e[4][4][kRouteCap];  // their experts
  __shared__ int32_t out_id[4][4][MOE_KMAX_INTERNAL];
  __shared__ float out_s[4][4][MOE_KMAX_INTERNAL];  // unbiased logits of the picks
  __shared__ float kk[4][4][2];                 // K-th and (K+1)-th score
  if constexpr (CENTRE) {
    __shared__ float q_s[qraw_cap(NC)];  // raw quantiles
    for (int i = (int)threadIdx.x; i < E; i += 256) q_s[i] = qraw[i];
    __syncthreads();
    const double mean = block_raw_bias_mean<256>(q_s, E);
    for (int i = (int)threadIdx.x; i < 16 * NC; i += 256) {
      const int e0 = 4 * (i & 15) + 64 * (i >> 4);
      float b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (FULL || e0 + c < E) {
          const float bc = (float)((double)(-q_s[e0 + c]) - mean);
          if (blockIdx.x == 0 && beta_out) beta_out[e0 + c] = bc;
          b[c] = bc + 0.0f;
        }
      }
      sbeta[i] = make_float4(b[0], b[1], b[2], b[3]);
    }
  } else {
    for (int i = (int)threadIdx.x; i < 16 * NC; i += 256) {
      const int e0 = 4 * (i & 15) + 64 * (i >> 4);
      float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
      if (beta && (FULL || e0 < E))
        b = make_float4(beta[e0] + 0.0f, beta[e0 + 1] + 0.0f, beta[e0 + 2] + 0.0f,
                        beta[e0 + 3] + 0.0f);
      sbeta[i] = b;
    }
  }
  __syncthreads();
  const int64_t nquads = (N + 3) / 4;
  const int64_t quad = (int64_t)blockIdx.x * 4 + wib;  // one quad of rows per wave
  if (quad >= nquads) return;  // whole wave leaves together

  const uint64_t gmask = 0xFFFFull << (16 * grp);
  float* cs = cand_s[wib][grp];
  uint32_t* ce = cand_e[wib][grp];
  int32_t* oid = out_id[wib][grp];
  float* os = out_s[wib][grp];
  float* kl = kk[wib][grp];

  auto load_rows = [&](int64_t q, float4 (&v)[NC]) {
    const int64_t r = min(q * 4 + grp, N - 1);
    const float* zr = Z + r * (int64_t)E;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int e0 = 4 * g + 64 * j;
      v[j] = (FULL || e0 < E) ? *reinterpret_cast<const float4*>(zr + e0)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  // the results of quad q, from LDS to memory
  auto flush = [&](int64_t q) {
    const int64_t row = q * 4 + grp;
    if (row < N) {
      if (g < K) {
        if (ids) ids[row * K + g] = oid[g];
        if (S) S[row * K + g] = sigmoid_weight(os[g]);
      }
      if (g == 0) {
        if (alpha) alpha[row] = -kl[1];
        if (margin) margin[row] = kl[0] - kl[1];
      }
    }
  };

  auto select = [&](const float4 (&cur)[NC]) {
    float v[NVL];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const bool ok = FULL || 4 * g + 64 * j < E;
      const float4 b = sbeta[16 * j + g];
      v[4 * j + 0] = ok ? cur[j].x + b.x : -INFINITY;
      v[4 * j + 1] = ok ? cur[j].y + b.y : -INFINITY;
      v[4 * j + 2] = ok ? cur[j].z + b.z : -INFINITY;
      v[4 * j + 3] = ok ? cur[j].w + b.w : -INFINITY;
    }
    // (1)
    float lm = v[0];
#pragma unroll
    for (int i = 1; i < NVL; ++i) lm = fmaxf(lm, v[i]);
    float L = -INFINITY;
#pragma unroll
    for (int k = 0; k <= MOE_KMAX_INTERNAL; ++k) {
      if (k > K) break;  // uniform
      L = row16_max_f32(lm);
      const int win = __ffsll((unsigned long long)(ballot(lm == L) & gmask)) - 1;
      if (lane == win) lm = -INFINITY;
    }
    // (2) candidates of the row, in lane order
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < NVL; ++i) cnt += (v[i] >= L) ? 1u : 0u;
    uint32_t off = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {  // cnt <= 24
      const uint64_t m = ballot(((cnt >> b) & 1u) != 0u) & gmask;
      off += (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
      total += (uint32_t)__popcll(m) << b;
    }
    if (ballot(total > (uint32_t)kRouteCap) == 0) {
#pragma unroll
      for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = 4 * j + c;
          if (v[i] >= L) {
            cs[off] = v[i];
            ce[off] = (uint32_t)(4 * g + 64 * j + c);
            ++off;
          }
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own list is written
      for (uint32_t i = (uint32_t)g; i < total; i += 16) {
        const float si = cs[i];
        const uint32_t ei = ce[i];
        uint32_t rank = 0;
#pragma unroll 4
        for (uint32_t j = 0; j < total; ++j) {
          const float sj = cs[j];
          const uint32_t ej = ce[j];
          rank += (uint32_t)((sj > si) | ((sj == si) & (ej < ei)));
        }
        if (rank < (uint32_t)K) {
          oid[rank] = (int32_t)ei;
          os[rank] = Z[(quad * 4 + grp) * (int64_t)E + ei];
        }
        if (rank == (uint32_t)K - 1) kl[0] = si;
        if (rank == (uint32_t)K) kl[1] = si;
      }
    } else {
      // (2') pops in the order (score descending, expert ascending): pop r
      // takes the row's best (score, expert) that comes after pop r - 1 in
      // that order, so the scores are only read, never cleared.  A lane's
      // experts 64*(i >> 2) + 4g + (i & 3) rise with its slot i, so "expert
      // above ep" is "slot at least k_le", the number of the lane's experts
      // up to ep, and the lane's lowest expert of equal scores is its first
      // slot of them: no expert ids are held per slot.
      float sp = INFINITY, vK = 0.f, vK1 = 0.f;
      int k_le = 0;
#pragma unroll 1
      for (int r = 0; r <= K; ++r) {
        float bs = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
          const float sv = v[i];
          const bool after = r == 0 || sv < sp || (sv == sp && i >= k_le);
          const bool better = after && sv > bs;
          bs = better ? sv : bs;
          bi = better ? i : bi;
        }
        const uint32_t be = bi >= 0 ? (uint32_t)(64 * (bi >> 2) + 4 * g + (bi & 3)) : 0xFFFFFFFFu;
        const float rmx = row16_max_f32(bs);
        const uint32_t we = row16_min_u32(bs == rmx ? be : 0xFFFFFFFFu);
        if (r == K - 1) vK = rmx;
        if (r == K) vK1 = rmx;
        if (r < K && be == we) {
          oid[r] = (int32_t)we;
          os[r] = Z[(quad * 4 + grp) * (int64_t)E + we];
        }
        sp = rmx;
        const int wa = (int)(we >> 6), wg2 = (int)((we >> 2) & 15u), wc = (int)(we & 3u);
        k_le = 4 * wa + (g < wg2 ? 4 : (g == wg2 ? wc + 1 : 0));
      }
      if (g == 0) {
        kl[0] = vK;
        kl[1] = vK1;
      }
    }
    // the results are in LDS before the flush reads them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  };

  float4 cur[NC];
  load_rows(quad, cur);
  select(cur);
  flush(quad);
}

// ---------------------------------------------------------------- merge
// The end of the selection fused into the router GEMM: each of the row's
// T column tiles left its KC = K + 1 first (biased score, expert) entries,
// and the row's own first KC entries are the first KC of that union (an
// entry among a row's KC first is among its tile's KC first).  16 lanes per
// row rank the T * KC <= 32 entries exactly in the order (score descending,
// expert ascending); the outputs are those of route_group_kernel: ids and
// weights sigma(z) of the K picks (z, the unbiased logit, read back from
// Z), alpha = -(K+1)-th score, margin = K-th minus (K+1)-th score.
__global__ __launch_bounds__(256) void route_merge_kernel(
    const float* __restrict__ cand_s, const uint32_t* __restrict__ cand_e, int C,
    const float* __restrict__ Z, int64_t N, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ S, float* __restrict__ alpha, float* __restrict__ margin,
    uint32_t* __restrict__ zero, int64_t zero_n) {
  clear_words<256>(zero, zero_n);
  __shared__ float ls[16][32];
  __shared__ uint32_t le[16][32];
  __shared__ float kk[16][2];
  const int g = threadIdx.x & 15;
  const int rl = threadIdx.x >> 4;
  const int64_t row = (int64_t)blockIdx.x * 16 + rl;
  const bool ok = row < N;
  if (ok) {
    for (int c = g; c < C; c += 16) {
      ls[rl][c] = cand_s[row * C + c];
      le[rl][c] = cand_e[row * C + c];
    }
  }
  __syncthreads();
  if (ok) {
    for (int i = g; i < C; i += 16) {
      const float si = ls[rl][i];
      const uint32_t ei = le[rl][i];
      uint32_t rank = 0;
      for (int j = 0; j < C; ++j) {
        const float sj = ls[rl][j];
        const uint32_t ej = le[rl][j];
        rank += (uint32_t)((sj > si) | ((sj == si) & (ej < ei)));
      }
      if (rank < (uint32_t)K) {
        if (ids) ids[row * K + rank] = (int32_t)ei;
        if (S && ei < (uint32_t)E) S[row * K + rank] = sigmoid_weight(Z[row * (int64_t)E + ei]);
      }
      if (rank == (uint32_t)K - 1) kk[rl][0] = si;
      if (rank == (uint32_t)K) kk[rl][1] = si;
    }
  }
  __syncthreads();
  if (ok && g == 0) {
    if (alpha) alpha[row] = -kk[rl][1];
    if (margin) margin[row] = kk[rl][0] - kk[rl][1];
  }
}

int router_col_tiles(int E) { return (E + 255) / 256; }

hipError_t launch_route_merge(const float* cand_s, const uint32_t* cand_e, int n_col_tiles,
                              const float* Z, int64_t N, int E, int K, int32_t* ids, float* S,
                              float* alpha, float* margin, hipStream_t stream, uint32_t* zero,
                              size_t zero_n) {
  const int C = n_col_tiles * (K + 1);
  if (C > 32 || K > MOE_KMAX_INTERNAL || N < 1) return hipErrorInvalidValue;
  const int64_t blocks = (N + 15) / 16;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, cand_s,
                     cand_e, C, Z, N, E, K, ids, S, alpha, margin, zero,
                     zero ? (int64_t)zero_n : (int64_t)0);
  return hipGetLastError();
}

// Blocks of 256 threads of one variant of the one-wave kernel that the device
// holds at once (occupancy x compute units), queried once per variant and
// device.  kind 0: full selection, 1: the keys-only variant.  Host threads
// may race to fill an entry; each computes the same value.
static int64_t route_resident_blocks(int nv, int kind) {
  static std::atomic<int64_t> cache[2][8][7] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 8) return 2048;
  std::atomic<int64_t>& c = cache[kind][dev][nv];
  const int64_t known = c.load(std::memory_order_relaxed);
  if (known) return known;
  const void* fn = nullptr;
  switch (nv) {
#define MOE_ROUTE_FN(V)                                                        \
    case V:                                                                    \
      fn = kind == 1 ? (const void*)route_topk_kernel<V, true>                 \
                     : (const void*)route_topk_kernel<V, false>;               \
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
  const int64_t v = (int64_t)per_cu * cus;
  c.store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_route(const float* Z, const float* beta, int64_t N, int E, int K,
                        int32_t* ids, float* S, float* alpha, float* margin,
                        hipStream_t stream, uint32_t* zero, size_t zero_n) {
  return launch_route_centred(Z, beta, nullptr, nullptr, N, E, K, ids, S, alpha, margin, stream,
                              zero, zero_n);
}

hipError_t launch_route_centred(const float* Z, const float* beta, const float* qraw,
                                float* beta_out, int64_t N, int E, int K, int32_t* ids,
                                float* S, float* alpha, float* margin, hipStream_t stream,
                                uint32_t* zero, size_t zero_n) {
  const int64_t zn = zero ? (int64_t)zero_n : 0;
  const int nv = (E + kWave - 1) / kWave;
  // alpha alone: keys-only variant
  const bool alpha_only = ids == nullptr && S == nullptr && margin == nullptr && alpha != nullptr;
  const dim3 block(256);
  if (E % 4 == 0 && (uintptr_t)Z % 16 == 0) {
    // 16 lanes per row, one quad of rows per wave
    const int64_t blocks = ((N + 3) / 4 + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (nv) {
#define MOE_ROUTE_GROUP_LAUNCH(V, F, C)                                                   \
  hipLaunchKernelGGL((route_group_kernel<V, F, C>), grid, block, 0, stream, Z, beta, N, E, K, \
                     ids, S, alpha, margin, zero, zn, qraw, beta_out)
#define MOE_ROUTE_GROUP_CASE(V)                                                           \
      case V:                                                                             \
        if (E == 64 * V) {                                                                \
          if (qraw) MOE_ROUTE_GROUP_LAUNCH(V, true, true);                                \
          else MOE_ROUTE_GROUP_LAUNCH(V, true, false);                                    \
        } else {                                                                          \
          if (qraw) MOE_ROUTE_GROUP_LAUNCH(V, false, true);                               \
          else MOE_ROUTE_GROUP_LAUNCH(V, false, false);                                   \
        }                                                                                 \
        break;
      MOE_ROUTE_GROUP_CASE(1) MOE_ROUTE_GROUP_CASE(2) MOE_ROUTE_GROUP_CASE(3)
      MOE_ROUTE_GROUP_CASE(4) MOE_ROUTE_GROUP_CASE(5) MOE_ROUTE_GROUP_CASE(6)
#undef MOE_ROUTE_GROUP_CASE
#undef MOE_ROUTE_GROUP_LAUNCH
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (qraw) {
    // the one-wave kernel takes a finished bias: centre in a launch of its own
    const hipError_t err = launch_eqb_centre(qraw, E, beta_out, stream);
    if (err != hipSuccess) return err;
    beta = beta_out;
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
                           E, K, ids, S, alpha, margin, zero, zn);                          \
      else                                                                                  \
        hipLaunchKernelGGL((route_topk_kernel<V, false>), grid, block, 0, stream, Z, beta,  \
                           N, E, K, ids, S, alpha, margin, zero, zn);                       \
      break;
    MOE_ROUTE_CASE(1) MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(3)
    MOE_ROUTE_CASE(4) MOE_ROUTE_CASE(5) MOE_ROUTE_CASE(6)
#undef MOE_ROUTE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
