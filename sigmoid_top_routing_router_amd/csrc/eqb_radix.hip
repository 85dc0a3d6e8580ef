// Exact Quantile Balancing: the expert bias from an exact per-expert batch
// quantile, found by radix selection.
//
// "Kolibri Pre-Training from Scratch" §7.1: beta_e = -Q_r(Z[:,e] + alpha),
// r = T*K/E, then centred.  §7.3: every bfloat16 value is mapped to an
// order-preserving 16-bit key; a 256-bin histogram of the high byte shows
// which bin holds the wanted rank, and a second histogram of the low byte of
// the keys inside that bin gives the exact key.  Q_m is the (m+1)-th largest
// entry (§1).  The 32-bit variant runs the same selection over four bytes of
// order-preserving fp32 keys.
//
// Per pass:
//  * eqb_hist_kernel: a block owns 64 expert columns and a slab of rows; each
//    lane of a wave takes one column of one row (coalesced 256-byte row
//    segments), builds the key of fp32(Z + alpha) and counts the current byte
//    into a padded per-column LDS histogram (stride 257 words so that the 64
//    columns fall into different banks).  Every lane remembers the lowest and
//    highest bin it touched, so only that range of each column (one expert's
//    values fall into few bins) is added to the global [E][256] histogram,
//    with integer atomics (order-independent, so deterministic).
//  * eqb_scan_kernel: one wave per expert scans its 256 bins from the top,
//    finds the bin that holds the wanted rank and narrows the key prefix.
// After the last pass a one-block kernel subtracts the mean of the raw biases:
// one thread sums them in expert order in fp64, every thread then writes
// fp32(fp64(beta_raw) - mean).
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kEqbCols = 64;
constexpr int kEqbPad = 257;
constexpr int kEqbMaxE = 384;
constexpr int kEqbThreads = 512;              // 8 waves: 8 rows at a time
constexpr int kEqbRowLanes = kEqbThreads / kEqbCols;
constexpr int kEqbUnroll = 12;                // rows per lane with loads in flight

// Histograms of all passes.
size_t eqb_hist_bytes(int E, int key_bits) {
  return (size_t)(key_bits / 8) * (size_t)E * 256u * sizeof(uint32_t);
}
size_t eqb_state_bytes(int E) { return (size_t)(2 * E + 4) * sizeof(uint32_t); }

template <int KB, int PASS>
__global__ __launch_bounds__(kEqbThreads) void eqb_hist_kernel(
    const float* __restrict__ Z, const float* __restrict__ alpha, int64_t N, int E,
    int64_t rows_per_block, const uint32_t* __restrict__ prefix,
    uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[kEqbCols * kEqbPad];
  __shared__ int lo_s[kEqbRowLanes][kEqbCols], hi_s[kEqbRowLanes][kEqbCols];
  const int cl = threadIdx.x & (kEqbCols - 1);
  const int rs = threadIdx.x >> 6;
  const int e = blockIdx.x * kEqbCols + cl;
  for (int i = threadIdx.x; i < kEqbCols * kEqbPad; i += kEqbThreads) lh[i] = 0u;
  __syncthreads();

  constexpr int shift = KB - 8 * (PASS + 1);
  const bool col_ok = e < E;
  const uint32_t want = (PASS > 0 && col_ok) ? prefix[e] : 0u;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(N, r0 + rows_per_block);
  int lo = 256, hi = -1;
  if (col_ok) {
    uint32_t* my = lh + cl * kEqbPad;
    auto bump = [&](uint32_t key) {  // key: the KB-bit order key of one value
      if (PASS == 0 || (key >> (shift + 8)) == want) {
        const int b = (int)((key >> shift) & 0xFFu);
        atomicAdd(my + b, 1u);
        lo = min(lo, b);
        hi = max(hi, b);
      }
    };
    auto key_of = [&](float v) {
      return (KB == 16) ? bf16_order_key(f32_to_bf16_rne_bits(v)) : f32_order_key(v);
    };
    int64_t t = r0 + rs;
    constexpr int kTrip = kEqbUnroll * kEqbRowLanes;
    for (; t + (kTrip - kEqbRowLanes) < r1; t += kTrip) {  // loads of the whole trip first
      float z[kEqbUnroll], al[kEqbUnroll];
#pragma unroll
      for (int u = 0; u < kEqbUnroll; ++u) {
        z[u] = Z[(t + kEqbRowLanes * u) * E + e];
        al[u] = alpha[t + kEqbRowLanes * u];
      }
      if constexpr (KB == 16) {
        // two rows per conversion (v_cvt_pk_bf16_f32, round to nearest even)
        // and per packed key
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int u = 0; u < kEqbUnroll; u += 2) {
          const bf16x2_t bb = {(__bf16)(z[u] + al[u]), (__bf16)(z[u + 1] + al[u + 1])};
          const uint32_t k2 = bf16_order_key2(__builtin_bit_cast(uint32_t, bb));
          bump(k2 & 0xFFFFu);
          bump(k2 >> 16);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kEqbUnroll; ++u) bump(key_of(z[u] + al[u]));
      }
    }
    for (; t < r1; t += kEqbRowLanes) bump(key_of(Z[t * E + e] + alpha[t]));
  }
  lo_s[rs][cl] = lo;
  hi_s[rs][cl] = hi;
  __syncthreads();
  // flush: wave w takes columns w, w+8, ...; its lanes walk the touched bins
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int c = w; c < kEqbCols; c += kEqbRowLanes) {
    const int ee = blockIdx.x * kEqbCols + c;
    if (ee >= E) break;
    int clo = lo_s[0][c], chi = hi_s[0][c];
#pragma unroll
    for (int q = 1; q < kEqbRowLanes; ++q) {
      clo = min(clo, lo_s[q][c]);
      chi = max(chi, hi_s[q][c]);
    }
    for (int b = clo + lane; b <= chi; b += 64) {
      const uint32_t cnt = lh[c * kEqbPad + b];
      if (cnt != 0u) atomicAdd(hist + (size_t)ee * 256 + b, cnt);
    }
  }
}

// One wave per expert.  rank0 is the wanted 1-based rank for pass 0 (r+1).
// In the last pass the quantile is decoded into qraw (and quantile_out).
__global__ __launch_bounds__(256) void eqb_scan_kernel(
    const uint32_t* __restrict__ hist, uint32_t* __restrict__ prefix,
    uint32_t* __restrict__ rank, int E, int pass, int last, int key_bits,
    uint32_t rank0, float* __restrict__ qraw, float* __restrict__ quantile_out) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (e >= E) return;
  const uint4 v = reinterpret_cast<const uint4*>(hist + (size_t)e * 256)[lane];
  const uint32_t s = v.x + v.y + v.z + v.w;
  const uint32_t incl = wave_inclusive_sum_u32(s);
  const uint32_t total = readlane_u32(incl, 63);
  const uint32_t want = (pass == 0) ? rank0 : rank[e];
  // Bins of this lane from the top: 4l+3, 4l+2, 4l+1, 4l.
  uint32_t c = total - incl;  // entries in the bins above this lane's four
  int found = -1;
  uint32_t nr = 0;
  const uint32_t bins[4] = {v.w, v.z, v.y, v.x};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (found < 0 && c < want && want <= c + bins[i]) { found = 4 * lane + 3 - i; nr = want - c; }
    c += bins[i];
  }
  const uint64_t hit = ballot(found >= 0);
  const int src = hit ? (__ffsll((unsigned long long)hit) - 1) : 0;
  const uint32_t bin = readlane_u32((uint32_t)found, src);
  const uint32_t new_rank = readlane_u32(nr, src);
  if (lane == 0) {
    const uint32_t p = ((pass == 0) ? 0u : (prefix[e] << 8)) | (bin & 0xFFu);
    prefix[e] = p;
    rank[e] = new_rank;
    if (last) {
      const float q = (key_bits == 16) ? bf16_bits_to_f32(bf16_from_order_key(p))
                                       : f32_from_order_key(p);
      qraw[e] = q;
      if (quantile_out) quantile_out[e] = q;
    }
  }
}

// Centring of the raw biases -Q_e: one thread sums them in expert order in
// fp64, every thread writes fp32(fp64(-Q_e) - mean).  A kernel of its own
// (one block) after the last scan, so the quantiles of all scan blocks are
// visible without device-wide fences.
__global__ __launch_bounds__(256) void eqb_centre_kernel(const float* __restrict__ qraw, int E,
                                                         float* __restrict__ beta_out) {
  __shared__ double mean_s;
  __shared__ float q_s[kEqbMaxE];
  for (int i = threadIdx.x; i < E; i += blockDim.x) q_s[i] = qraw[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int i = 0; i < E; ++i) acc += (double)(-q_s[i]);
    mean_s = acc / (double)E;
  }
  __syncthreads();
  const double mean = mean_s;
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    beta_out[i] = (float)((double)(-q_s[i]) - mean);
}

static int64_t eqb_rows_per_block(int64_t N, int E) {
  const int col_groups = (E + kEqbCols - 1) / kEqbCols;
  // at most two blocks (70 KB of LDS each) per CU of the 256, so that the
  // whole grid is resident at once (no second round)
  const int64_t chunks = 512 / col_groups;
  int64_t rows_per_block = (N + chunks - 1) / chunks;
  if (rows_per_block < 96) rows_per_block = 96;
  return (rows_per_block + kEqbRowLanes - 1) / kEqbRowLanes * kEqbRowLanes;
}

hipError_t launch_eqb_hist(const float* Z, const float* alpha, int64_t N, int E, int key_bits,
                           int pass, const uint32_t* prefix, uint32_t* hist_pass,
                           hipStream_t stream) {
  const int col_groups = (E + kEqbCols - 1) / kEqbCols;
  const int64_t rows_per_block = eqb_rows_per_block(N, E);
  const int64_t chunks = (N + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)col_groups, (unsigned)chunks), block(kEqbThreads);
#define MOE_EQB_HIST(KB, P)                                                                  \
  hipLaunchKernelGGL((eqb_hist_kernel<KB, P>), grid, block, 0, stream, Z, alpha, N, E,     \
                     rows_per_block, prefix, hist_pass)
  if (key_bits == 16) {
    if (pass == 0) MOE_EQB_HIST(16, 0);
    else if (pass == 1) MOE_EQB_HIST(16, 1);
    else return hipErrorInvalidValue;
  } else {
    switch (pass) {
      case 0: MOE_EQB_HIST(32, 0); break;
      case 1: MOE_EQB_HIST(32, 1); break;
      case 2: MOE_EQB_HIST(32, 2); break;
      case 3: MOE_EQB_HIST(32, 3); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_EQB_HIST
  return hipGetLastError();
}

hipError_t launch_eqb_scan(const EqbWork& w, int E, int K, int key_bits, int pass,
                           int64_t n_total, float* beta_out, float* quantile_out,
                           hipStream_t stream) {
  const int passes = key_bits / 8;
  const int64_t r = (n_total * (int64_t)K) / E;
  const bool last = pass == passes - 1;
  hipLaunchKernelGGL(eqb_scan_kernel, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, stream,
                     w.hist + (size_t)pass * E * 256, w.state, w.state + E, E, pass,
                     last ? 1 : 0, key_bits, (uint32_t)(r + 1), w.qraw, quantile_out);
  if (last && beta_out)
    hipLaunchKernelGGL(eqb_centre_kernel, dim3(1), dim3(256), 0, stream, w.qraw, E, beta_out);
  return hipGetLastError();
}

hipError_t launch_eqb(const float* Z, const float* alpha, int64_t N, int E, int K,
                      int key_bits, float* beta_out, float* quantile_out,
                      const EqbWork& w, hipStream_t stream) {
  const int passes = key_bits / 8;
  hipError_t err = launch_fill_u32(w.hist, 0u, eqb_hist_bytes(E, key_bits) / 4, stream);
  if (err != hipSuccess) return err;
  for (int p = 0; p < passes; ++p) {
    err = launch_eqb_hist(Z, alpha, N, E, key_bits, p, w.state,
                          w.hist + (size_t)p * E * 256, stream);
    if (err != hipSuccess) return err;
    err = launch_eqb_scan(w, E, K, key_bits, p, N, beta_out, quantile_out, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
