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
// One update over a whole batch (launch_eqb), key_bits / 8 histogram passes:
//  * eqb_hist_kernel: a block owns 64 expert columns and a slab of rows; a
//    wave takes four rows at a time, 16 lanes per row, each lane four
//    adjacent columns (one 16-byte load; the 16 lanes cover the block's
//    256-byte piece of the row), with eight such quads of rows in flight per
//    wave; each lane builds the keys of fp32(Z + alpha) and counts the current
//    byte into a padded per-column LDS histogram (stride 257 words so that
//    the 64 columns fall into different banks).  Every lane remembers the lowest and
//    highest bin it touched, so only that range of each column (one expert's
//    values fall into few bins) is added to the global [E][256] histogram,
//    with integer atomics (order-independent, so deterministic).
//    From the second pass on, the block first selects, for each of its 64
//    columns, the bin of the previous pass that holds the wanted rank (one
//    wave per column scans the 256 bins from the top), which gives the key
//    prefix the pass counts under; the blocks of the first row slab also
//    store that prefix and the remaining rank for the next launch.  The
//    blocks of the first row slab zero the next pass's histogram of their
//    columns, so no launch is spent on clearing it (the first pass's
//    histogram is cleared by the kernel before, the routing pass that gives
//    alpha, or by a fill).
//  * eqb_last_kernel: one wave per expert selects the last byte of its key
//    from the last histogram and decodes the quantile.
//  * eqb_centre_kernel (one block): the mean of the raw biases in fp64 as
//    their sum in expert order (block_raw_bias_mean: a tree over the block
//    where every partial sum is exact, else one thread in order), then every
//    thread writes fp32(fp64(beta_raw) - mean).
// Five launches for 16-bit keys with alpha given: the fill, two histogram
// passes, the last selection and the centring.
//
// Over a batch given in parts (launch_eqb_hist / launch_eqb_scan): every
// part's histogram of a pass is added into the same [E][256] buffer, and
// eqb_scan_kernel (one wave per expert) selects the bin between passes; the
// centring then runs as eqb_centre_kernel.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kEqbCols = 64;
constexpr int kEqbPad = 257;
constexpr int kEqbMaxE = 384;
constexpr int kEqbThreads = 512;              // 8 waves, each 4 rows at a time
constexpr int kEqbWaves = kEqbThreads / 64;
constexpr int kEqbQuadUnroll = 8;             // row quads per wave with loads in flight

// Histograms of all passes.
size_t eqb_hist_bytes(int E, int key_bits) {
  return (size_t)(key_bits / 8) * (size_t)E * 256u * sizeof(uint32_t);
}
// State: [0, 2E) prefix and remaining rank for the parts path; [2E, 6E) two
// (prefix, rank) buffers that the passes of one launch_eqb alternate
// (pass p writes buffer p & 1 while its blocks read buffer (p - 1) & 1 of the
// previous launch); 4 spare words.
size_t eqb_state_bytes(int E) { return (size_t)(6 * E + 4) * sizeof(uint32_t); }

// Wave-wide selection step of the radix walk: the 256 bins of one expert's
// histogram h, scanned from the top; want is the 1-based rank among the
// entries still selected.  Returns the bin holding it and the rank inside
// that bin (every lane gets both).
// v: this lane's four bins 4l .. 4l+3, loaded by the caller (so that the
// loads of several experts can be in flight together).
__device__ __forceinline__ void select_bin_v(const uint4 v, uint32_t want, uint32_t& bin,
                                             uint32_t& rank_in_bin) {
  const int lane = lane_id();
  const uint32_t s = v.x + v.y + v.z + v.w;
  const uint32_t incl = wave_inclusive_sum_dpp_u32(s);
  const uint32_t total = readlane_u32(incl, 63);
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
  bin = readlane_u32((uint32_t)found, src) & 0xFFu;
  rank_in_bin = readlane_u32(nr, src);
}
__device__ __forceinline__ void select_bin(const uint32_t* __restrict__ h, uint32_t want,
                                           uint32_t& bin, uint32_t& rank_in_bin) {
  select_bin_v(reinterpret_cast<const uint4*>(h)[lane_id()], want, bin, rank_in_bin);
}

__device__ __forceinline__ float quantile_from_key(uint32_t p, int key_bits) {
  return (key_bits == 16) ? bf16_bits_to_f32(bf16_from_order_key(p)) : f32_from_order_key(p);
}

// Arguments of one histogram pass.  Parts path: prefix[e] is the key prefix
// of the pass (PASS > 0).  Whole-batch path (SCAN): hist_prev is the previous
// pass's histogram, st_in its (prefix, rank) state (NULL after the first
// pass: prefix 0, rank rank0), st_out where the first row slab stores the
// selected prefix and rank; zero_next (or NULL) the next pass's histogram.
struct EqbPassArgs {
  const uint32_t* prefix;
  const uint32_t* hist_prev;
  const uint32_t* st_in;
  uint32_t* st_out;
  uint32_t* zero_next;
  uint32_t rank0;
};

template <int KB, int PASS, bool SCAN, bool VEC>
__global__ __launch_bounds__(kEqbThreads) void eqb_hist_kernel(
    const float* __restrict__ Z, const float* __restrict__ alpha, int64_t N, int E,
    int64_t rows_per_block, EqbPassArgs pa, uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[kEqbCols * kEqbPad];
  __shared__ int lo_s[kEqbWaves][kEqbCols], hi_s[kEqbWaves][kEqbCols];
  __shared__ uint32_t want_s[kEqbCols];
  const int w = threadIdx.x >> 6;
  const int lane = lane_id();
  for (int i = threadIdx.x; i < kEqbCols * kEqbPad; i += kEqbThreads) lh[i] = 0u;
  if (pa.zero_next && blockIdx.y == 0) {
    const int ncols = min(kEqbCols, E - (int)blockIdx.x * kEqbCols);
    uint32_t* zn = pa.zero_next + (size_t)blockIdx.x * kEqbCols * 256;
    for (int i = threadIdx.x; i < ncols * 256; i += kEqbThreads) zn[i] = 0u;
  }
  if (SCAN && PASS > 0) {
    // the prefix of this pass: wave w selects the bins of columns w, w + 8,
    // ..., with the loads of all its columns in flight together
    constexpr int kPer = kEqbCols / kEqbWaves;
    uint4 v[kPer];
    uint32_t p_in[kPer], r_in[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ee = blockIdx.x * kEqbCols + w + kEqbWaves * i;
      if (ee < E) {
        v[i] = reinterpret_cast<const uint4*>(pa.hist_prev + (size_t)ee * 256)[lane];
        p_in[i] = pa.st_in ? pa.st_in[ee] : 0u;
        r_in[i] = pa.st_in ? pa.st_in[E + ee] : pa.rank0;
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = w + kEqbWaves * i;
      const int ee = blockIdx.x * kEqbCols + c;
      if (ee >= E) break;  // uniform over the wave
      uint32_t bin, nr;
      select_bin_v(v[i], r_in[i], bin, nr);
      const uint32_t p_out = (PASS == 1) ? bin : ((p_in[i] << 8) | bin);
      if (lane == 0) {
        want_s[c] = p_out;
        if (blockIdx.y == 0) {
          pa.st_out[ee] = p_out;
          pa.st_out[E + ee] = nr;
        }
      }
    }
  }
  __syncthreads();

  // Lane l of a wave: row (l >> 4) of the wave's current quad of rows, and
  // the four columns 4 (l & 15) .. +3 of the block's 64 (one 16-byte load).
  const int g = lane & 15;
  const int rq = lane >> 4;
  const int c0 = 4 * g;
  const int e0 = blockIdx.x * kEqbCols + c0;
  constexpr int shift = KB - 8 * (PASS + 1);
  bool col_ok[4];
  uint32_t want[4];
  int lo[4], hi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    col_ok[j] = e0 + j < E;
    want[j] = (PASS > 0 && col_ok[j]) ? (SCAN ? want_s[c0 + j] : pa.prefix[e0 + j]) : 0u;
    lo[j] = 256;
    hi[j] = -1;
  }
  auto bump = [&](int j, uint32_t key) {  // key: the KB-bit order key of one value
    if (PASS == 0 || (key >> (shift + 8)) == want[j]) {
      const int b = (int)((key >> shift) & 0xFFu);
      atomicAdd(lh + (c0 + j) * kEqbPad + b, 1u);
      lo[j] = min(lo[j], b);
      hi[j] = max(hi[j], b);
    }
  };
  auto load4 = [&](int64_t t, float (&v)[4]) {
    const float* zr = Z + t * (int64_t)E + e0;
    if constexpr (VEC) {
      // E % 4 == 0: a column quad is either inside E or past it
      const float4 q = col_ok[0] ? *reinterpret_cast<const float4*>(zr)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = col_ok[j] ? zr[j] : 0.0f;
    }
  };
  auto count = [&](const float (&z)[4], float al, bool row_ok) {
    if (!row_ok) return;
    if constexpr (KB == 16) {
      // two values per conversion (v_cvt_pk_bf16_f32, round to nearest even)
      // and per packed key
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const bf16x2_t bb = {(__bf16)(z[j] + al), (__bf16)(z[j + 1] + al)};
        const uint32_t k2 = bf16_order_key2(__builtin_bit_cast(uint32_t, bb));
        if (col_ok[j]) bump(j, k2 & 0xFFFFu);
        if (col_ok[j + 1]) bump(j + 1, k2 >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (col_ok[j]) bump(j, f32_order_key(z[j] + al));
    }
  };
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(N, r0 + rows_per_block);
  const int64_t nq = (r1 - r0 + 3) / 4;  // quads of rows of the block (the last may be partial)
  int64_t q = w;
  // trips of kEqbQuadUnroll quads per wave (quads w, w + 8, ...): the loads of
  // the whole trip are issued first
  for (; q + (int64_t)kEqbWaves * (kEqbQuadUnroll - 1) < nq; q += kEqbWaves * kEqbQuadUnroll) {
    float z[kEqbQuadUnroll][4], al[kEqbQuadUnroll];
    bool rok[kEqbQuadUnroll];
#pragma unroll
    for (int u = 0; u < kEqbQuadUnroll; ++u) {
      const int64_t t = r0 + 4 * (q + kEqbWaves * u) + rq;
      rok[u] = t < r1;
      const int64_t ts = rok[u] ? t : r0;
      load4(ts, z[u]);
      al[u] = alpha[ts];
    }
#pragma unroll
    for (int u = 0; u < kEqbQuadUnroll; ++u) count(z[u], al[u], rok[u]);
  }
  for (; q < nq; q += kEqbWaves) {
    const int64_t t = r0 + 4 * q + rq;
    const bool rok = t < r1;
    const int64_t ts = rok ? t : r0;
    float z[4];
    load4(ts, z);
    count(z, alpha[ts], rok);
  }
  // the touched bin range of each column over the four rows of a lane quad,
  // then over the waves (flush below)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo[j] = min(lo[j], __shfl_xor(lo[j], 16));
    lo[j] = min(lo[j], __shfl_xor(lo[j], 32));
    hi[j] = max(hi[j], __shfl_xor(hi[j], 16));
    hi[j] = max(hi[j], __shfl_xor(hi[j], 32));
  }
  if (rq == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo_s[w][c0 + j] = lo[j];
      hi_s[w][c0 + j] = hi[j];
    }
  }
  __syncthreads();
  // flush: wave w takes columns w, w+8, ...; its lanes walk the touched bins
  for (int c = w; c < kEqbCols; c += kEqbWaves) {
    const int ee = blockIdx.x * kEqbCols + c;
    if (ee >= E) break;
    int clo = lo_s[0][c], chi = hi_s[0][c];
#pragma unroll
    for (int q2 = 1; q2 < kEqbWaves; ++q2) {
      clo = min(clo, lo_s[q2][c]);
      chi = max(chi, hi_s[q2][c]);
    }
    for (int b = clo + lane; b <= chi; b += 64) {
      const uint32_t cnt = lh[c * kEqbPad + b];
      if (cnt != 0u) atomicAdd(hist + (size_t)ee * 256 + b, cnt);
    }
  }
}

// One wave per expert (parts path).  rank0 is the wanted 1-based rank for
// pass 0 (r+1).  In the last pass the quantile is decoded into qraw (and
// quantile_out).
__global__ __launch_bounds__(256) void eqb_scan_kernel(
    const uint32_t* __restrict__ hist, uint32_t* __restrict__ prefix,
    uint32_t* __restrict__ rank, int E, int pass, int last, int key_bits,
    uint32_t rank0, float* __restrict__ qraw, float* __restrict__ quantile_out) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (e >= E) return;
  const uint32_t want = (pass == 0) ? rank0 : rank[e];
  uint32_t bin, new_rank;
  select_bin(hist + (size_t)e * 256, want, bin, new_rank);
  if (lane == 0) {
    const uint32_t p = ((pass == 0) ? 0u : (prefix[e] << 8)) | bin;
    prefix[e] = p;
    rank[e] = new_rank;
    if (last) {
      const float q = quantile_from_key(p, key_bits);
      qraw[e] = q;
      if (quantile_out) quantile_out[e] = q;
    }
  }
}

// Centring of the raw biases -Q_e: their fp64 sum in expert order (formed by
// block_raw_bias_mean), every thread writes fp32(fp64(-Q_e) - mean).  A kernel of its own
// (one block) after the last scan, so the quantiles of all scan blocks are
// visible without device-wide fences.
__global__ __launch_bounds__(256) void eqb_centre_kernel(const float* __restrict__ qraw, int E,
                                                         float* __restrict__ beta_out) {
  __shared__ float q_s[kEqbMaxE];
  for (int i = threadIdx.x; i < E; i += blockDim.x) q_s[i] = qraw[i];
  __syncthreads();
  const double mean = block_raw_bias_mean<256>(q_s, E);
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    beta_out[i] = (float)((double)(-q_s[i]) - mean);
}

// Last pass of a whole-batch update: one wave per expert selects the last
// byte of its key from the last histogram (state st_in from the pass before)
// and decodes the quantile into qraw (and quantile_out); eqb_centre_kernel
// then centres the biases.
__global__ __launch_bounds__(256) void eqb_last_kernel(
    const uint32_t* __restrict__ hist_last, const uint32_t* __restrict__ st_in, int E,
    int key_bits, float* __restrict__ qraw, float* __restrict__ quantile_out) {
  const int ee = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (ee >= E) return;  // whole wave
  uint32_t bin, nr;
  select_bin(hist_last + (size_t)ee * 256, st_in[E + ee], bin, nr);
  if (lane_id() == 0) {
    const float q = quantile_from_key((st_in[ee] << 8) | bin, key_bits);
    qraw[ee] = q;
    if (quantile_out) quantile_out[ee] = q;
  }
}

static int64_t eqb_rows_per_block(int64_t N, int E) {
  const int col_groups = (E + kEqbCols - 1) / kEqbCols;
  // one block per CU of the 256: each row slab's block flushes its LDS
  // histogram into the global one with device-scope atomics, whose number
  // grows with the number of slabs, and one block of 8 waves keeps enough
  // loads in flight
  const int64_t chunks = 256 / col_groups;
  int64_t rows_per_block = (N + chunks - 1) / chunks;
  if (rows_per_block < 128) rows_per_block = 128;
  constexpr int64_t kStep = 4 * kEqbWaves;  // rows of one step of the block
  return (rows_per_block + kStep - 1) / kStep * kStep;
}

template <bool SCAN>
static hipError_t launch_hist(const float* Z, const float* alpha, int64_t N, int E, int key_bits,
                              int pass, const EqbPassArgs& pa, uint32_t* hist_pass,
                              hipStream_t stream) {
  const int col_groups = (E + kEqbCols - 1) / kEqbCols;
  const int64_t rows_per_block = eqb_rows_per_block(N, E);
  const int64_t chunks = (N + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)col_groups, (unsigned)chunks), block(kEqbThreads);
  const bool vec = E % 4 == 0 && (uintptr_t)Z % 16 == 0;
#define MOE_EQB_HIST(KB, P)                                                                    \
  do {                                                                                         \
    if (vec)                                                                                   \
      hipLaunchKernelGGL((eqb_hist_kernel<KB, P, SCAN, true>), grid, block, 0, stream, Z,      \
                         alpha, N, E, rows_per_block, pa, hist_pass);                          \
    else                                                                                       \
      hipLaunchKernelGGL((eqb_hist_kernel<KB, P, SCAN, false>), grid, block, 0, stream, Z,     \
                         alpha, N, E, rows_per_block, pa, hist_pass);                          \
  } while (0)
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

hipError_t launch_eqb_hist(const float* Z, const float* alpha, int64_t N, int E, int key_bits,
                           int pass, const uint32_t* prefix, uint32_t* hist_pass,
                           hipStream_t stream) {
  EqbPassArgs pa{};
  pa.prefix = prefix;
  return launch_hist<false>(Z, alpha, N, E, key_bits, pass, pa, hist_pass, stream);
}

hipError_t launch_eqb_centre(const float* qraw, int E, float* beta_out, hipStream_t stream) {
  hipLaunchKernelGGL(eqb_centre_kernel, dim3(1), dim3(256), 0, stream, qraw, E, beta_out);
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
                      const EqbWork& w, hipStream_t stream, bool hist0_zeroed) {
  const int passes = key_bits / 8;
  const int64_t r = (N * (int64_t)K) / E;
  const size_t per = (size_t)E * 256;
  if (!hist0_zeroed) {
    hipError_t err = launch_fill_u32(w.hist, 0u, per, stream);
    if (err != hipSuccess) return err;
  }
  uint32_t* st[2] = {w.state + 2 * E, w.state + 4 * E};
  for (int p = 0; p < passes; ++p) {
    EqbPassArgs pa{};
    pa.hist_prev = p > 0 ? w.hist + (size_t)(p - 1) * per : nullptr;
    pa.st_in = p > 1 ? st[(p - 1) & 1] : nullptr;
    pa.st_out = st[p & 1];
    pa.zero_next = p + 1 < passes ? w.hist + (size_t)(p + 1) * per : nullptr;
    pa.rank0 = (uint32_t)(r + 1);
    hipError_t err = launch_hist<true>(Z, alpha, N, E, key_bits, p, pa, w.hist + (size_t)p * per,
                                       stream);
    if (err != hipSuccess) return err;
  }
  // the last byte: state of the last histogram pass (or rank r + 1 with one
  // pass, which 16- and 32-bit keys never have)
  hipLaunchKernelGGL(eqb_last_kernel, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, stream,
                     w.hist + (size_t)(passes - 1) * per, st[(passes - 1) & 1], E, key_bits,
                     w.qraw, quantile_out);
  if (beta_out)
    hipLaunchKernelGGL(eqb_centre_kernel, dim3(1), dim3(256), 0, stream, w.qraw, E, beta_out);
  return hipGetLastError();
}

}  // namespace moe
