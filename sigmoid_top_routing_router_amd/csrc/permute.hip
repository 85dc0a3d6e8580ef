// Grouping of the (token, slot) pairs by expert: a stable counting sort.
//
// The routing equations of "Kolibri Pre-Training from Scratch" §6.1 send
// token t to the experts I_t; the German guide "Kolibri 1 im Detail"
// (section on routing) notes that tokens have to be brought to their experts
// with no per-expert capacity.  On one GPU that is a permutation of the N*K
// pairs into contiguous per-expert segments, tokens ascending within each
// segment (pair index t*K+k; the K experts of a token are distinct, so this
// is also the order of t).
//
// Kernels (all integer work, bit-exact and deterministic); batches of at most
// 16384 pairs use perm_small_kernel, one block doing all four steps.  Larger
// batches take two launches.  The pairs are cut into blocks of four chunks,
// one chunk of cw consecutive pairs per wave (cw grows with the batch so that
// there are at most kPermMaxBlocks blocks):
//  1. perm_count_kernel: block b counts the experts of its pairs in LDS ->
//     block_counts[b][e].
//  2. perm_scatter_kernel: every block reads the whole count table (at most
//     kPermMaxBlocks x E words), which gives it each expert's total and the
//     pairs of that expert in the blocks before it; a block-wide scan in
//     expert order turns the totals into the segment offsets, and block 0
//     writes counts, offsets and the table of m-tiles (expert, first row,
//     rows) that drives the grouped GEMMs from device memory.  A segment is
//     cut into tiles of bm rows, except that its last tile takes up to
//     bm + xr rows: a remainder of at most xr rows rides with the tile before
//     it instead of streaming the expert's weights once more.  Each wave then
//     counts its own chunk again, which places the four chunks inside the
//     block, and walks its pairs in order, 64 at a time; lanes holding the
//     same expert are found with nine ballots over the bits of the expert
//     id, so the rank among them is a popcount and the lowest such lane
//     advances the expert's running position in LDS.
// The scan and the tile table ride in the scatter launch instead of two
// launches of their own: each launch in this dependent chain waits for free
// CUs while the shared expert's GEMM blocks hold them.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kChunkMin = 512;      // pairs per chunk (one wave), at least
constexpr int kPermWaves = 4;       // waves (chunks) per block
constexpr int kPermMaxBlocks = 64;  // blocks of the two chunk kernels, at most
constexpr int kMaxE = 384;

// Pairs per chunk: 512, or more so that the batch needs at most
// kPermMaxBlocks blocks; a multiple of 64.
static int64_t perm_chunk(int64_t pairs) {
  const int64_t per = (pairs + kPermWaves * kPermMaxBlocks - 1) / (kPermWaves * kPermMaxBlocks);
  const int64_t cw = (per + 63) / 64 * 64;
  return cw < kChunkMin ? kChunkMin : cw;
}
int64_t perm_count_rows(int64_t pairs) {
  const int64_t bp = perm_chunk(pairs) * kPermWaves;
  return (pairs + bp - 1) / bp;
}
int64_t perm_max_tiles(int64_t pairs, int E, int bm) { return pairs / bm + E; }

// Number of m-tiles of a segment of c rows: bm rows each, the last one up to
// bm + xr rows (never more tiles than ceil(c / bm)).
__device__ __forceinline__ uint32_t seg_tiles(uint32_t c, int bm, int xr) {
  if (c == 0u) return 0u;
  if (c <= (uint32_t)(bm + xr)) return 1u;
  return (c - (uint32_t)xr + (uint32_t)bm - 1u) / (uint32_t)bm;
}

// Writes the nt m-tiles of expert e (segment start off, c rows) at t0.
__device__ __forceinline__ void emit_tiles(int32_t* tiles, uint32_t t0, int e, uint32_t off,
                                           uint32_t c, uint32_t nt, int bm) {
  for (uint32_t i = 0; i < nt; ++i) {
    const uint32_t r = i * (uint32_t)bm;
    int4 ent;
    ent.x = e;
    ent.y = (int32_t)(off + r);
    ent.z = (int32_t)(i + 1 == nt ? c - r : (uint32_t)bm);
    ent.w = (int32_t)r;
    reinterpret_cast<int4*>(tiles)[t0 + i] = ent;
  }
}

__global__ __launch_bounds__(256) void perm_count_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int E, int64_t cw,
    uint32_t* __restrict__ block_counts) {
  __shared__ uint32_t cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0u;
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kPermWaves * cw;
  const int64_t i1 = min(pairs, i0 + kPermWaves * cw);
  for (int64_t i = i0 + threadIdx.x; i < i1; i += blockDim.x) atomicAdd(&cnt[ids[i]], 1u);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    block_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int E, int64_t cw, int64_t n_blocks,
    const uint32_t* __restrict__ block_counts, int bm, int xr, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ sorted_src, int32_t* __restrict__ src_pos) {
  __shared__ uint32_t pos[kPermWaves][kMaxE];  // chunk counts, then chunk bases
  __shared__ uint32_t base_s[kMaxE];           // segment start + pairs of earlier blocks
  __shared__ uint32_t wsum_c[4], wsum_t[4];
  const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
  const int64_t b = blockIdx.x;
  const int64_t i0 = (b * kPermWaves + w) * cw;
  const int64_t i1 = min(pairs, i0 + cw);
  for (int e = lane; e < E; e += kWave) pos[w][e] = 0u;
  __builtin_amdgcn_wave_barrier();
  for (int64_t i = i0 + lane; i < i1; i += kWave) atomicAdd(&pos[w][ids[i]], 1u);

  // Totals and earlier-block sums of experts 2 tid and 2 tid + 1 (E <= 512),
  // so that the block-wide scan below runs in expert order.
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  uint32_t tot0 = 0u, tot1 = 0u, pre0 = 0u, pre1 = 0u;
  if (e0 < E) {
    const bool two = e1 < E;
    int64_t r = 0;
    for (; r + 8 <= n_blocks; r += 8) {
      uint32_t v0[8], v1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t* row = block_counts + (size_t)(r + j) * E;
        v0[j] = row[e0];
        v1[j] = two ? row[e1] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot0 += v0[j];
        tot1 += v1[j];
        if (r + j < b) { pre0 += v0[j]; pre1 += v1[j]; }
      }
    }
    for (; r < n_blocks; ++r) {
      const uint32_t* row = block_counts + (size_t)r * E;
      const uint32_t v0 = row[e0], v1 = two ? row[e1] : 0u;
      tot0 += v0;
      tot1 += v1;
      if (r < b) { pre0 += v0; pre1 += v1; }
    }
  }
  const uint32_t t0 = seg_tiles(tot0, bm, xr), t1 = seg_tiles(tot1, bm, xr);
  const uint32_t ic = wave_inclusive_sum_u32(tot0 + tot1);
  const uint32_t it = wave_inclusive_sum_u32(t0 + t1);
  if (lane == kWave - 1) { wsum_c[w] = ic; wsum_t[w] = it; }
  __syncthreads();
  uint32_t bc = 0, bt = 0;
  for (int i = 0; i < w; ++i) { bc += wsum_c[i]; bt += wsum_t[i]; }
  const uint32_t off0 = bc + ic - (tot0 + tot1), toff0 = bt + it - (t0 + t1);
  if (b == 0) {
    if (tid == 255) {
      offsets[E] = (int32_t)(bc + ic);
      *n_tiles = (int32_t)(bt + it);
    }
    if (e0 < E) {
      counts[e0] = (int32_t)tot0;
      offsets[e0] = (int32_t)off0;
      emit_tiles(tiles, toff0, e0, off0, tot0, t0, bm);
    }
    if (e1 < E) {
      counts[e1] = (int32_t)tot1;
      offsets[e1] = (int32_t)(off0 + tot0);
      emit_tiles(tiles, toff0 + t0, e1, off0 + tot0, tot1, t1, bm);
    }
  }
  if (e0 < E) base_s[e0] = off0 + pre0;
  if (e1 < E) base_s[e1] = off0 + tot0 + pre1;
  __syncthreads();
  // the four chunks of the block in order inside each expert's run
  for (int e = tid; e < E; e += blockDim.x) {
    uint32_t run = base_s[e];
#pragma unroll
    for (int q = 0; q < kPermWaves; ++q) {
      const uint32_t c = pos[q][e];
      pos[q][e] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int64_t j = i0; j < i1; j += kWave) {
    const int64_t i = j + lane;
    const bool ok = i < i1;
    const uint32_t e = ok ? (uint32_t)ids[i] : 0u;
    uint64_t mask = ballot(ok);
#pragma unroll
    for (int bit_i = 0; bit_i < 9; ++bit_i) {
      const bool bit = (e >> bit_i) & 1u;
      const uint64_t bb = ballot(bit);
      mask &= bit ? bb : ~bb;
    }
    const uint64_t lower = mask & lanemask_lt();
    if (ok) {
      const uint32_t dst = pos[w][e] + (uint32_t)__popcll(lower);
      sorted_src[dst] = (int32_t)i;
      src_pos[i] = (int32_t)dst;
    }
    __builtin_amdgcn_wave_barrier();
    if (ok && lower == 0ull) pos[w][e] += (uint32_t)__popcll(mask);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ ids,
                                                    int64_t pairs, int E,
                                                    int32_t* __restrict__ counts) {
  __shared__ uint32_t cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0u;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs; i += stride) {
    const int32_t e = ids[i];
    if ((uint32_t)e < (uint32_t)E) atomicAdd(&cnt[e], 1u);  // ids outside [0,E) are not counted
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (cnt[e]) atomicAdd((uint32_t*)counts + e, cnt[e]);
}

// Small batches (pairs <= kSmallPairs): the whole stable counting sort in one
// block of 16 waves.  Wave w owns the contiguous chunk of pairs
// [w*len, (w+1)*len): (1) it counts its chunk's experts into LDS; (2) thread e
// walks the 16 wave counts of expert e in order, giving each wave its base
// inside the expert's segment, and the expert totals; (3) a block-wide scan
// gives the offsets and the m-tile table; (4) each wave scatters its chunk in
// order, 64 pairs at a time, with the same nine-ballot ranking as
// perm_scatter_kernel.  One launch instead of four.
constexpr int kSmallWaves = 16;
constexpr int64_t kSmallPairs = 16384;

__global__ __launch_bounds__(1024) void perm_small_kernel(
    const int32_t* __restrict__ ids, int64_t pairs, int E, int bm, int xr,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_src, int32_t* __restrict__ src_pos,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, int shared_rows) {
  __shared__ uint32_t wcnt[kSmallWaves][kMaxE];  // counts, then bases per wave
  __shared__ uint32_t tot[kMaxE];
  __shared__ uint32_t wsum_c[kSmallWaves], wsum_t[kSmallWaves];
  const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
  const int64_t len = (pairs + kSmallWaves - 1) / kSmallWaves;
  const int64_t i0 = (int64_t)w * len;
  const int64_t i1 = min(pairs, i0 + len);
  for (int i = tid; i < kSmallWaves * kMaxE; i += blockDim.x) (&wcnt[0][0])[i] = 0u;
  __syncthreads();
  for (int64_t i = i0 + lane; i < i1; i += kWave) atomicAdd(&wcnt[w][ids[i]], 1u);
  __syncthreads();
  // (2) bases of the waves inside each expert's segment (exclusive), totals
  for (int e = tid; e < E; e += blockDim.x) {
    uint32_t run = 0;
    for (int q = 0; q < kSmallWaves; ++q) {
      const uint32_t c = wcnt[q][e];
      wcnt[q][e] = run;
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();
  // (3) offsets and the m-tile table: a scan in expert order; E <= 384 fits
  // one expert per thread of the first 384 threads (7 waves)
  const uint32_t c = tid < E ? tot[tid] : 0u;
  const uint32_t t = seg_tiles(c, bm, xr);
  const uint32_t ic = wave_inclusive_sum_u32(c);
  const uint32_t it = wave_inclusive_sum_u32(t);
  if (lane == kWave - 1) { wsum_c[w] = ic; wsum_t[w] = it; }
  __syncthreads();
  uint32_t bc = 0, bt = 0;
  for (int q = 0; q < w; ++q) { bc += wsum_c[q]; bt += wsum_t[q]; }
  const uint32_t off = bc + ic - c;
  uint32_t toff = bt + it - t;
  if (tid == blockDim.x - 1) {
    offsets[E] = (int32_t)(bc + ic);
    // the shared expert's tiles after the routed ones, 16 rows each: the
    // weight-streaming kernel streams a tile's weights once per 16 rows, so
    // a 64-row tile would take one block four times as long as the others
    uint32_t nt = bt + it;
    for (int r = 0; r < shared_rows; r += 16)
      reinterpret_cast<int4*>(tiles)[nt++] =
          make_int4(-1, (int32_t)(pairs + r), min(16, shared_rows - r), r);
    *n_tiles = (int32_t)nt;
  }
  if (tid < E) {
    counts[tid] = (int32_t)c;
    offsets[tid] = (int32_t)off;
    emit_tiles(tiles, toff, tid, off, c, t, bm);
    tot[tid] = off;  // segment starts, for the scatter
  }
  __syncthreads();
  // (4) scatter, each wave its chunk in order
  for (int e = lane; e < E; e += kWave) wcnt[w][e] += tot[e];
  __builtin_amdgcn_wave_barrier();
  for (int64_t j = i0; j < i1; j += kWave) {
    const int64_t i = j + lane;
    const bool ok = i < i1;
    const uint32_t e = ok ? (uint32_t)ids[i] : 0u;
    uint64_t mask = ballot(ok);
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (e >> b) & 1u;
      const uint64_t bb = ballot(bit);
      mask &= bit ? bb : ~bb;
    }
    const uint64_t lower = mask & lanemask_lt();
    if (ok) {
      const uint32_t dst = wcnt[w][e] + (uint32_t)__popcll(lower);
      sorted_src[dst] = (int32_t)i;
      src_pos[i] = (int32_t)dst;
    }
    __builtin_amdgcn_wave_barrier();
    if (ok && lower == 0ull) wcnt[w][e] += (uint32_t)__popcll(mask);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_permute(const int32_t* ids, int64_t N, int E, int K, int bm, int xr,
                          const PermWork& w, hipStream_t stream, int shared_rows) {
  const int64_t pairs = N * (int64_t)K;
  if (pairs <= kSmallPairs) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), 0, stream, ids, pairs, E, bm, xr,
                       w.counts, w.offsets, w.sorted_src, w.src_pos, w.tiles, w.n_tiles,
                       shared_rows);
    return hipGetLastError();
  }
  if (shared_rows > 0) return hipErrorInvalidValue;
  const int64_t cw = perm_chunk(pairs);
  const int64_t n_blocks = perm_count_rows(pairs);
  const dim3 grid((unsigned)n_blocks), block(256);
  hipLaunchKernelGGL(perm_count_kernel, grid, block, 0, stream, ids, pairs, E, cw,
                     w.block_counts);
  hipLaunchKernelGGL(perm_scatter_kernel, grid, block, 0, stream, ids, pairs, E, cw, n_blocks,
                     w.block_counts, bm, xr, w.counts, w.offsets, w.tiles, w.n_tiles,
                     w.sorted_src, w.src_pos);
  return hipGetLastError();
}

hipError_t launch_count(const int32_t* ids, int64_t pairs, int E, int32_t* counts,
                        hipStream_t stream) {
  hipError_t err = launch_fill_u32((uint32_t*)counts, 0u, (size_t)E, stream);
  if (err != hipSuccess) return err;
  int64_t blocks = (pairs + 4095) / 4096;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(count_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ids, pairs, E,
                     counts);
  return hipGetLastError();
}

}  // namespace moe
