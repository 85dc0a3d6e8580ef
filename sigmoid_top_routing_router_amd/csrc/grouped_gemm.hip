// bf16 MFMA GEMMs of the MoE layer on gfx950: router logits, grouped SwiGLU
// gate/up and grouped down projection over ragged expert segments.
//
// Expert MLP ("Kolibri 1 im Detail", section on routing, SwiGLU paragraph):
// two d -> h projections give SiLU(gate) * up, then one h -> d projection; no
// biases.  Router ("Kolibri 1 im Detail", same section): bf16 weights, fp32
// logits [N, E].
//
// All three products have both operands K-contiguous (x[N,d] with W[h,d];
// H[rows,h] with W_down[d,h]; x with W_r[E,d]), so one tile engine serves
// them:
//  * Block tile 256 (rows) x 256 (rows of the B operand) x 64 (k), 8 waves as
//    2 (rows) x 4 (columns), two waves per SIMD; each wave owns 128 x 64
//    outputs as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16 (128 fp32 per
//    lane), so one wave's LDS reads and loads overlap the other's MFMAs.  The
//    256 x 256 tile is what bounds the operand traffic from L2 per flop (the
//    CU's register file holds at most this many fp32 accumulators).
//  * Operands move global -> LDS with the gfx950 LDS-DMA load in its buffer
//    form (buffer_load_dwordx4 ... lds: 64 lanes x 16 bytes per instruction,
//    no VGPR staging), 8 rows x 128 bytes per instruction: every row access is one
//    whole 128-byte cache line, which on this chip moves about twice the
//    bytes per second of half-line accesses.  All 160 KB of LDS hold operand
//    slots of 32 KB: two for A and three for B (the weights, whose first
//    touch usually misses L2), so the A loads run one stage and the B loads
//    two stages ahead of the MFMAs.  Loads are retired with explicit vmcnt
//    waits plus a bare s_barrier so the compiler does not drain outstanding
//    loads at every barrier.
//  * LDS rows are 128 bytes (64 bf16); the eight 16-byte chunks of row r sit
//    at slot c ^ ((r >> 1) & 7).  The LDS serves a 16-byte read for 16 lanes
//    per cycle from 64 four-byte banks (256 bytes), i.e. from two adjacent
//    rows; 16 consecutive rows with one chunk then fall on 16 distinct
//    16-byte bank groups (even and odd rows on the two halves, (r >> 1) & 7
//    spreading each half), so the fragment reads are free of bank conflicts.
//    The swizzle is applied on the global side (each lane picks the chunk
//    that belongs in its fixed LDS slot).
//  * Within a stage the fragments of k-step s+1 are read from LDS while the
//    MFMAs of k-step s run (two fragment register sets).
//  * Gate/up: the B tile holds 128 gate rows then the 128 up rows of the same
//    hidden columns; each wave takes 64 of each, so SiLU(g) * u is formed in
//    registers (the lane layouts of the two accumulators coincide) and H is
//    written once in bf16.  The gathered token rows of x are loaded directly
//    into the A tile (the permuted copy of x is never built).
//  * Epilogue: bf16 results (H, Y) are converted in registers (hardware
//    round-to-nearest-even), staged row-major in the then idle LDS and written
//    as whole 16-byte row chunks; router logits are stored directly in fp32.
//  * Ragged segments: an m-tile table (expert, first row, rows) produced on
//    the device by the grouping kernels drives the grid; the grid is sized
//    for the worst case and surplus blocks exit after reading the tile count.
//    The last tile of a segment may hold up to 288 rows; such tiles run a
//    variant with 288-row A slots (see gemm_tile).
//    Waves skip the MFMAs of 32-row blocks that hold no valid rows; rows past
//    the segment (and B rows past the matrix) load zeros through an offset
//    beyond the buffer and are never stored.
//  * XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
//    block b works on the logical tile (b % 8) * share + b / 8; each XCD then
//    walks a contiguous run of (m-tile, n-tile) pairs, n fastest, and the
//    blocks that share an A tile or an expert's weights meet in that XCD's
//    L2.
#include <type_traits>

#include "common.h"
#include "gemm_args.h"
#include "kernels.h"

namespace moe {

constexpr int BM = 256;
constexpr int BN = kTileN;
constexpr int BK = 64;
constexpr int A_SLOTS = 2;                           // A ring: stages kt, kt+1
constexpr int B_SLOTS = 3;                           // B ring: stages kt .. kt+2
constexpr int ROW_BYTES = BK * 2;                    // 128
constexpr int TILE_BYTES = BM * ROW_BYTES;           // 32 KB per operand and stage
constexpr int B_RING = A_SLOTS * TILE_BYTES;         // byte offset of the B ring
constexpr int LDS_BYTES = (A_SLOTS + B_SLOTS) * TILE_BYTES;  // 160 KB
constexpr int kXcd = 8;

constexpr int kXRows = 32;                           // extra rows of a grouped tile

int gemm_bm() { return BM; }
int gemm_xrows() { return kXRows; }

__device__ __forceinline__ void wait_all_mem() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint16_t f32_to_bf16_u16(float v) {
  return (uint16_t)f32_to_bf16_rne_bits(v);
}

// Logical tile of this block: workgroups are dealt round-robin to the XCDs,
// so block b takes tile (b % 8) * share + b / 8 and each XCD walks a
// contiguous run.  Returns false for surplus blocks.
__device__ __forceinline__ bool xcd_tile(int64_t work, int64_t& logical) {
  const int64_t share = (work + kXcd - 1) / kXcd;
  const int64_t local = blockIdx.x / kXcd;
  if (local >= share) return false;
  logical = (int64_t)(blockIdx.x % kXcd) * share + local;
  return logical < work;
}

// Quantised H of the E4M3 gate/up tile: the tile's fp32 values are staged in
// LDS (row stride QSTRIDE bytes); the 128 columns of a tile row are one
// 1 x 128 group (ldo % 128 == 0), held by 16 neighbouring lanes of 8 values
// each, quantised as s = amax / 448 and the E4M3 codes of
// min(max(v / s, -448), 448), straight from fp32.
constexpr int QSTRIDE = (kTileN / 2) * 4 + 16;
template <int TROWS>
__device__ __forceinline__ void epilogue_store_q(const GemmArgs& a, int nt, int64_t row0,
                                                 int rows, int tid, const char* lds_raw) {
  constexpr int CPR = (kTileN / 2) / 8;  // 8-value pieces per tile row
  const int col0 = nt * (kTileN / 2);
  uint8_t* q = reinterpret_cast<uint8_t*>(a.out);
  const int groups = (int)(a.ldo / 128);
  for (int c = tid; c < TROWS * CPR; c += 512) {
    const int rr = c / CPR, ch = c % CPR;
    if (rr >= rows) break;  // the 16 lanes of a row leave together
    const char* src = lds_raw + rr * QSTRIDE + ch * 32;
    const float4 lo = *reinterpret_cast<const float4*>(src);
    const float4 hi = *reinterpret_cast<const float4*>(src + 16);
    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(fabsf(v[j])));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    const float amax = __uint_as_float(m);
    const float sc = amax / 448.0f;
    uint32_t cw[2] = {0u, 0u};
    if (amax != 0.0f) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = fminf(fmaxf(v[4 * j + i] / sc, -448.0f), 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], pk, true);
        cw[j] = (uint32_t)pk;
      }
    }
    *reinterpret_cast<uint2*>(q + (row0 + rr) * a.ldo + col0 + ch * 8) = make_uint2(cw[0], cw[1]);
    if (ch == 0) a.out_scale[(row0 + rr) * groups + nt] = (amax != 0.0f) ? sc : 0.0f;
  }
}

// Second half of the bf16-output epilogue: the tile staged in LDS (row
// stride OSTRIDE bytes) goes to global memory in whole rows.
template <int MODE, int TROWS = BM>
__device__ __forceinline__ void epilogue_store(const GemmArgs& a, int nt, int64_t row0, int rows,
                                               int tid, const char* lds_raw) {
  constexpr int OCOLS = (MODE == kGateUp) ? BN / 2 : BN;
  constexpr int OSTRIDE = OCOLS * 2 + 8;
  constexpr int CPR = OCOLS / 8;  // 16-byte chunks per tile row
  const int col0 = nt * OCOLS;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  if constexpr (MODE == kDown) {
    // Every LDS read of the tile first, then the stores: a lane keeps one
    // 16-byte chunk column (512 % CPR == 0) and up to TROWS / 16 rows of it.
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    constexpr int ITERS = (TROWS * CPR + 511) / 512;
    const int ch = tid % CPR;
    const int col = col0 + ch * 8;
    u32x2_t lo[ITERS], hi[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int rr = (tid + it * 512) / CPR;
      if (rr < rows) {
        const char* src = lds_raw + rr * OSTRIDE + ch * 16;  // 8-byte aligned
        lo[it] = *reinterpret_cast<const u32x2_t*>(src);
        hi[it] = *reinterpret_cast<const u32x2_t*>(src + 8);
      }
    }
    if (col >= a.b_rows) return;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int rr = (tid + it * 512) / CPR;
      if (rr < rows)
        *reinterpret_cast<uint4*>(out + (row0 + rr) * a.ldo + col) =
            make_uint4(lo[it].x, lo[it].y, hi[it].x, hi[it].y);
    }
    return;
  }
  for (int c = tid; c < TROWS * CPR; c += 512) {
    const int rr = c / CPR, ch = c % CPR;
    if (rr >= rows) break;  // chunks are walked in row order
    const int col = col0 + ch * 8;
    if (col >= a.b_rows) continue;
    const char* src = lds_raw + rr * OSTRIDE + ch * 16;  // 8-byte aligned
    const uint2 lo = *reinterpret_cast<const uint2*>(src);
    const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
    *reinterpret_cast<uint4*>(out + (row0 + rr) * a.ldo + col) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// ---- selection fused into the router tile ("Kolibri Pre-Training from
// Scratch" §6.1, routing equations: the bias enters the selection only; §7.1:
// the token bias needs the (K+1)-th largest biased score).  Once the tile's
// logits are stored, the block reads them back (its own stores, visible
// after the barrier; L2 hits) 16 lanes per row, 32 rows per round, the next
// round's rows in flight while one is selected.  Each row's biased scores
// b = z + (beta + 0) (-0 becomes +0) over the tile's columns give its
// KC = K + 1 first entries in the order (score descending, expert
// ascending), as the routing kernel does over a whole row: L = the KC-th
// largest of the 16 lane maxima bounds the KC-th largest score from below,
// the candidates (score >= L, usually a few) are ranked exactly in a
// per-row LDS list, and a row with more than kSelCap candidates (many tied
// scores) pops its KC entries one by one.  Columns past E score -inf.  The
// KC first entries of a whole row are among the union of its tiles' lists,
// so a small merge finishes the selection.
constexpr int kSelCap = 64;

template <bool NARROW>
__device__ __forceinline__ void router_tile_select(const GemmArgs& a, int nt, int64_t row0,
                                                   int rows, int lane, int tid, char* lds_raw) {
  constexpr int TC = NARROW ? BN / 2 : BN;  // columns of the tile
  constexpr int NC = TC / 64;               // 4-column pieces per lane and row
  constexpr int NVL = 4 * NC;               // scores per lane and row
  static_assert(32 * kSelCap * 8 <= LDS_BYTES, "selection LDS");
  const float* Z = reinterpret_cast<const float*>(a.out);
  const int E = a.b_rows;
  const int KC = a.sel_k;
  const int col_base = nt * TC;
  const int ntn = a.n_tiles_n;
  const int rsel = tid >> 4;  // row of this thread in a round of 32
  const int g = tid & 15;     // lane within the row's 16
  const uint64_t gmask = 0xFFFFull << (16 * ((tid >> 4) & 3));
  float* cs = reinterpret_cast<float*>(lds_raw) + rsel * kSelCap;
  uint32_t* ce = reinterpret_cast<uint32_t*>(lds_raw) + 32 * kSelCap + rsel * kSelCap;
  // bias of this lane's columns; -inf marks columns past E
  float bv[NVL];
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int e = col_base + 64 * (i >> 2) + 4 * g + (i & 3);
    bv[i] = e < E ? (a.sel_beta ? a.sel_beta[e] + 0.0f : 0.0f) : -INFINITY;
  }
  const bool vec = (E & 3) == 0 && ((uintptr_t)Z & 15) == 0;
  auto load_row = [&](int r0, float (&v)[NVL]) {
    const int rl = min(r0 + rsel, rows - 1);
    const float* zr = Z + (row0 + rl) * (int64_t)E + col_base;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = 4 * g + 64 * j;
      if (vec) {
        const float4 t = col_base + c < E ? *reinterpret_cast<const float4*>(zr + c)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[4 * j + k] = col_base + c + k < E ? zr[c + k] : 0.0f;
      }
    }
  };
  __syncthreads();  // the tile's logits are stored; the fragment reads are done
  float cur[NVL], nxt[NVL];
  load_row(0, cur);
#pragma unroll 1
  for (int r0 = 0; r0 < rows; r0 += 32) {
    if (r0 + 32 < rows) load_row(r0 + 32, nxt);
    const int rl = r0 + rsel;
    const bool live = rl < rows;
    float v[NVL];
#pragma unroll
    for (int i = 0; i < NVL; ++i) v[i] = bv[i] == -INFINITY ? -INFINITY : cur[i] + bv[i];
    float* os = a.cand_s + ((row0 + rl) * ntn + nt) * KC;
    uint32_t* oe = a.cand_e + ((row0 + rl) * ntn + nt) * KC;
    // (1) lower bound L of the KC-th largest score
    float lm = v[0];
#pragma unroll
    for (int i = 1; i < NVL; ++i) lm = fmaxf(lm, v[i]);
    float L = -INFINITY;
#pragma unroll
    for (int k = 0; k <= MOE_KMAX_INTERNAL; ++k) {
      if (k >= KC) break;  // uniform
      L = row16_max_f32(lm);
      const int win = __ffsll((unsigned long long)(ballot(lm == L) & gmask)) - 1;
      if (lane == win) lm = -INFINITY;
    }
    // (2) the candidates, compacted in lane order
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < NVL; ++i) cnt += (v[i] >= L) ? 1u : 0u;
    uint32_t off = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {  // cnt <= 16
      const uint64_t mk = ballot(((cnt >> bit) & 1u) != 0u) & gmask;
      off += (uint32_t)__builtin_amdgcn_mbcnt_hi(
                 (uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u)) << bit;
      total += (uint32_t)__popcll(mk) << bit;
    }
    if (ballot(total > (uint32_t)kSelCap) == 0) {
#pragma unroll
      for (int i = 0; i < NVL; ++i) {
        if (v[i] >= L) {
          cs[off] = v[i];
          ce[off] = (uint32_t)(col_base + 64 * (i >> 2) + 4 * g + (i & 3));
          ++off;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the row's list is written
      for (uint32_t i = (uint32_t)g; i < total; i += 16) {
        const float si = cs[i];
        const uint32_t ei = ce[i];
        uint32_t rank = 0;
        for (uint32_t j = 0; j < total; ++j) {
          const float sj = cs[j];
          const uint32_t ej = ce[j];
          rank += (uint32_t)((sj > si) | ((sj == si) & (ej < ei)));
        }
        if (live && rank < (uint32_t)KC) {
          os[rank] = si;
          oe[rank] = ei;
        }
      }
    } else {
      // (2') KC pops: pop r takes the row's first (score, expert) after pop
      // r - 1.  A lane's experts rise with its slot i, so "expert after the
      // last pop's" is "slot >= k_le" among scores equal to the last pop's.
      float sp = INFINITY;
      int k_le = 0;
#pragma unroll 1
      for (int r = 0; r < KC; ++r) {
        float bs = -INFINITY;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
          const float sv = v[i];
          const bool after = r == 0 || sv < sp || (sv == sp && i >= k_le);
          const bool better = after && (sv > bs || (bi < 0 && sv == bs));
          bs = better ? sv : bs;
          bi = better ? i : bi;
        }
        const uint32_t be =
            bi >= 0 ? (uint32_t)(64 * (bi >> 2) + 4 * g + (bi & 3)) : 0xFFFFFFFFu;
        const float rmx = row16_max_f32(bs);
        const uint32_t we = row16_min_u32(bs == rmx ? be : 0xFFFFFFFFu);
        if (live && g == 0) {
          os[r] = rmx;
          oe[r] = we == 0xFFFFFFFFu ? we : (uint32_t)col_base + we;
        }
        sp = rmx;
        const int wa = (int)(we >> 6), wl = (int)((we >> 2) & 15u), wc = (int)(we & 3u);
        k_le = we == 0xFFFFFFFFu ? NVL : 4 * wa + (g < wl ? 4 : (g == wl ? wc + 1 : 0));
      }
    }
    // the row lists are read before the next round writes them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NVL; ++i) cur[i] = nxt[i];
  }
}

// Epilogue of one tile: accumulators acc[m][f] of wave (wg, wp) -> the output
// (router: fp32 logits + offset; gate/up: SiLU(g) * u in bf16; down: bf16).
template <int MODE, int XR, bool NARROW = false>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, floatx16_t (&acc)[4][2],
                                              floatx16_t& accx, int nt, int64_t row0, int rows,
                                              int lane, int wg, int wp, int tid,
                                              const int (&b_row)[2], bool any, int live_m,
                                              char* lds_raw) {
  // ---- epilogue.  The MFMAs take the B fragment as their first operand, so
  // each 32 x 32 accumulator holds the tile transposed: lane l has output row
  // (l & 31) and, for register r, output column 8*(r/4) + 4*(l/32) + r%4, i.e.
  // four consecutive columns per group of four registers.
  const int orow_l = lane & 31;
  const int ocol_l = 4 * (lane >> 5);
  if (MODE == kRouter) {
    float* Zo = reinterpret_cast<float*>(a.out);
    const bool vec = (a.ldo % 4) == 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (!any || m >= live_m) break;
      // narrow tiles: wave (wg, wp) holds rows wg*128 + (wp>>1)*64 .. +64
      const int rr = wg * 128 + (NARROW ? (wp >> 1) * 64 : 0) + m * 32 + orow_l;
      if (rr >= rows) continue;
      const int64_t orow = row0 + rr;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * (NARROW ? BN / 2 : BN) + b_row[f] + 8 * q + ocol_l;
          float z[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            z[j] = acc[m][f][4 * q + j];
            if (a.offset && col + j < a.b_rows) z[j] += a.offset[col + j];
          }
          if (vec && col + 3 < a.b_rows) {
            *reinterpret_cast<float4*>(Zo + orow * a.ldo + col) = make_float4(z[0], z[1], z[2], z[3]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (col + j < a.b_rows) Zo[orow * a.ldo + col + j] = z[j];
          }
        }
      }
    }
    // uniform: every wave takes part in the selection's barrier
    if (a.cand_s) router_tile_select<NARROW>(a, nt, row0, rows, lane, tid, lds_raw);
    return;
  }
  // bf16 outputs (H or Y) go through LDS: every wave converts its
  // accumulators (hardware round-to-nearest-even, two values per
  // instruction) and writes four consecutive columns per 8-byte LDS store
  // into a row-major tile; the row stride of 2 (mod 32) words spreads the 32
  // rows of one store over all banks.  Then the block writes whole rows with
  // 16-byte global stores.
  constexpr int OCOLS = (MODE == kGateUp) ? BN / 2 : BN;   // tile columns
  constexpr int OSTRIDE = OCOLS * 2 + 8;                   // bytes per LDS row
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  auto pack2 = [](float x, float y) {
    const bf16x2_t v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  };
  auto silu_mul = [](float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; };
  // Extra rows (XR > 0), gate/up: the gate block of rows 256.. is held by
  // wave (0, wp), the up block of the same hidden columns by wave (1, wp); the
  // latter passes its accumulators through LDS, past the staged tile.
  constexpr int kExOff = 80 * 1024;
  static_assert(XR == 0 || MODE != kGateUp || (BM + XR) * OSTRIDE <= kExOff,
                "staging overlaps the exchange area");
  static_assert((BM + XR) * OSTRIDE <= LDS_BYTES, "staged tile exceeds the LDS");
  float4* ex = reinterpret_cast<float4*>(lds_raw + kExOff) + wp * 256;
  __syncthreads();  // all fragment reads of the last stage are done
  if (any) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m >= live_m) break;
      char* lrow = lds_raw + (wg * 128 + m * 32 + orow_l) * OSTRIDE;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (MODE == kGateUp) {
          // with extra rows, waves of the second row half hold up in acc[m][0]
          float hv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v0 = acc[m][0][4 * q + j], v1 = acc[m][1][4 * q + j];
            const float g = (XR > 0 && wg) ? v1 : v0;
            const float u = (XR > 0 && wg) ? v0 : v1;
            hv[j] = silu_mul(g, u);
          }
          *reinterpret_cast<uint2*>(lrow + (wp * 32 + 8 * q + ocol_l) * 2) =
              make_uint2(pack2(hv[0], hv[1]), pack2(hv[2], hv[3]));
        } else {
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            *reinterpret_cast<uint2*>(lrow + (b_row[f] + 8 * q + ocol_l) * 2) =
                make_uint2(pack2(acc[m][f][4 * q], acc[m][f][4 * q + 1]),
                           pack2(acc[m][f][4 * q + 2], acc[m][f][4 * q + 3]));
          }
        }
      }
    }
    if constexpr (XR > 0) {
      if (MODE == kGateUp) {
        if (wg == 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            ex[q * 64 + lane] = make_float4(accx[4 * q], accx[4 * q + 1], accx[4 * q + 2],
                                            accx[4 * q + 3]);
        }
      } else {
        char* lrow = lds_raw + (BM + orow_l) * OSTRIDE;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(lrow + (b_row[0] + 8 * q + ocol_l) * 2) =
              make_uint2(pack2(accx[4 * q], accx[4 * q + 1]),
                         pack2(accx[4 * q + 2], accx[4 * q + 3]));
      }
    }
  }
  __syncthreads();
  if constexpr (XR > 0 && MODE == kGateUp) {
    if (any && wg == 0) {
      char* lrow = lds_raw + (BM + orow_l) * OSTRIDE;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 u = ex[q * 64 + lane];
        *reinterpret_cast<uint2*>(lrow + (wp * 32 + 8 * q + ocol_l) * 2) =
            make_uint2(pack2(silu_mul(accx[4 * q], u.x), silu_mul(accx[4 * q + 1], u.y)),
                       pack2(silu_mul(accx[4 * q + 2], u.z), silu_mul(accx[4 * q + 3], u.w)));
      }
    }
    __syncthreads();
  }
  epilogue_store<MODE, BM + XR>(a, nt, row0, rows, tid, lds_raw);
}

// One 256 x 256 output tile (m-tile mt, n-tile nt).  GROUPED: rows come from
// the m-tile table (routed experts); otherwise the rows are
// 0 .. rows_dense-1 (router, shared expert).
//
// XR = 32: a grouped tile of 257 .. 288 rows (the last tile of an expert
// segment, whose remainder rides along instead of streaming the expert's
// weights once more).  The A slots hold 288 rows (2 x 36 KB), which leaves
// 88 KB for B: the B ring is kept in quarters (64 B rows, 8 KB) and has 11 of
// them, so stage s occupies quarters 4s .. 4s+3 mod 11.  Each wave adds one
// 32 x 32 accumulator for rows 256 .. 287 against the B fragment it already
// holds in b_row[0] (for gate/up the waves of the second row half take the
// up rows there).  The 32 extra A rows are one more load per wave and stage,
// four rows from half of the wave's lanes.
template <int MODE, bool GROUPED, int XR = 0, bool BNT = false, bool NARROW = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int64_t mt, int nt,
                                          char* lds_raw) {
  static_assert(XR == 0 || (XR == 32 && GROUPED && MODE != kRouter), "extra rows: grouped only");
  static_assert(!NARROW || (MODE == kRouter && XR == 0), "narrow tiles: router only");
  constexpr int A_TILE = (BM + XR) * ROW_BYTES;          // bytes per A slot
  constexpr int B_BASE = A_SLOTS * A_TILE;               // byte offset of the B ring
  constexpr int QUARTER = 64 * ROW_BYTES;                // 64 B rows of one stage
  constexpr int NB_Q = XR ? 11 : 4 * B_SLOTS;            // quarters in the B ring
  constexpr int NA_LD = XR ? 5 : 4;                      // A loads per wave and stage
  static_assert(B_BASE + NB_Q * QUARTER <= LDS_BYTES, "LDS ring too large");
  // ring position of quarter j of stage kt
  auto bq = [](int kt, int j) { return XR ? (4 * kt + j) % NB_Q : (kt % B_SLOTS) * 4 + j; };
  int expert = 0;
  int64_t row0;
  int rows;
  if (GROUPED) {
    const int4 ent = reinterpret_cast<const int4*>(a.tiles)[mt];
    expert = ent.x;
    row0 = ent.y;
    rows = ent.z;
  } else {
    row0 = mt * BM;
    rows = (int)min((int64_t)BM, a.rows_dense - row0);
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7; w and w+4 share a SIMD
  const int wg = wave >> 2;           // row half of the tile
  const int wp = wave & 3;            // column quarter of the tile

  // ---- LDS-DMA assignment.  Per stage and operand each wave issues 4 loads;
  // load i covers tile rows r = 8*(8*i + wave) .. +7, lane l -> row +(l>>3),
  // LDS slot (l&7), which holds global chunk (l&7) ^ ((r >> 1) & 7); that is
  // (l&7) ^ ((4*wave + (l>>4)) & 7) for every i.  The extra A load (XR) of
  // wave w covers rows 256 + 4*w .. +3 from lanes 0-31, whose chunk is
  // (l&7) ^ ((2*w + (l>>4)) & 7).
  const int sub = lane >> 3;
  const int chunk = (lane & 7) ^ ((4 * wave + (sub >> 1)) & 7);
  // Byte offsets of each lane's 16-byte piece, fixed for the whole tile; the
  // stage's k offset goes in the scalar offset of the load.  Rows past the
  // segment and B rows past the matrix get an offset beyond the end of the
  // buffer: the load returns zeros without a memory access, and those rows
  // are never stored.
  constexpr uint32_t kNoRow = 0xFFFFFFFFu - 16u * 1024u;  // past any 4 GiB buffer
  uint32_t a_voff[NA_LD], b_voff[4];
#pragma unroll
  for (int i = 0; i < NA_LD; ++i) {
    // the extra load (XR) of wave w: rows 256 + 4w .. +3 from lanes 0-31
    const int r = (i < 4) ? 8 * (8 * i + wave) + sub : BM + 4 * wave + (sub & 3);
    const int ch = (i < 4) ? chunk : ((lane & 7) ^ ((2 * wave + (sub >> 1)) & 7));
    if (r < rows) {
      int64_t arow = row0 + r;
      if (GROUPED && a.gather) arow = a.gather[arow] / a.gather_div;
      a_voff[i] = (uint32_t)(arow * a.lda * 2) + (uint32_t)ch * 16u;
    } else {
      a_voff[i] = kNoRow;
    }
    if (i < 4) {
      // narrow tiles: B rows nt*128 .. +127 in quarters 0 and 1; quarters 2
      // and 3 load zeros without a memory access and are never read
      const int brow = (MODE == kGateUp) ? nt * (BN / 2) + (r & (BN / 2 - 1))
                       : NARROW ? (r < BN / 2 ? nt * (BN / 2) + r : a.b_rows)
                                : nt * BN + r;
      b_voff[i] = (brow < a.b_rows) ? (uint32_t)brow * a.b_row_pitch + (uint32_t)chunk * 16u
                                    : kNoRow;
    }
  }
  const uint32_t b_bytes = (uint32_t)a.b_rows * (uint32_t)a.kdim * 2u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(a.B0 + (int64_t)expert * a.b_expert_stride, b_bytes);
  const __amdgpu_buffer_rsrc_t rb1 =
      make_rsrc((MODE == kGateUp ? a.B1 : a.B0) + (int64_t)expert * a.b_expert_stride, b_bytes);
  // K tail: kdim % 64 == 32 leaves a last stage with 32 valid k.  There the
  // upper four chunks of each row are loaded from the lower four (64 bytes
  // lower), so every access stays inside its row; they are never multiplied.
  const int nk = (a.kdim + BK - 1) / BK;
  const bool k_tail = (a.kdim % BK) != 0;
  const uint32_t tail_adj = (chunk >= 4) ? 64u : 0u;
  const uint32_t tail_adj_x = (((lane & 7) ^ ((2 * wave + (sub >> 1)) & 7)) >= 4) ? 64u : 0u;
  auto voff_at = [&](uint32_t v, int ks, uint32_t adj) {
    return (k_tail && ks == nk - 1) ? v - adj : v;
  };
  // load i covers tile rows 8*(8*i + wave) .. +7; for gate/up, loads 0 and 1
  // fill the 128 gate rows of the B tile and loads 2 and 3 the up rows.
  auto dma_a = [&](int ks, int i) {
    if (i == 4) {
      // half a load: lanes 0-31 write 512 bytes (four rows); every wave
      // still issues the instruction, so the waits count the same loads
      if (lane < 32)
        dma16(ra, voff_at(a_voff[i], ks, tail_adj_x), (uint32_t)ks * (BK * 2),
              (lds_void_t*)(lds_raw + (ks % A_SLOTS) * A_TILE + (BM + 4 * wave) * ROW_BYTES));
      return;
    }
    dma16(ra, voff_at(a_voff[i], ks, tail_adj), (uint32_t)ks * (BK * 2),
          (lds_void_t*)(lds_raw + (ks % A_SLOTS) * A_TILE + (8 * i + wave) * 1024));
  };
  // B load i of stage ks fills quarter i (B rows 64*i .. +63)
  auto dma_b = [&](int ks, int i) {
    dma16<BNT ? kCpolNT : 0>((MODE == kGateUp && i >= 2) ? rb1 : rb0, voff_at(b_voff[i], ks, tail_adj),
          (uint32_t)ks * a.b_kblk_pitch,
          (lds_void_t*)(lds_raw + B_BASE + bq(ks, i) * QUARTER + wave * 1024));
  };

  // ---- accumulators: wave (wg, wp) owns rows wg*128 .. +128 and two
  // 32-column blocks of the B rows: gate/up -> gate rows wp*32 and the up
  // rows of the same hidden columns; otherwise B rows wp*64 .. +64.  With
  // extra rows, b_row[0] is the block the wave multiplies rows 256.. with:
  // the two halves of the wave's column range (down) or gate and up
  // (gate/up) are taken by the two row halves.
  floatx16_t acc[4][2];
  floatx16_t accx;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) accx[r] = 0.0f;
  int b_row[2];
  if (MODE == kGateUp) { b_row[0] = wp * 32; b_row[1] = BN / 2 + wp * 32; }
  else if (NARROW) { b_row[0] = (wp & 1) * 64; b_row[1] = (wp & 1) * 64 + 32; }
  else { b_row[0] = wp * 64; b_row[1] = wp * 64 + 32; }
  if (XR > 0 && wg == 1) { const int t = b_row[0]; b_row[0] = b_row[1]; b_row[1] = t; }
  const int fr = lane & 31;
  // first tile row of the wave: a narrow (256 x 128) tile gives each wave
  // 64 rows and 64 columns, so the waves sharing a SIMD both have work
  const int row_base = wg * 128 + (NARROW ? (wp >> 1) * 64 : 0);
  const int a_base = (row_base + fr) * ROW_BYTES;
  const int x_base = (BM + fr) * ROW_BYTES;
  const int b_off[2] = {((b_row[0] & 63) + fr) * ROW_BYTES, ((b_row[1] & 63) + fr) * ROW_BYTES};
  // fragment rows start on multiples of 32, so (row >> 1) & 7 = (l >> 1) & 7
  auto slot_of = [&](int ks) { return ((2 * ks + (lane >> 5)) ^ ((lane >> 1) & 7)) * 16; };

  constexpr int MAX_LIVE = NARROW ? 2 : 4;
  int live_m = (rows - row_base + 31) / 32;
  live_m = live_m < 0 ? 0 : (live_m > MAX_LIVE ? MAX_LIVE : live_m);
  live_m = __builtin_amdgcn_readfirstlane(live_m);
  const bool live_n = (MODE == kGateUp) ? true
                      : NARROW ? (nt * (BN / 2) + b_row[0]) < a.b_rows
                               : (nt * BN + wp * 64) < a.b_rows;
  const bool any = __builtin_amdgcn_readfirstlane((live_m > 0 && live_n) ? 1 : 0) != 0;

  typedef bf16x8_t afrag_t[4];
  typedef bf16x8_t bfrag_t[2];
  using T = std::true_type;
  using F = std::false_type;

  auto read_frags = [&](afrag_t& A, bfrag_t& B, int kt, int ks, int q, auto live_tag) {
    // fragments of quarter q (A frag q; B frag q for q < 2)
    constexpr int LIVE = decltype(live_tag)::value;
    const char* sa = lds_raw + (kt % A_SLOTS) * A_TILE;
    const int so = slot_of(ks);
    if (q < LIVE)
      A[q] = *reinterpret_cast<const bf16x8_t*>(sa + a_base + 32 * q * ROW_BYTES + so);
    if (q < 2)
      B[q] = *reinterpret_cast<const bf16x8_t*>(lds_raw + B_BASE + bq(kt, b_row[q] >> 6) * QUARTER +
                                                b_off[q] + so);
  };

  // Schedule (every wave, whatever its MFMA work).  The prologue loads A0 B0
  // A1 B1 B2.  Stage kt runs four k-steps; the barrier at its last k-step
  // releases A slot kt%2 and the B quarters of stage kt, after which the
  // loads of A(kt+2) (two instructions at once, the rest in the next stage's
  // first k-step) and of B(kt+3) (in that stage's second and third k-steps)
  // are issued, each pinned with scheduling barriers next to the LDS reads of
  // the next k-step's fragments.  Two waves share each SIMD, so one wave's
  // loads and LDS reads overlap the other's MFMAs.  With extra rows the B ring
  // is one quarter short of three stages: quarter 3 of stage kt+2 only frees
  // at the barrier of stage kt, so it is loaded in the second k-step of stage
  // kt+1, ahead of quarters 0-2 of B(kt+3), and the barrier waits for three
  // loads instead of four.
  //
  // The steady-state stages (1 <= kt <= nk-3) are compiled without any
  // branch: every condition below is a compile-time constant there, so the
  // compiler's wait counting stays exact and the MFMAs of a k-step wait only
  // for the fragments read one k-step earlier.  The first stage and the last
  // two are peeled with run-time conditions.  LIVE (0, 2 or 4) is the number
  // of 32-row accumulator blocks this wave multiplies, also a compile-time
  // constant; rows past the segment inside a live block are computed and
  // never stored.
  auto run = [&](auto live_tag) {
    constexpr int LIVE = decltype(live_tag)::value;
    constexpr int NB3 = XR ? 3 : 4;  // B(kt+3) loads issued ahead of the barrier
    afrag_t A0, A1;
    bfrag_t B0, B1;
    bf16x8_t X0, X1;  // extra-row A fragments
    auto read_x = [&](bf16x8_t& X, int kt, int ks) {
      X = *reinterpret_cast<const bf16x8_t*>(lds_raw + (kt % A_SLOTS) * A_TILE + x_base +
                                             slot_of(ks));
    };
#pragma unroll
    for (int i = 0; i < NA_LD; ++i) dma_a(0, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_b(0, i);
    if (nk > 1) {
#pragma unroll
      for (int i = 0; i < NA_LD; ++i) dma_a(1, i);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma_b(1, i);
    }
    if (nk > 2) {
#pragma unroll
      for (int i = 0; i < NB3; ++i) dma_b(2, i);
    }
    if (nk > 2) wait_vmcnt<NA_LD + 4 + NB3>();
    else if (nk > 1) wait_vmcnt<NA_LD + 4>();
    else wait_vmcnt<0>();
    block_barrier();
    if (LIVE > 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) read_frags(A0, B0, 0, 0, q, live_tag);
      if (XR > 0) read_x(X0, 0, 0);
    }
    // One stage.  The flags are bools (peeled stages) or std::integral_constant
    // (steady state):
    //   ld_a2  - loads 0,1 of A(kt+2) after the last barrier of this stage
    //   ld_a1  - the other loads of A(kt+1) in the first k-step (with extra
    //            rows also quarter 3 of B(kt+1) in the second)
    //   ld_b   - the loads of B(kt+2) in k-steps 1 and 2
    //   next   - a next stage exists (barrier + its first fragments)
    //   vmb    - at the barrier the B(kt+2) loads may still be in flight
    //   half   - the last 32 k of this stage are padding
    auto stage = [&](int kt, auto ld_a2, auto ld_a1, auto ld_b, auto next, auto vmb,
                     auto half) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        afrag_t& Ac = (ks & 1) ? A1 : A0;
        bfrag_t& Bc = (ks & 1) ? B1 : B0;
        bf16x8_t& Xc = (ks & 1) ? X1 : X0;
        afrag_t& An = (ks & 1) ? A0 : A1;
        bfrag_t& Bn = (ks & 1) ? B0 : B1;
        bf16x8_t& Xn = (ks & 1) ? X0 : X1;
        const int nkt = (ks == 3) ? kt + 1 : kt;
        const int nks = (ks == 3) ? 0 : ks + 1;
        const bool have_next = (ks < 3) || next;
        if (ks == 3 && next) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (vmb) wait_vmcnt<NB3>(); else wait_vmcnt<0>();
          block_barrier();  // every wave done with A slot kt%2 and the B quarters of kt
        }
        const bool do_mfma = !(ks >= 2 && half);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          if (ks == 3 && ld_a2) dma_a(kt + 2, h2);
          if (ks == 0 && ld_a1) {
            dma_a(kt + 1, 2 + h2);
            if (XR > 0 && h2 == 1) dma_a(kt + 1, 4);
          }
          if (XR > 0) {
            if (ks == 1 && h2 == 0 && ld_a1) dma_b(kt + 1, 3);
            if (ks == 1 && h2 == 1 && ld_b) dma_b(kt + 2, 0);
            if (ks == 2 && ld_b) dma_b(kt + 2, 1 + h2);
          } else {
            if (ks == 1 && ld_b) dma_b(kt + 2, h2);
            if (ks == 2 && ld_b) dma_b(kt + 2, 2 + h2);
          }
          if (LIVE > 0 && have_next) {
            read_frags(An, Bn, nkt, nks, 2 * h2, live_tag);
            read_frags(An, Bn, nkt, nks, 2 * h2 + 1, live_tag);
            if (XR > 0 && h2 == 1) read_x(Xn, nkt, nks);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (do_mfma) {
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              const int m = 2 * h2 + mm;
              if (m < LIVE) {
#pragma unroll
                for (int f = 0; f < 2; ++f)
                  acc[m][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bc[f], Ac[m], acc[m][f], 0, 0, 0);
              }
            }
            if (XR > 0 && h2 == 1 && LIVE > 0)
              accx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bc[0], Xc, accx, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // stage 0: its B(2) came with the prologue; A(1) and B(1) are whole
    stage(0, nk > 2, F{}, F{}, nk > 1, nk > 2, nk == 1 && k_tail);
    // steady state: 1 <= kt <= nk-3
    for (int kt = 1; kt + 2 < nk; ++kt) stage(kt, T{}, T{}, T{}, T{}, T{}, F{});
    if (nk >= 3) stage(nk - 2, F{}, T{}, F{}, T{}, F{}, F{});
    if (nk >= 2) stage(nk - 1, F{}, F{}, F{}, F{}, F{}, k_tail);
  };
  if constexpr (XR > 0) {
    // rows > 256: every wave has four live row blocks
    if (!any) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 4>{});
  } else {
    if (!any) run(std::integral_constant<int, 0>{});
    else if (!NARROW && live_m > 2) run(std::integral_constant<int, 4>{});
    else run(std::integral_constant<int, 2>{});
  }

  gemm_epilogue<MODE, XR, NARROW>(a, acc, accx, nt, row0, rows, lane, wg, wp, tid, b_row, any,
                                  live_m, lds_raw);
}

// ---------------------------------------------------------------- FP8 tiles
// The same 256 x 256 tile engine over E4M3 operands ("Kolibri 1 im Detail",
// FP8 section: 128 x 128 weight blocks with fp32 scales, activations in
// 1 x 128 groups).  A stage is 128 k: 128 bytes per row, so loads, LDS ring
// and swizzle are those of the bf16 engine, and exactly one scale block in
// k.  One v_mfma_f32_16x16x128_f8f6f4 covers the whole stage for a 16 x 16
// block, so its product (four values per lane, formed from zero) is added
// into the fp32 accumulator times s_A(row, kb) * s_B(block, kb): one scaling
// FMA per accumulator element per 128 k.  kdim is a multiple of 128.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// XR = 32: a grouped tile of 257 .. 288 rows, as in the bf16 engine: 288-row
// A slots (the 32 extra rows are one more load per wave and stage, four rows
// from half of the lanes), a B ring of 10 quarters, and one more 16-row block
// per wave (rows 256 + 16*wg ..) against the wave's four B fragments, so the
// gate and up values of those rows meet in the same lanes.
template <int MODE, bool GROUPED, int XR = 0, bool BNT = false>
__device__ __forceinline__ void gemm_tile_fp8(const GemmArgs& a, int64_t mt, int nt,
                                              char* lds_raw) {
  static_assert(MODE != kRouter, "the router product stays bf16");
  static_assert(XR == 0 || (XR == 32 && GROUPED), "extra rows: grouped only");
  int expert = 0;
  int64_t row0;
  int rows;
  if (GROUPED) {
    const int4 ent = reinterpret_cast<const int4*>(a.tiles)[mt];
    expert = ent.x;
    row0 = ent.y;
    rows = ent.z;
  } else {
    row0 = mt * BM;
    rows = (int)min((int64_t)BM, a.rows_dense - row0);
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar descriptors
  const int wg = wave >> 2;
  const int wp = wave & 3;
  const int sub = lane >> 3;
  // LDS layout of an operand row (128 bytes, eight 16-byte chunks): chunk c
  // of row r sits at slot g(c) ^ ((r >> 1) & 7), g(c) = c ^ 4 ((c >> 1) & 1),
  // so the 32-byte fragment reads below (lane l: row l & 15, chunks 2q and
  // 2q + 1 of q = l >> 4) put lanes of quads 0 and 1 (2 and 3) on different
  // banks; with the bf16 tile's c ^ ((r >> 1) & 7) they shared them (0.7
  // conflicts per LDS access).  g is its own inverse: LDS slot (l & 7) of a
  // lane's row receives global chunk g((l & 7) ^ ((r >> 1) & 7)).
  auto g_chunk = [](int c) { return c ^ (4 * ((c >> 1) & 1)); };
  const int chunk = g_chunk((lane & 7) ^ ((4 * wave + (sub >> 1)) & 7));
  constexpr uint32_t kNoRow = 0xFFFFFFFFu - 64u * 1024u;  // past any 4 GiB buffer
  constexpr int NA_LD = XR ? 5 : 4;
  uint32_t a_voff[NA_LD], b_voff[4];
#pragma unroll
  for (int i = 0; i < NA_LD; ++i) {
    // the extra load (XR) of wave w: rows 256 + 4w .. +3 from lanes 0-31
    const int r = (i < 4) ? 8 * (8 * i + wave) + sub : BM + 4 * wave + (sub & 3);
    const int ch = (i < 4) ? chunk : g_chunk((lane & 7) ^ ((2 * wave + (sub >> 1)) & 7));
    if (r < rows) {
      int64_t arow = row0 + r;
      if (GROUPED && a.gather) arow = a.gather[arow] / a.gather_div;
      a_voff[i] = (uint32_t)(arow * a.lda) + (uint32_t)ch * 16u;
    } else {
      a_voff[i] = kNoRow;
    }
    if (i < 4) {
      const int brow = (MODE == kGateUp) ? nt * (BN / 2) + (r & (BN / 2 - 1)) : nt * BN + r;
      b_voff[i] = (brow < a.b_rows) ? (uint32_t)brow * a.b_row_pitch + (uint32_t)chunk * 16u
                                    : kNoRow;
    }
  }
  const uint32_t b_bytes = (uint32_t)a.b_rows * (uint32_t)a.kdim;
  const uint8_t* A8 = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* B08 = reinterpret_cast<const uint8_t*>(a.B0);
  const uint8_t* B18 = reinterpret_cast<const uint8_t*>(MODE == kGateUp ? a.B1 : a.B0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A8, a.a_bytes);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B08 + (int64_t)expert * a.b_expert_stride, b_bytes);
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(B18 + (int64_t)expert * a.b_expert_stride, b_bytes);
  const int nk = a.kdim / 128;
  // LDS: A ring of two slots (32 KB, or 36 KB with extra rows); B ring of
  // NB_Q quarters (64 B rows, 8 KB), stage s in quarters 4s .. 4s+3 mod NB_Q;
  // then two slots of scales (with the A ring's parity): the row scales of
  // A (256, or 288 with the 32 extra rows and a copy of those), and 64
  // copies each of the two weight-block scales the tile uses.
  constexpr int A_TILE8 = (BM + XR) * ROW_BYTES;
  constexpr int QUARTER = 8 * 1024;
  constexpr int NB_Q = XR ? 10 : 11;
  constexpr int NPRE = NB_Q - 8;  // quarters of B(kt+2) free during stage kt
  constexpr int B_BASE8 = A_SLOTS * A_TILE8;
  constexpr int SC_BASE = B_BASE8 + NB_Q * QUARTER;
  constexpr int SB0_OFF = XR ? 1280 : 1024;  // in a scale slot
  constexpr int SB1_OFF = SB0_OFF + 256;
  constexpr int SC_SLOT = SB1_OFF + 256;
  constexpr int NSC = XR ? 2 : 1;            // scale loads per wave and stage
  static_assert(SC_BASE + 2 * SC_SLOT <= LDS_BYTES, "LDS layout");
  auto bq = [](int kt, int j) { return (4 * kt + j) % NB_Q; };
  auto dma_a = [&](int ks, int i) {
    if (i == 4) {
      // half a load: lanes 0-31 write 512 bytes (four rows); every wave
      // still issues the instruction, so the waits count the same loads
      if (lane < 32)
        dma16(ra, a_voff[i], (uint32_t)ks * 128u,
              (lds_void_t*)(lds_raw + (ks % A_SLOTS) * A_TILE8 + (BM + 4 * wave) * ROW_BYTES));
      return;
    }
    dma16(ra, a_voff[i], (uint32_t)ks * 128u,
          (lds_void_t*)(lds_raw + (ks % A_SLOTS) * A_TILE8 + (8 * i + wave) * 1024));
  };
  auto dma_b = [&](int ks, int i) {  // quarter i: B rows 64*i .. +63
    dma16<BNT ? kCpolNT : 0>((MODE == kGateUp && i >= 2) ? rb1 : rb0, b_voff[i], (uint32_t)ks * a.b_kblk_pitch,
          (lds_void_t*)(lds_raw + B_BASE8 + bq(ks, i) * QUARTER + wave * 1024));
  };

  // ---- accumulators: wave (wg, wp) owns tile rows wg*128 .. +128 as eight
  // 16-row blocks, and four 16-column blocks of B rows: gate/up -> gate rows
  // wp*32, wp*32+16 and the up rows of the same hidden columns; down -> B
  // rows wp*64 + 16*f.  The MFMAs take the B fragment first, so lane l holds
  // output row (l & 15) of a block and its four consecutive columns
  // 4*(l >> 4) .. +3.  With extra rows, accx holds block 256 + 16*wg.
  floatx4_t acc[8][4];
  floatx4_t accx[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) accx[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  int b_col[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
    b_col[f] = (MODE == kGateUp) ? (f >> 1) * (BN / 2) + wp * 32 + (f & 1) * 16 : wp * 64 + 16 * f;
  const int fr = lane & 15;
  const int quad = lane >> 4;

  int live_m = (rows - wg * 128 + 31) / 32;
  live_m = live_m < 0 ? 0 : (live_m > 4 ? 4 : live_m);
  live_m = __builtin_amdgcn_readfirstlane(live_m);
  const bool live_n = (MODE == kGateUp) ? true : (nt * BN + wp * 64) < a.b_rows;
  const bool any = __builtin_amdgcn_readfirstlane((live_m > 0 && live_n) ? 1 : 0) != 0;

  // ---- scales, staged through LDS with 4-byte LDS-DMA loads (the same
  // number per wave and stage, so every wave counts the same loads).  Waves
  // 0-3: lane l loads the scale of tile row 64*wave + l (through the gather
  // for the routed gate/up; rows past the segment load zero); with extra rows
  // a second load brings rows 256 + (l & 31) (lanes 32-63 repeat 0-31).
  // Waves 4, 5: the first weight-block scale of the tile (gate block nt;
  // down: the block of columns 0-127), waves 6, 7: the second (up block nt;
  // down: columns 128-255); the two waves of a pair write the same bytes, and
  // with extra rows their second load repeats the first.  Offsets fit 32
  // bits: rows * kdim < 4 GiB.
  const int nkb = nk;
  const int nblk = (a.b_rows + 127) / 128;
  uint32_t sc_voff, sc_voff_x = kNoRow;
  __amdgpu_buffer_rsrc_t rsc;
  if (wave < 4) {
    auto row_off = [&](int r) {
      if (r >= rows) return kNoRow;
      int64_t arow = row0 + r;
      if (GROUPED && a.gather) arow = a.gather[arow] / a.gather_div;
      return (uint32_t)arow * (uint32_t)nkb * 4u;
    };
    sc_voff = row_off(64 * wave + lane);
    if (XR > 0) sc_voff_x = row_off(BM + (lane & 31));
    rsc = make_rsrc(a.sa, a.a_bytes / 128u * 4u);
  } else {
    const int second = wave >= 6 ? 1 : 0;
    const int bblk = (MODE == kGateUp) ? nt : min(2 * nt + second, nblk - 1);
    const float* base = (MODE == kGateUp && second) ? a.sb1 : a.sb0;
    sc_voff = (uint32_t)(((int64_t)expert * a.sb_es + (int64_t)bblk * nkb) * 4);
    sc_voff_x = sc_voff;
    rsc = make_rsrc(base, 0xFFFFFFF0u);
  }
  auto dma_sc = [&](int ks, int which) {
    const int dst = (wave < 4) ? (which ? 1024 : wave * 256) : (wave < 6 ? SB0_OFF : SB1_OFF);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsc, (lds_void_t*)(lds_raw + SC_BASE + (ks % 2) * SC_SLOT + dst), 4,
        which ? sc_voff_x : sc_voff, (uint32_t)ks * 4u, 0, 0);
  };
  auto dma_scales = [&](int ks) {
    dma_sc(ks, 0);
    if (XR > 0) dma_sc(ks, 1);
  };

  // Schedule (the bf16 engine's, with one MFMA per 16 x 16 block and stage):
  // the prologue loads A0 B0 A1 B1 and the first NPRE quarters of B2 (with
  // the scales of stages 0 and 1).  Stage kt loads the rest of A(kt+1) and of
  // B(kt+1), then the first NPRE quarters of B(kt+2), spread over its row
  // blocks; its closing barrier waits for all but those and is followed by
  // loads 0,1 of A(kt+2) and its scales.  The steady-state stages are
  // compiled without branches, so the waits stay exact.  LIVE (0, 2 or 4) is
  // the number of 32-row halves of its rows this wave multiplies.
  auto run = [&](auto live_tag) {
    constexpr int LIVE = decltype(live_tag)::value;
    constexpr int MB = 2 * LIVE;  // 16-row blocks
    constexpr bool XB = XR > 0 && LIVE > 0;  // the extra block
    const int s0 = ((2 * quad) ^ (4 * (quad & 1)) ^ ((lane >> 1) & 7)) * 16;
    const int s1 = ((2 * quad + 1) ^ (4 * (quad & 1)) ^ ((lane >> 1) & 7)) * 16;
    // lane l reads 32 bytes of its row: chunks 2*(l>>4) and +1 at their
    // slots g(c) ^ ((row >> 1) & 7) (fragments start on multiples of 16
    // rows, so (row >> 1) & 7 = (l >> 1) & 7)
    auto frag = [&](const char* rowp) {
      typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(rowp + s0);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(rowp + s1);
      return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    i32x8_t Bf[4], Af[2];
    float sa_r[8], sa_x = 0.f, sb_r[2];
    // row of block m (8: the extra block)
    auto a_row = [&](int kt, int m) {
      const int r = (m < 8) ? wg * 128 + 16 * m + fr : BM + 16 * wg + fr;
      return lds_raw + (kt % A_SLOTS) * A_TILE8 + r * ROW_BYTES;
    };
    auto read_stage = [&](int kt) {  // B fragments, A block 0 and the scales of stage kt
      if (MB > 0) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
          Bf[f] = frag(lds_raw + B_BASE8 + bq(kt, b_col[f] >> 6) * QUARTER +
                       ((b_col[f] & 63) + fr) * ROW_BYTES);
        Af[0] = frag(a_row(kt, 0));
        const char* sc = lds_raw + SC_BASE + (kt % 2) * SC_SLOT;
#pragma unroll
        for (int m = 0; m < MB; ++m)
          sa_r[m] = *reinterpret_cast<const float*>(sc + (wg * 128 + 16 * m + fr) * 4);
        if (XB) sa_x = *reinterpret_cast<const float*>(sc + 1024 + (16 * wg + fr) * 4);
        sb_r[0] = *reinterpret_cast<const float*>(sc + SB0_OFF);
        sb_r[1] = *reinterpret_cast<const float*>(sc + SB1_OFF);
      }
    };
    auto mfma_block = [&](floatx4_t (&c)[4], const i32x8_t& A, float sa) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const floatx4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            Bf[f], A, floatx4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        const float fac = sa * sb_r[(MODE == kGateUp) ? (f >> 1) : (wp >> 1)];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[f][r] = fmaf(p[r], fac, c[f][r]);
        // keeps the compiler from sinking the FMAs below later blocks'
        // MFMAs, which would hold every product live at once
        asm volatile("" : "+v"(c[f]));
      }
    };
#pragma unroll
    for (int i = 0; i < NA_LD; ++i) dma_a(0, i);
    dma_scales(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_b(0, i);
    if (nk > 1) {
#pragma unroll
      for (int i = 0; i < NA_LD; ++i) dma_a(1, i);
      dma_scales(1);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma_b(1, i);
    }
    if (nk > 2) {
#pragma unroll
      for (int i = 0; i < NPRE; ++i) dma_b(2, i);
    }
    constexpr int STAGE_LD = NA_LD + NSC + 4;  // loads of one stage
    if (nk > 2) wait_vmcnt<STAGE_LD + NPRE>();
    else if (nk > 1) wait_vmcnt<STAGE_LD>();
    else wait_vmcnt<0>();
    block_barrier();
    read_stage(0);
    //   ld_a2 - loads 0,1 of A(kt+2) and its scales after the closing barrier
    //   ld_a1 - the other loads of A(kt+1), and quarters NPRE.. of B(kt+1)
    //   ld_b  - quarters 0 .. NPRE-1 of B(kt+2)
    //   next  - a next stage exists (barrier + its fragments)
    //   vmb   - at the barrier the B(kt+2) quarters may still be in flight
    auto stage = [&](int kt, auto ld_a2, auto ld_a1, auto ld_b, auto next, auto vmb) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        __builtin_amdgcn_sched_barrier(0);
        if (m == 1 && ld_a1) { dma_a(kt + 1, 2); dma_a(kt + 1, 3); }
        if (m == 2 && ld_a1 && XR > 0) dma_a(kt + 1, 4);
        if (NPRE == 3) {
          if (m == 3 && ld_a1) dma_b(kt + 1, 3);
          if (m == 3 && ld_b) dma_b(kt + 2, 0);
          if (m == 5 && ld_b) { dma_b(kt + 2, 1); dma_b(kt + 2, 2); }
        } else {
          if (m == 3 && ld_a1) dma_b(kt + 1, 2);
          if (m == 4 && ld_a1) dma_b(kt + 1, 3);
          if (m == 5 && ld_b) dma_b(kt + 2, 0);
          if (m == 6 && ld_b) dma_b(kt + 2, 1);
        }
        if (m < MB) {
          if (m + 1 < MB) Af[(m + 1) & 1] = frag(a_row(kt, m + 1));
          else if (XB) Af[(m + 1) & 1] = frag(a_row(kt, 8));
          mfma_block(acc[m], Af[m & 1], sa_r[m]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (XB) mfma_block(accx, Af[0], sa_x);
      __builtin_amdgcn_sched_barrier(0);
      if (next) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (vmb) wait_vmcnt<NPRE>(); else wait_vmcnt<0>();
        block_barrier();  // every wave done with A slot kt%2, B(kt) and the scales of kt
        if (ld_a2) {
          dma_a(kt + 2, 0);
          dma_a(kt + 2, 1);
          dma_scales(kt + 2);
        }
        read_stage(kt + 1);
      }
    };
    using T = std::true_type;
    using F = std::false_type;
    stage(0, nk > 2, F{}, F{}, nk > 1, nk > 2);
    for (int kt = 1; kt + 2 < nk; ++kt) stage(kt, T{}, T{}, T{}, T{}, T{});
    if (nk >= 3) stage(nk - 2, F{}, T{}, F{}, T{}, F{});
    if (nk >= 2) stage(nk - 1, F{}, F{}, F{}, F{}, F{});
  };
  if constexpr (XR > 0) {
    // rows > 256: every wave has four live row blocks
    if (!any) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 4>{});
  } else {
    if (!any) run(std::integral_constant<int, 0>{});
    else if (live_m <= 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 4>{});
  }

  // ---- epilogue: stage the tile in LDS (four consecutive columns per lane
  // and store; gate/up: H in fp32, 16 bytes; down: bf16, 8 bytes), then write
  // whole rows (gate/up: quantised to E4M3)
  constexpr int OCOLS = (MODE == kGateUp) ? BN / 2 : BN;
  constexpr int OSTRIDE = (MODE == kGateUp) ? QSTRIDE : OCOLS * 2 + 8;
  static_assert((BM + XR) * OSTRIDE <= LDS_BYTES, "staged tile exceeds the LDS");
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  auto pack2 = [](float x, float y) {
    const bf16x2_t v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  };
  auto stage_block = [&](const floatx4_t (&c)[4], int row) {
    char* lrow = lds_raw + row * OSTRIDE;
    if (MODE == kGateUp) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        float hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float g = c[f][j];
          const float u = c[f + 2][j];
          hv[j] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
        }
        *reinterpret_cast<float4*>(lrow + (b_col[f] + 4 * quad) * 4) =
            make_float4(hv[0], hv[1], hv[2], hv[3]);
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f)
        *reinterpret_cast<uint2*>(lrow + (b_col[f] + 4 * quad) * 2) =
            make_uint2(pack2(c[f][0], c[f][1]), pack2(c[f][2], c[f][3]));
    }
  };
  __syncthreads();  // all fragment reads of the last stage are done
  if (any) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m >= 2 * live_m) break;
      stage_block(acc[m], wg * 128 + m * 16 + fr);
    }
    if (XR > 0) stage_block(accx, BM + 16 * wg + fr);
  }
  __syncthreads();
  if constexpr (MODE == kGateUp) epilogue_store_q<BM + XR>(a, nt, row0, rows, tid, lds_raw);
  else epilogue_store<MODE, BM + XR>(a, nt, row0, rows, tid, lds_raw);
}

// A segment held by one m-tile (its first tile is also its last) multiplies
// each of its expert's B tiles once, so those loads are marked non-temporal
// and leave L2 to the A rows, which the segment's column tiles share.
// Segments of several m-tiles reuse their B tiles and keep the default
// policy.  Tile entries are (expert, first row, rows, row offset in the
// segment); only the last tile of a segment can differ from BM rows.
__device__ __forceinline__ bool single_tile_segment(const GemmArgs& a, int4 ent, int64_t mt,
                                                    int64_t m_tiles) {
  if (ent.w != 0) return false;
  if (ent.z != BM) return true;
  return mt + 1 == m_tiles || reinterpret_cast<const int4*>(a.tiles)[mt + 1].x != ent.x;
}

template <int MODE>
__global__ __launch_bounds__(512, 2) void gemm_fp8_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const bool grouped = a.tiles != nullptr;
  const int64_t m_tiles = grouped ? (int64_t)(*a.n_tiles) : (a.rows_dense + BM - 1) / BM;
  int64_t logical;
  if (!xcd_tile(m_tiles * a.n_tiles_n, logical)) return;
  const int64_t mt = logical / a.n_tiles_n;
  const int nt = (int)(logical % a.n_tiles_n);
  if (grouped) {
    const int4 ent = reinterpret_cast<const int4*>(a.tiles)[mt];
    const bool once = single_tile_segment(a, ent, mt, m_tiles);
    if (ent.z > BM) {
      if (once) gemm_tile_fp8<MODE, true, kXRows, true>(a, mt, nt, lds_raw);
      else gemm_tile_fp8<MODE, true, kXRows>(a, mt, nt, lds_raw);
    } else {
      if (once) gemm_tile_fp8<MODE, true, 0, true>(a, mt, nt, lds_raw);
      else gemm_tile_fp8<MODE, true>(a, mt, nt, lds_raw);
    }
  } else {
    gemm_tile_fp8<MODE, false>(a, mt, nt, lds_raw);
  }
}

template <int MODE, bool GROUPED>
__global__ __launch_bounds__(512, 2) void gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const int64_t m_tiles = GROUPED ? (int64_t)(*a.n_tiles) : (a.rows_dense + BM - 1) / BM;
  int64_t logical;
  if (!xcd_tile(m_tiles * a.n_tiles_n, logical)) return;
  const int64_t mt = logical / a.n_tiles_n;
  const int nt = (int)(logical % a.n_tiles_n);
  if constexpr (GROUPED && MODE != kRouter) {
    const int4 ent = reinterpret_cast<const int4*>(a.tiles)[mt];
    const bool once = single_tile_segment(a, ent, mt, m_tiles);
    if (ent.z > BM) {
      if (once) gemm_tile<MODE, true, kXRows, true>(a, mt, nt, lds_raw);
      else gemm_tile<MODE, true, kXRows>(a, mt, nt, lds_raw);
      return;
    }
    if (once) {
      gemm_tile<MODE, true, 0, true>(a, mt, nt, lds_raw);
      return;
    }
  }
  if constexpr (MODE == kRouterNarrow) {
    gemm_tile<kRouter, GROUPED, 0, false, true>(a, mt, nt, lds_raw);
    return;
  } else {
    gemm_tile<MODE, GROUPED>(a, mt, nt, lds_raw);
  }
}

// The two products over x before routing in one launch: the router logits
// (first r.n_tiles_n column tiles of every m-tile) and the shared expert's
// gate/up (the next g.n_tiles_n).  The column tiles of one m-tile are
// neighbours in the XCD walk, so each x row block is fetched from HBM once.
__global__ __launch_bounds__(512, 2) void gemm_x_kernel(GemmArgs r, GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const int64_t m_tiles = (r.rows_dense + BM - 1) / BM;
  const int n_all = r.n_tiles_n + g.n_tiles_n;
  int64_t logical;
  if (!xcd_tile(m_tiles * n_all, logical)) return;
  const int64_t mt = logical / n_all;
  const int nt = (int)(logical % n_all);
  if (nt < r.n_tiles_n) gemm_tile<kRouter, false>(r, mt, nt, lds_raw);
  else gemm_tile<kGateUp, false>(g, mt, nt - r.n_tiles_n, lds_raw);
}

// As gemm_x_kernel with the shared expert's gate/up on E4M3 operands (the
// router stays bf16).
__global__ __launch_bounds__(512, 2) void gemm_x_fp8_kernel(GemmArgs r, GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const int64_t m_tiles = (r.rows_dense + BM - 1) / BM;
  const int n_all = r.n_tiles_n + g.n_tiles_n;
  int64_t logical;
  if (!xcd_tile(m_tiles * n_all, logical)) return;
  const int64_t mt = logical / n_all;
  const int nt = (int)(logical % n_all);
  if (nt < r.n_tiles_n) gemm_tile<kRouter, false>(r, mt, nt, lds_raw);
  else gemm_tile_fp8<kGateUp, false>(g, mt, nt - r.n_tiles_n, lds_raw);
}

template <int MODE, bool GROUPED>
static hipError_t launch_mode(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  static std::atomic<uint32_t> configured{0};
  {
    const hipError_t e =
        set_lds_limit_once((const void*)gemm_kernel<MODE, GROUPED>, LDS_BYTES, configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gemm_kernel<MODE, GROUPED>), grid, dim3(512), LDS_BYTES, stream, a);
  return hipGetLastError();
}

static hipError_t launch_gemm(int mode, const GemmArgs& a, int64_t max_m_tiles,
                              hipStream_t stream) {
  const int64_t work = max_m_tiles * a.n_tiles_n;
  if (work <= 0) return hipSuccess;
  const int64_t share = (work + kXcd - 1) / kXcd;
  const int64_t blocks = share * kXcd;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  const bool grouped = a.tiles != nullptr;
  switch (mode) {
    case kGateUp:
      return grouped ? launch_mode<kGateUp, true>(a, grid, stream)
                     : launch_mode<kGateUp, false>(a, grid, stream);
    case kDown:
      return grouped ? launch_mode<kDown, true>(a, grid, stream)
                     : launch_mode<kDown, false>(a, grid, stream);
    case kRouterNarrow: return launch_mode<kRouterNarrow, false>(a, grid, stream);
    default: return launch_mode<kRouter, false>(a, grid, stream);
  }
}




// With E <= 128 experts the router runs in 256 x 128 tiles: a 256-wide tile
// would leave half of its columns empty, while a narrow one gives each wave
// 64 rows x 64 columns, so both waves of every SIMD multiply and the tile
// takes half the MFMA time for the same A loads (E = 128, N = 4096: layer
// 0.551 -> 0.541 ms on one box, 0.535 -> 0.532 ms on another).  Wider
// routers keep the 256-wide tiles: narrow ones re-read the A rows once more
// per 128 columns and measured no faster at E = 384.
static void apply_sel(GemmArgs& a, const RouterSel* sel) {
  if (!sel) return;
  a.sel_beta = sel->beta;
  a.cand_s = sel->cand_s;
  a.cand_e = sel->cand_e;
  a.sel_k = sel->K + 1;
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w_router,
                              const float* offset, int64_t N, int d, int E, float* Z,
                              hipStream_t stream, const RouterSel* sel) {
  GemmArgs a = router_args(x, w_router, offset, N, d, E, Z);
  apply_sel(a, sel);
  if (E <= BN / 2) {
    a.n_tiles_n = 1;
    return launch_gemm(kRouterNarrow, a, (N + BM - 1) / BM, stream);
  }
  return launch_gemm(kRouter, a, (N + BM - 1) / BM, stream);
}

hipError_t launch_gateup(const uint16_t* x, int64_t x_rows, const int32_t* sorted_src, int K,
                         const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                         int64_t rows_dense, const uint16_t* w_gate,
                         const uint16_t* w_up, int d, int h, uint16_t* H,
                         hipStream_t stream, bool kblock_major) {
  GemmArgs a = gateup_args(x, x_rows, sorted_src, K, tiles, n_tiles, rows_dense, w_gate, w_up, d,
                           h, H);
  if (kblock_major) b_kblock_major(a);
  const int64_t mt = tiles ? max_tiles : (rows_dense + BM - 1) / BM;
  return launch_gemm(kGateUp, a, mt, stream);
}

hipError_t launch_down(const uint16_t* H, int64_t h_rows, const int32_t* tiles, const int32_t* n_tiles,
                       int64_t max_tiles, int64_t rows_dense, const uint16_t* w_down,
                       int d, int h, uint16_t* Y, hipStream_t stream) {
  const GemmArgs a = down_args(H, h_rows, tiles, n_tiles, rows_dense, w_down, d, h, Y);
  const int64_t mt = tiles ? max_tiles : (rows_dense + BM - 1) / BM;
  return launch_gemm(kDown, a, mt, stream);
}

static dim3 xcd_grid(int64_t work) {
  const int64_t share = (work + kXcd - 1) / kXcd;
  return dim3((unsigned)(share * kXcd));
}

hipError_t launch_router_shared_gateup(const uint16_t* x, int64_t N, int d,
                                       const uint16_t* w_router, const float* offset, int E,
                                       float* Z, const uint16_t* ws_gate,
                                       const uint16_t* ws_up, int hs, uint16_t* Hs,
                                       hipStream_t stream, const RouterSel* sel) {
  GemmArgs r = router_args(x, w_router, offset, N, d, E, Z);
  apply_sel(r, sel);
  const GemmArgs g = gateup_args(x, N, nullptr, 1, nullptr, nullptr, N, ws_gate, ws_up, d, hs, Hs);
  const int64_t work = ((N + BM - 1) / BM) * (r.n_tiles_n + g.n_tiles_n);
  if (work <= 0) return hipSuccess;
  if (work > 0x7FFFFFF0LL) return hipErrorInvalidConfiguration;
  static std::atomic<uint32_t> configured{0};
  {
    const hipError_t e =
        set_lds_limit_once((const void*)gemm_x_kernel, LDS_BYTES, configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gemm_x_kernel, xcd_grid(work), dim3(512), LDS_BYTES, stream, r, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- FP8 launches

static hipError_t launch_fp8(int mode, const GemmArgs& a, int64_t max_m_tiles,
                             hipStream_t stream) {
  const int64_t work = max_m_tiles * a.n_tiles_n;
  if (work <= 0) return hipSuccess;
  if (work > 0x7FFFFFF0LL) return hipErrorInvalidConfiguration;
  const void* fn = mode == kGateUp ? (const void*)gemm_fp8_kernel<kGateUp>
                                   : (const void*)gemm_fp8_kernel<kDown>;
  static std::atomic<uint32_t> configured[2] = {{0}, {0}};
  {
    const hipError_t e = set_lds_limit_once(fn, LDS_BYTES, configured[mode]);
    if (e != hipSuccess) return e;
  }
  if (mode == kGateUp)
    hipLaunchKernelGGL(gemm_fp8_kernel<kGateUp>, xcd_grid(work), dim3(512), LDS_BYTES, stream, a);
  else
    hipLaunchKernelGGL(gemm_fp8_kernel<kDown>, xcd_grid(work), dim3(512), LDS_BYTES, stream, a);
  return hipGetLastError();
}

hipError_t launch_gateup_fp8(const uint8_t* xq, const float* xs, int64_t x_rows,
                             const int32_t* sorted_src, int K, const int32_t* tiles,
                             const int32_t* n_tiles, int64_t max_tiles, int64_t rows_dense,
                             const uint8_t* wg, const float* sg, const uint8_t* wu,
                             const float* su, int d, int h, uint8_t* Hq, float* Hs,
                             hipStream_t stream, bool kblock_major) {
  GemmArgs a = gateup_fp8_args(xq, xs, x_rows, sorted_src, K, tiles, n_tiles, rows_dense, wg, sg,
                               wu, su, d, h, Hq, Hs);
  if (kblock_major) b_kblock_major(a);
  return launch_fp8(kGateUp, a, tiles ? max_tiles : (rows_dense + BM - 1) / BM, stream);
}

hipError_t launch_down_fp8(const uint8_t* Hq, const float* Hs, int64_t h_rows,
                           const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                           int64_t rows_dense, const uint8_t* wd, const float* sd, int d, int h,
                           uint16_t* Y, hipStream_t stream) {
  const GemmArgs a = down_fp8_args(Hq, Hs, h_rows, tiles, n_tiles, rows_dense, wd, sd, d, h, Y);
  return launch_fp8(kDown, a, tiles ? max_tiles : (rows_dense + BM - 1) / BM, stream);
}

hipError_t launch_router_shared_gateup_fp8(const uint16_t* x, const uint8_t* xq, const float* xs,
                                           int64_t N, int d, const uint16_t* w_router,
                                           const float* offset, int E, float* Z,
                                           const uint8_t* wsg, const float* ssg,
                                           const uint8_t* wsu, const float* ssu, int hs,
                                           uint8_t* Hsq, float* Hss, hipStream_t stream,
                                           const RouterSel* sel) {
  GemmArgs r = router_args(x, w_router, offset, N, d, E, Z);
  apply_sel(r, sel);
  const GemmArgs g = gateup_fp8_args(xq, xs, N, nullptr, 1, nullptr, nullptr, N, wsg, ssg, wsu,
                                     ssu, d, hs, Hsq, Hss);
  const int64_t work = ((N + BM - 1) / BM) * (r.n_tiles_n + g.n_tiles_n);
  if (work <= 0) return hipSuccess;
  if (work > 0x7FFFFFF0LL) return hipErrorInvalidConfiguration;
  static std::atomic<uint32_t> configured{0};
  {
    const hipError_t e =
        set_lds_limit_once((const void*)gemm_x_fp8_kernel, LDS_BYTES, configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gemm_x_fp8_kernel, xcd_grid(work), dim3(512), LDS_BYTES, stream, r, g);
  return hipGetLastError();
}

}  // namespace moe
