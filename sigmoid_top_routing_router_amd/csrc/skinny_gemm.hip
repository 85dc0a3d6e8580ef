// Weight-streaming GEMMs of the MoE layer for small batches (decode).
//
// Same products as the 256 x 256 tile engine ("Kolibri 1 im Detail", routing
// section: router x W_r^T, SwiGLU gate/up and down projections; FP8 section
// for the E4M3 variant), for tiles of few rows: with N <= 64 tokens every
// expert holds at most 64 rows, and the layer is bound by reading each
// touched expert's weights once from HBM.  The tile engine's 256 x 256 tile
// keeps too few weight bytes in flight per CU for that when a tile has few
// rows; here every wave streams its own weight rows:
//  * a block of 4 waves covers 256 weight rows (gate/up: 128 gate rows and
//    the 128 up rows of the same hidden columns, one 1 x 128 group of H);
//    each wave streams 64 of them as four 16-row MFMA blocks through a ring
//    of k-sets in LDS (below), with the next k-sets loading while the
//    current one multiplies;
//  * the (few) activation rows are read from global memory (L2-resident) in
//    the MFMA layout, 16 rows per pass; a tile with more than 16 rows runs
//    one pass per 16 rows;
//  * bf16: v_mfma_f32_16x16x32_bf16, weights as the first operand, so lane l
//    ends up with activation row (l & 15) and four consecutive output columns;
//  * E4M3: v_mfma_f32_16x16x128_f8f6f4 covers one 128-k scale block; its
//    product (from zero) is added to the fp32 accumulator times
//    s_A(row, kb) * s_B(block, kb);
//  * epilogues as in the tile engine: gate/up SiLU(g) * u in bf16 or, from
//    its fp32 value, quantised to E4M3 per 1 x 128 group (amax across the
//    block's four waves through LDS), down bf16.
// Only the routed (grouped) products use it; the grid covers the m-tile
// table's capacity and surplus blocks exit.
// Each wave streams its weight rows through a ring of its own in LDS (bf16:
// 4 x 10 KB k-sets per wave, 160 KB per block; E4M3: 3 x 11 KB per wave,
// 132 KB per block), so one block occupies a CU; the bytes in flight
// come from the three (two) k-sets each wave keeps loading ahead.
#include "common.h"
#include "gemm_args.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kPassRows = 16;    // activation rows per pass (MFMA N)
constexpr int kBlockRows = 256;  // weight rows per block (4 waves x 64)
// Per wave an LDS ring of k-sets: bf16 4 slots of 10 x 1 KB pieces (160 KB
// per block: three sets in flight), E4M3 3 slots of 10 pieces plus 3 x 256 B
// of scales, and 256 B for the amax exchange of the quantising epilogue.
template <bool FP8> struct Ring {
  static constexpr int kSets = FP8 ? 3 : 4;
  static constexpr int kSlot = FP8 ? 11 * 1024 : 10 * 1024;
  static constexpr int kAmax = 4 * kSets * kSlot;  // offset of the amax exchange
  static constexpr int kLds = kAmax + (FP8 ? 256 : 0);
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
// LDS fragments are read as clang vector types: a load of HIP's uint4 struct
// carries memory-operand information that makes the compiler wait for every
// LDS-DMA load in flight before it.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <int MODE, bool FP8>
__global__ __launch_bounds__(256) void skinny_kernel(GemmArgs a, int n_chunks) {
  const int64_t mt = (int64_t)blockIdx.x / n_chunks;
  const int nc = (int)((int64_t)blockIdx.x % n_chunks);
  int expert = 0;
  int64_t row0;
  int rows;
  if (mt >= (int64_t)(*a.n_tiles)) return;  // the grid covers the table's capacity
  {
    const int4 ent = reinterpret_cast<const int4*>(a.tiles)[mt];
    expert = ent.x;
    row0 = ent.y;
    rows = ent.z;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int fr = lane & 15;
  const int q = lane >> 4;
  constexpr int EB = FP8 ? 1 : 2;  // bytes per element

  // ---- this wave's 64 weight rows as four 16-row blocks (clamped to the
  // matrix; rows past it are computed and never stored)
  const int c0 = (MODE == kGateUp) ? nc * 128 + 32 * wave : nc * kBlockRows + 64 * wave;
  int wcol[4];  // first output column of each block (gate/up: hidden column)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
    wcol[mb] = (MODE == kGateUp) ? c0 + 16 * (mb & 1) : c0 + 16 * mb;
  const int nkb = a.kdim / 128;  // E4M3 scale blocks along k

  // A k-set is 128 bytes of every row: bf16 two k-steps of 32 (64 k), E4M3
  // one k-step of 128.  Each LDS-DMA load moves 8 whole rows of a set (lane i:
  // row i >> 3, 16-byte chunk i & 7 of the LDS row), so every access is one
  // whole 128-byte line; a 16-row block takes two loads.  The eight chunks of
  // row r sit at LDS slot g(c) ^ ((r >> 1) & 7) (the loads pick their global
  // chunk accordingly), so the fragment reads of 16 rows with one chunk hit
  // 16 different bank groups; g(c) = c for bf16, and for E4M3, whose lanes of
  // quads 0 and 1 (2 and 3) read chunks 2q and 2q + 1 of the same rows,
  // g(c) = c ^ 4 ((c >> 1) & 1) keeps those quads on different banks too.  A set: 4 weight blocks, the block of 16
  // activation rows, and for E4M3 the activation scale of each lane's row
  // and the two weight-block scales (4-byte loads).  The loads do not go
  // through registers, so the compiler inserts no waits for them; the
  // explicit vmcnt waits below keep kRing - 1 sets in flight.
  constexpr int SET_K = FP8 ? 128 : 64;   // k per set
  constexpr int OPS = FP8 ? 13 : 10;      // loads per set and wave
  const int nsets = (a.kdim + SET_K - 1) / SET_K;
  const bool half_last = !FP8 && (a.kdim % 64) != 0;  // last bf16 set holds one k-step
  // DMA lane roles: row 8*h + (lane >> 3) of a 16-row block (h = 0, 1), LDS
  // chunk lane & 7, global chunk g((lane & 7) ^ ((4*h + (lane >> 4)) & 7))
  // (g is its own inverse)
  auto g_chunk = [](int c) { return FP8 ? (c ^ (4 * ((c >> 1) & 1))) : c; };
  const uint32_t gchunk0 = (uint32_t)g_chunk((lane & 7) ^ ((lane >> 4) & 7)) * 16u;
  const uint32_t gchunk1 = (uint32_t)g_chunk((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 16u;
  const uint32_t set_bytes = SET_K * EB;
  const uint32_t b_bytes = (uint32_t)a.b_rows * (uint32_t)a.kdim * EB;
  // the shared expert's tile (expert -1): its own row-major weights
  const bool shared = expert < 0;
  const uint32_t row_pitch = shared ? (uint32_t)a.kdim * EB : a.b_row_pitch;
  const uint32_t kblk_pitch = shared ? 128u : a.b_kblk_pitch;
  const char* bexp0 =
      shared ? reinterpret_cast<const char*>(a.Bs0)
             : reinterpret_cast<const char*>(a.B0) + (int64_t)expert * a.b_expert_stride * EB;
  const char* bexp1 =
      shared ? reinterpret_cast<const char*>(MODE == kGateUp ? a.Bs1 : a.Bs0)
             : reinterpret_cast<const char*>(MODE == kGateUp ? a.B1 : a.B0) +
                   (int64_t)expert * a.b_expert_stride * EB;
  const __amdgpu_buffer_rsrc_t rw0 = make_rsrc(bexp0, b_bytes);
  const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(bexp1, b_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.a_bytes);
  uint32_t w_voff[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = min(wcol[mb] + 8 * h + (lane >> 3), a.b_rows - 1);
      w_voff[mb][h] = (uint32_t)r * row_pitch + (h ? gchunk1 : gchunk0);
    }
  // E4M3 scales: [A rows][kdim / 128] for the activations, the expert's
  // [b_rows / 128][kdim / 128] for the weights (unused resources cover 0 bytes)
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(FP8 ? (const void*)a.sa : a.A, FP8 ? a.a_bytes / 32 : 0u);
  const float* sbase0 = shared ? a.sbs0 : a.sb0 + (int64_t)expert * a.sb_es;
  const float* sbase1 = shared ? (MODE == kGateUp ? a.sbs1 : a.sbs0)
                               : (MODE == kGateUp ? a.sb1 : a.sb0) + (int64_t)expert * a.sb_es;
  const __amdgpu_buffer_rsrc_t rsb0 = make_rsrc(FP8 ? (const void*)sbase0 : a.A,
                                                FP8 ? (uint32_t)a.sb_es * 4u : 0u);
  const __amdgpu_buffer_rsrc_t rsb1 = make_rsrc(FP8 ? (const void*)sbase1 : a.A,
                                                FP8 ? (uint32_t)a.sb_es * 4u : 0u);
  const int nblk = (a.b_rows + 127) / 128;
  const int sblk = (MODE == kGateUp) ? nc : min(c0 / 128, nblk - 1);
  const uint32_t sb_voff0 = (uint32_t)(sblk * nkb) * 4u, sb_voff1 = sb_voff0;
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  constexpr int kRing = Ring<FP8>::kSets, kSlot = Ring<FP8>::kSlot;
  char* ring = lds_raw + wave * (kRing * kSlot);
  float (*s_amax)[kPassRows] = reinterpret_cast<float (*)[kPassRows]>(lds_raw + Ring<FP8>::kAmax);

  const int passes = (rows + kPassRows - 1) / kPassRows;
  for (int pass = 0; pass < passes; ++pass) {
    const int t = pass * kPassRows + fr;  // this lane's activation row in the tile
    const bool t_ok = t < rows;
    // A row of tile row tt (rows past the tile read the first row)
    auto a_row = [&](int tt) -> int64_t {
      const int64_t r = row0 + (tt < rows ? tt : 0);
      if (!a.gather) return r;
      return shared ? r - a.shared_row0 : (int64_t)(a.gather[r] / a.gather_div);
    };
    uint32_t t_voff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      t_voff[h] = (uint32_t)(a_row(pass * kPassRows + 8 * h + (lane >> 3)) * a.lda * EB) +
                  (h ? gchunk1 : gchunk0);
    const uint32_t ts_voff = FP8 ? (uint32_t)(a_row(t) * nkb) * 4u : 0u;

    auto issue = [&](int s) {
      char* slot = ring + (s % kRing) * kSlot;
      const uint32_t soff = (uint32_t)s * set_bytes;
      const uint32_t soff_w = (uint32_t)s * kblk_pitch;  // a set is one 128-byte k-block
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const __amdgpu_buffer_rsrc_t rw = (MODE == kGateUp && mb >= 2) ? rw1 : rw0;
        dma16(rw, w_voff[mb][0], soff_w, (lds_void_t*)(slot + (2 * mb) * 1024));
        dma16(rw, w_voff[mb][1], soff_w, (lds_void_t*)(slot + (2 * mb + 1) * 1024));
      }
      dma16(ra, t_voff[0], soff, (lds_void_t*)(slot + 8 * 1024));
      dma16(ra, t_voff[1], soff, (lds_void_t*)(slot + 9 * 1024));
      if (FP8) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void_t*)(slot + 10 * 1024), 4,
                                                 ts_voff, (uint32_t)s * 4u, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb0, (lds_void_t*)(slot + 10 * 1024 + 256), 4,
                                                 sb_voff0, (uint32_t)s * 4u, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb1, (lds_void_t*)(slot + 10 * 1024 + 512), 4,
                                                 sb_voff1, (uint32_t)s * 4u, 0, 0);
      }
    };

    floatx4_t acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < kRing - 1; ++s)
      if (s < nsets) issue(s);
    for (int s = 0; s < nsets; ++s) {
      // set s has landed once only the loads of the sets issued after it
      // (at most kRing - 2 of them) are pending
      if (kRing > 3 && s + 2 < nsets) wait_vmcnt<(kRing > 3 ? 2 : 1) * OPS>();
      else if (s + 1 < nsets) wait_vmcnt<OPS>();
      else wait_vmcnt<0>();
      const char* slot = ring + (s % kRing) * kSlot;
      // fragment piece j of lane l: row l & 15, chunk 4j + (l >> 4) (bf16)
      // or 2(l >> 4) + j (E4M3), at its swizzled slot
      u32x4_t W[4][2], T[2];
      int foff[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = FP8 ? 2 * q + j : 4 * j + q;
        foff[j] = fr * 128 + ((g_chunk(c) ^ ((fr >> 1) & 7)) * 16);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          W[mb][j] = *reinterpret_cast<const u32x4_t*>(slot + mb * 2048 + foff[j]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        T[j] = *reinterpret_cast<const u32x4_t*>(slot + 8 * 1024 + foff[j]);
      float sc[3] = {0.f, 0.f, 0.f};
      if (FP8) {
        sc[0] = *reinterpret_cast<const float*>(slot + 10 * 1024 + lane * 4);
        sc[1] = *reinterpret_cast<const float*>(slot + 10 * 1024 + 256 + lane * 4);
        sc[2] = *reinterpret_cast<const float*>(slot + 10 * 1024 + 512 + lane * 4);
      }
      if (s + kRing - 1 < nsets) issue(s + kRing - 1);  // into the slot freed by set s-1
      if (FP8) {
        const i32x8_t tf = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(T[0], T[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const i32x8_t wf = __builtin_bit_cast(
              i32x8_t, __builtin_shufflevector(W[mb][0], W[mb][1], 0, 1, 2, 3, 4, 5, 6, 7));
          const floatx4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf, tf, floatx4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          const float fac = sc[0] * sc[(MODE == kGateUp && mb >= 2) ? 2 : 1];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][r] = fmaf(p[r], fac, acc[mb][r]);
        }
      } else {
        const bool two = !(half_last && s == nsets - 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // the second piece of a half set lies past the row: multiply it by zero
          const u32x4_t tj = (j == 1 && !two) ? u32x4_t{0u, 0u, 0u, 0u} : T[j];
          const bf16x8_t tf = __builtin_bit_cast(bf16x8_t, tj);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, W[mb][j]), tf, acc[mb], 0, 0, 0);
        }
      }
    }

    // ---- epilogue.  Lane l: activation row t, and for block mb the output
    // columns wcol[mb] + 4*(l >> 4) + r, r = 0..3.
    const int64_t orow = row0 + t;
    static_assert(MODE != kRouter, "the router product uses the tile engine");
    if (MODE == kGateUp) {
      // H in bf16 (hardware round-to-nearest-even)
      uint32_t hb[2][2];
      float hv[2][4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[mb][r] = silu_mul(acc[mb][r], acc[mb + 2][r]);
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        hb[mb][0] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)hv[mb][0], (__bf16)hv[mb][1]});
        hb[mb][1] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)hv[mb][2], (__bf16)hv[mb][3]});
      }
      if (FP8 && a.out_scale) {
        // the block's 128 hidden columns of row t are one 1 x 128 group: amax
        // of the fp32 values over the 4 lanes of the row in each wave, then
        // over the waves through LDS
        float v[8];
        uint32_t m = 0;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[4 * mb + r] = hv[mb][r];
            m = max(m, __float_as_uint(fabsf(hv[mb][r])));
          }
        m = max(m, (uint32_t)__shfl_xor((int)m, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 32));
        if (q == 0) s_amax[wave][fr] = __uint_as_float(m);
        __syncthreads();
        const float amax = fmaxf(fmaxf(s_amax[0][fr], s_amax[1][fr]),
                                 fmaxf(s_amax[2][fr], s_amax[3][fr]));
        __syncthreads();  // s_amax is rewritten by the next pass
        const float sc = amax / 448.0f;
        if (t_ok) {
          uint8_t* Q = reinterpret_cast<uint8_t*>(a.out);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            int pk = 0;
            if (amax != 0.0f) {
              float u[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) u[r] = fminf(fmaxf(v[4 * mb + r] / sc, -448.0f), 448.0f);
              pk = __builtin_amdgcn_cvt_pk_fp8_f32(u[0], u[1], 0, false);
              pk = __builtin_amdgcn_cvt_pk_fp8_f32(u[2], u[3], pk, true);
            }
            *reinterpret_cast<uint32_t*>(Q + orow * a.ldo + wcol[mb] + 4 * q) = (uint32_t)pk;
          }
          if (wave == 0 && q == 0)
            a.out_scale[orow * (a.ldo / 128) + nc] = (amax != 0.0f) ? sc : 0.0f;
        }
      } else if (t_ok) {
        uint16_t* H = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int col = wcol[mb] + 4 * q;
          if (col < a.b_rows)
            *reinterpret_cast<uint2*>(H + orow * a.ldo + col) = make_uint2(hb[mb][0], hb[mb][1]);
        }
      }
    } else {  // down: Y in bf16
      if (t_ok) {
        uint16_t* Y = reinterpret_cast<uint16_t*>(a.out);
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int col = wcol[mb] + 4 * q;
          if (col < a.b_rows)
            *reinterpret_cast<uint2*>(Y + orow * a.ldo + col) = make_uint2(
                __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)acc[mb][0], (__bf16)acc[mb][1]}),
                __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)acc[mb][2], (__bf16)acc[mb][3]}));
        }
      }
    }
  }
}

template <int MODE, bool FP8>
hipError_t launch_skinny_mode(const GemmArgs& a, int64_t m_tiles, hipStream_t stream) {
  const int n_chunks = (MODE == kGateUp) ? (a.b_rows + 127) / 128
                                         : (a.b_rows + kBlockRows - 1) / kBlockRows;
  const int64_t blocks = m_tiles * n_chunks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  constexpr int lds = Ring<FP8>::kLds;
  static std::atomic<uint32_t> configured{0};
  {
    const hipError_t e =
        set_lds_limit_once((const void*)skinny_kernel<MODE, FP8>, lds, configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((skinny_kernel<MODE, FP8>), dim3((unsigned)blocks), dim3(256), lds, stream,
                     a, n_chunks);
  return hipGetLastError();
}


}  // namespace

static void apply_fold(GemmArgs& a, const SharedFold* sf, int mode) {
  if (!sf) return;
  a.Bs0 = static_cast<const uint16_t*>(mode == kGateUp ? sf->gate : sf->down);
  a.Bs1 = static_cast<const uint16_t*>(sf->up);
  a.sbs0 = mode == kGateUp ? sf->s_gate : sf->s_down;
  a.sbs1 = sf->s_up;
  a.shared_row0 = sf->row0;
}

hipError_t launch_gateup_small(const uint16_t* x, int64_t x_rows, const int32_t* sorted_src,
                               int K, const int32_t* tiles, const int32_t* n_tiles,
                               int64_t max_tiles, int64_t rows_dense, const uint16_t* w_gate,
                               const uint16_t* w_up, int d, int h, uint16_t* H,
                               hipStream_t stream, bool kblock_major, const SharedFold* sf) {
  GemmArgs a = gateup_args(x, x_rows, sorted_src, K, tiles, n_tiles, rows_dense, w_gate, w_up, d,
                           h, H);
  if (kblock_major) b_kblock_major(a);
  apply_fold(a, sf, kGateUp);
  if (!tiles) return hipErrorInvalidValue;
  return launch_skinny_mode<kGateUp, false>(a, max_tiles, stream);
}

hipError_t launch_down_small(const uint16_t* H, int64_t h_rows, const int32_t* tiles,
                             const int32_t* n_tiles, int64_t max_tiles, int64_t rows_dense,
                             const uint16_t* w_down, int d, int h, uint16_t* Y,
                             hipStream_t stream, const SharedFold* sf) {
  GemmArgs a = down_args(H, h_rows, tiles, n_tiles, rows_dense, w_down, d, h, Y);
  apply_fold(a, sf, kDown);
  if (!tiles) return hipErrorInvalidValue;
  return launch_skinny_mode<kDown, false>(a, max_tiles, stream);
}

hipError_t launch_gateup_fp8_small(const uint8_t* xq, const float* xs, int64_t x_rows,
                                   const int32_t* sorted_src, int K, const int32_t* tiles,
                                   const int32_t* n_tiles, int64_t max_tiles, int64_t rows_dense,
                                   const uint8_t* wg, const float* sg, const uint8_t* wu,
                                   const float* su, int d, int h, uint8_t* Hq, float* Hs,
                                   hipStream_t stream, bool kblock_major, const SharedFold* sf) {
  GemmArgs a = gateup_fp8_args(xq, xs, x_rows, sorted_src, K, tiles, n_tiles, rows_dense, wg, sg,
                               wu, su, d, h, Hq, Hs);
  if (kblock_major) b_kblock_major(a);
  apply_fold(a, sf, kGateUp);
  if (!tiles) return hipErrorInvalidValue;
  return launch_skinny_mode<kGateUp, true>(a, max_tiles, stream);
}

hipError_t launch_down_fp8_small(const uint8_t* Hq, const float* Hs, int64_t h_rows,
                                 const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                                 int64_t rows_dense, const uint8_t* wd, const float* sd, int d,
                                 int h, uint16_t* Y, hipStream_t stream, const SharedFold* sf) {
  GemmArgs a = down_fp8_args(Hq, Hs, h_rows, tiles, n_tiles, rows_dense, wd, sd, d, h, Y);
  apply_fold(a, sf, kDown);
  if (!tiles) return hipErrorInvalidValue;
  return launch_skinny_mode<kDown, true>(a, max_tiles, stream);
}

}  // namespace moe
