// Arguments of the MoE layer's GEMM kernels (the 256 x 256 tile engine in
// grouped_gemm.hip and the weight-streaming kernel for small row counts in
// skinny_gemm.hip), their builders for the layer's products, and the
// global -> LDS load helpers both kernels use.  Included by HIP sources only.
#pragma once
#include <cstdint>

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kTileN = 256;  // output columns (B rows) of one n-tile of the tile engine

// kRouterNarrow: the router product in 256 x 128 tiles (a launch mode of
// gemm_kernel; the tile itself is gemm_tile<kRouter, ..., NARROW = true>)
enum Mode { kGateUp = 0, kDown = 1, kRouter = 2, kRouterNarrow = 3 };

struct GemmArgs {
  const uint16_t* A;       // x (gate/up, router) or H (down)
  int64_t lda;             // elements per A row
  const int32_t* gather;   // sorted_src (routed gate/up) or NULL
  int gather_div;          // K (pair index -> token)
  const int32_t* tiles;    // m-tile table or NULL (dense rows)
  const int32_t* n_tiles;  // device count of table entries
  int64_t rows_dense;      // rows when tiles == NULL
  const uint16_t* B0;      // gate / down / router weights
  const uint16_t* B1;      // up weights (gate/up only)
  int64_t b_expert_stride; // elements between experts' matrices
  int b_rows;              // valid rows of one expert's B (h, d or E)
  int kdim;                // reduction length (multiple of 32)
  int n_tiles_n;           // tiles along the output columns
  void* out;               // H / Y (bf16) or Z (fp32)
  int64_t ldo;             // elements per output row
  const float* offset;     // router: per-column fp32 offset or NULL
  uint32_t a_bytes;        // size of the whole A buffer (< 4 GiB)
  // FP8 operands only (A and B are E4M3 codes; lda and kdim count bytes):
  const float* sa;         // A scales [A rows][kdim/128] (1 x 128 groups)
  const float* sb0;        // B scales [E][ceil(b_rows/128)][kdim/128] (128 x 128 blocks)
  const float* sb1;        // up-projection scales (gate/up only)
  int64_t sb_es;           // floats between experts' scale matrices
  // gate/up only: when set, H leaves as E4M3 codes (out, ldo bytes per row)
  // with one fp32 scale per 1 x 128 group of a row (out_scale [rows][ldo/128])
  float* out_scale;
  // Layout of an expert's B matrix, in bytes: from one row to the next, and
  // from one 128-byte k-block of a row to the next.  Row-major: (kdim times
  // the element size, 128); k-block-major (bf16 gate/up weights packed by
  // moe_pack_gateup_weights): (128, b_rows * 128), so that the 128-byte
  // pieces one stage of the tile reads are one contiguous run.
  uint32_t b_row_pitch;
  uint32_t b_kblk_pitch;
  // Router only, the selection fused into the epilogue (off while cand_s is
  // NULL): every tile also writes, for each of its rows, the sel_k entries
  // of its columns that come first in the selection order (biased score
  // logit + sel_beta descending, then expert ascending) to
  // cand_s / cand_e [row][n_tiles_n][sel_k]; sel_beta NULL is a zero bias.
  const float* sel_beta;
  float* cand_s;
  uint32_t* cand_e;
  int sel_k;
  // Weight-streaming kernel only: an m-tile whose expert is -1 is the shared
  // expert's (rows shared_row0 .. of H and Y; for gate/up its A rows are the
  // tokens row - shared_row0, not gathered), with row-major weights Bs0 /
  // Bs1 (E4M3: block scales sbs0 / sbs1).
  const uint16_t* Bs0;
  const uint16_t* Bs1;
  const float* sbs0;
  const float* sbs1;
  int64_t shared_row0;
};

// Row-major B (every builder's default).
inline void b_row_major(GemmArgs& a, int elem_bytes) {
  a.b_row_pitch = (uint32_t)a.kdim * (uint32_t)elem_bytes;
  a.b_kblk_pitch = 128u;
}
// k-block-major B: [expert][kdim / 64][b_rows][64] bf16.
inline void b_kblock_major(GemmArgs& a) {
  a.b_row_pitch = 128u;
  a.b_kblk_pitch = (uint32_t)a.b_rows * 128u;
}

// ---- builders (bf16 operands unless named fp8)
inline GemmArgs router_args(const uint16_t* x, const uint16_t* w_router, const float* offset,
                            int64_t N, int d, int E, float* Z) {
  GemmArgs a{};
  a.A = x; a.lda = d; a.gather = nullptr; a.gather_div = 1;
  a.tiles = nullptr; a.n_tiles = nullptr; a.rows_dense = N;
  a.B0 = w_router; a.B1 = nullptr; a.b_expert_stride = 0; a.b_rows = E; a.kdim = d;
  a.n_tiles_n = (E + kTileN - 1) / kTileN; a.out = Z; a.ldo = E; a.offset = offset;
  a.a_bytes = (uint32_t)(N * d * 2);
  b_row_major(a, 2);
  return a;
}

inline GemmArgs gateup_args(const uint16_t* x, int64_t x_rows, const int32_t* sorted_src, int K,
                            const int32_t* tiles, const int32_t* n_tiles, int64_t rows_dense,
                            const uint16_t* w_gate, const uint16_t* w_up, int d, int h,
                            uint16_t* H) {
  GemmArgs a{};
  a.A = x; a.lda = d; a.gather = tiles ? sorted_src : nullptr; a.gather_div = K;
  a.tiles = tiles; a.n_tiles = n_tiles; a.rows_dense = rows_dense;
  a.B0 = w_gate; a.B1 = w_up; a.b_expert_stride = (int64_t)h * d; a.b_rows = h; a.kdim = d;
  a.n_tiles_n = (h + kTileN / 2 - 1) / (kTileN / 2); a.out = H; a.ldo = h; a.offset = nullptr;
  a.a_bytes = (uint32_t)(x_rows * d * 2);
  b_row_major(a, 2);
  return a;
}

inline GemmArgs down_args(const uint16_t* H, int64_t h_rows, const int32_t* tiles,
                          const int32_t* n_tiles, int64_t rows_dense, const uint16_t* w_down,
                          int d, int h, uint16_t* Y) {
  GemmArgs a{};
  a.A = H; a.lda = h; a.gather = nullptr; a.gather_div = 1;
  a.tiles = tiles; a.n_tiles = n_tiles; a.rows_dense = rows_dense;
  a.B0 = w_down; a.B1 = nullptr; a.b_expert_stride = (int64_t)d * h; a.b_rows = d; a.kdim = h;
  a.n_tiles_n = (d + kTileN - 1) / kTileN; a.out = Y; a.ldo = d; a.offset = nullptr;
  a.a_bytes = (uint32_t)(h_rows * h * 2);
  b_row_major(a, 2);
  return a;
}

inline GemmArgs gateup_fp8_args(const uint8_t* xq, const float* xs, int64_t x_rows,
                                const int32_t* sorted_src, int K, const int32_t* tiles,
                                const int32_t* n_tiles, int64_t rows_dense, const uint8_t* wg,
                                const float* sg, const uint8_t* wu, const float* su, int d, int h,
                                uint8_t* Hq, float* Hs) {
  GemmArgs a{};
  a.A = reinterpret_cast<const uint16_t*>(xq); a.lda = d;
  a.gather = tiles ? sorted_src : nullptr; a.gather_div = K;
  a.tiles = tiles; a.n_tiles = n_tiles; a.rows_dense = rows_dense;
  a.B0 = reinterpret_cast<const uint16_t*>(wg); a.B1 = reinterpret_cast<const uint16_t*>(wu);
  a.b_expert_stride = (int64_t)h * d; a.b_rows = h; a.kdim = d;
  a.n_tiles_n = h / (kTileN / 2); a.out = Hq; a.ldo = h; a.offset = nullptr;
  a.a_bytes = (uint32_t)(x_rows * d);
  a.sa = xs; a.sb0 = sg; a.sb1 = su; a.sb_es = (int64_t)(h / 128) * (d / 128);
  a.out_scale = Hs;
  b_row_major(a, 1);
  return a;
}

inline GemmArgs down_fp8_args(const uint8_t* Hq, const float* Hs, int64_t h_rows,
                              const int32_t* tiles, const int32_t* n_tiles, int64_t rows_dense,
                              const uint8_t* wd, const float* sd, int d, int h, uint16_t* Y) {
  GemmArgs a{};
  a.A = reinterpret_cast<const uint16_t*>(Hq); a.lda = h; a.gather = nullptr; a.gather_div = 1;
  a.tiles = tiles; a.n_tiles = n_tiles; a.rows_dense = rows_dense;
  a.B0 = reinterpret_cast<const uint16_t*>(wd); a.B1 = nullptr;
  a.b_expert_stride = (int64_t)d * h; a.b_rows = d; a.kdim = h;
  a.n_tiles_n = (d + kTileN - 1) / kTileN; a.out = Y; a.ldo = d; a.offset = nullptr;
  a.a_bytes = (uint32_t)(h_rows * h);
  a.sa = Hs; a.sb0 = sd; a.sb1 = sd; a.sb_es = (int64_t)(d / 128) * (h / 128);
  a.out_scale = nullptr;
  b_row_major(a, 1);
  return a;
}

// ---- global -> LDS loads
typedef __attribute__((address_space(3))) void lds_void_t;

// Raw buffer resource over `bytes` bytes at `base` (stride 0; reads past the
// end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// LDS-DMA: 16 bytes per lane from (resource, per-lane voff + uniform soff) to
// LDS at l + 16 * lane.  The buffer form (buffer_load_dwordx4 ... lds) is
// counted on vmcnt only, so the compiler keeps exact lgkmcnt waits for the
// LDS fragment reads around it.
// Cache-policy operand of a buffer load: the non-temporal bit marks the lines
// as streaming, so the caches give them up first.
constexpr int kCpolNT = 2;

template <int CPOL = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      lds_void_t* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, soff, 0, CPOL);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
}  // namespace moe
