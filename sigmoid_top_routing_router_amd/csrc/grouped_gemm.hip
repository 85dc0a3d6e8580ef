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
//  * 256 threads = 4 waves as 2 (M) x 2 (N); block tile 128 x 128 (rows of
//    the B operand) x 64 (k); each wave owns 64 x 64 outputs as 2 x 2
//    v_mfma_f32_32x32x16_bf16 accumulators (fp32).
//  * A and B tiles are staged through LDS with one 16-byte global load per
//    thread and chunk, double buffered so the loads of step k+1 are in flight
//    while the MFMAs of step k run; LDS rows are padded to 144 bytes so the
//    16-byte fragment reads of 8 consecutive rows cover all banks.
//  * Gate/up: the B tile holds 64 gate rows followed by the 64 up rows of the
//    same hidden columns, and each wave takes 32 of each, so SiLU(g) * u is
//    formed in registers (lane layouts of the two accumulators coincide) and
//    H is written once in bf16.  The gathered token rows of x are read
//    directly into the A tile (the permuted copy of x is never built).
//  * Ragged segments: an m-tile table (expert, first row, rows) produced on
//    the device by the grouping kernels drives the grid; the grid is sized
//    for the worst case and surplus blocks exit after reading the tile count.
//    Waves whose 32-row MFMA blocks hold no valid rows skip their MFMAs.
//  * XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
//    block b works on the logical tile (b % 8) * share + b / 8; each XCD then
//    walks a contiguous run of (m-tile, n-tile) pairs, n fastest, and the
//    blocks that share an A tile or an expert's weights meet in that XCD's
//    L2.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;                 // bf16 per LDS row (144 bytes)
constexpr int TILE_ELEMS = BM * LDS_LD;        // one operand tile
constexpr int kXcd = 8;

int gemm_bm() { return BM; }

enum Mode { kGateUp = 0, kDown = 1, kRouter = 2 };

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
  int kdim;                // reduction length
  int n_tiles_n;           // tiles along the output columns
  void* out;               // H / Y (bf16) or Z (fp32)
  int64_t ldo;             // elements per output row
  const float* offset;     // router: per-column fp32 offset or NULL
};

__device__ __forceinline__ uint16_t f32_to_bf16_u16(float v) {
  return (uint16_t)f32_to_bf16_rne_bits(v);
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * TILE_ELEMS];

  // ---- which tile -------------------------------------------------------
  const int64_t m_tiles = a.tiles ? (int64_t)(*a.n_tiles) : (a.rows_dense + BM - 1) / BM;
  const int64_t work = m_tiles * a.n_tiles_n;
  const int64_t share = (work + kXcd - 1) / kXcd;
  const int64_t local = blockIdx.x / kXcd;
  if (local >= share) return;
  const int64_t logical = (int64_t)(blockIdx.x % kXcd) * share + local;
  if (logical >= work) return;
  const int64_t mt = logical / a.n_tiles_n;
  const int nt = (int)(logical % a.n_tiles_n);

  int expert = 0;
  int64_t row0;
  int rows;
  if (a.tiles) {
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
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global load assignment: 4 chunks of 16 bytes per operand per thread
  const int kc = (tid & 7) * 8;          // k offset of this thread's chunk
  const int r_base = tid >> 3;           // rows r_base + 32*i
  const uint16_t* a_ptr[4];
  const uint16_t* b_ptr[4];
  bool a_ok[4], b_ok[4];
  const uint16_t* Bexp0 = a.B0 + (int64_t)expert * a.b_expert_stride;
  const uint16_t* Bexp1 = (MODE == kGateUp) ? a.B1 + (int64_t)expert * a.b_expert_stride : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r_base + 32 * i;
    a_ok[i] = r < rows;
    int64_t arow = 0;
    if (a_ok[i]) {
      if (a.gather) arow = a.gather[row0 + r] / a.gather_div;
      else arow = row0 + r;
    }
    a_ptr[i] = a.A + arow * a.lda + kc;
    int brow;
    const uint16_t* bbase;
    if (MODE == kGateUp) {
      // tile rows 0..63: gate rows nt*64 + r; 64..127: up rows nt*64 + r - 64
      const int hc = nt * 64 + (r & 63);
      brow = hc;
      bbase = (r < 64) ? Bexp0 : Bexp1;
    } else {
      brow = nt * BN + r;
      bbase = Bexp0;
    }
    b_ok[i] = brow < a.b_rows;
    b_ptr[i] = bbase + (int64_t)(b_ok[i] ? brow : 0) * a.kdim + kc;
  }

  uint4 ra[4], rb[4];
  auto load_global = [&](int k0) {
    const bool kin = (k0 + kc) < a.kdim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = (a_ok[i] && kin) ? *reinterpret_cast<const uint4*>(a_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = (b_ok[i] && kin) ? *reinterpret_cast<const uint4*>(b_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int buf) {
    uint16_t* As = lds + buf * 2 * TILE_ELEMS;
    uint16_t* Bs = As + TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r_base + 32 * i;
      *reinterpret_cast<uint4*>(As + r * LDS_LD + kc) = ra[i];
      *reinterpret_cast<uint4*>(Bs + r * LDS_LD + kc) = rb[i];
    }
  };

  floatx16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Row offsets of this wave's MFMA operands inside the LDS tiles.
  const int a_row0 = wm * 64;
  int b_row[2];
  if (MODE == kGateUp) { b_row[0] = 32 * wn; b_row[1] = 64 + 32 * wn; }
  else { b_row[0] = 64 * wn; b_row[1] = 64 * wn + 32; }
  const bool mf_live0 = (a_row0) < rows;
  const bool mf_live1 = (a_row0 + 32) < rows;
  const int frag_k = (lane >> 5) * 8;
  const int frag_r = lane & 31;

  const int nk = (a.kdim + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const uint16_t* As = lds + cur * 2 * TILE_ELEMS;
    const uint16_t* Bs = As + TILE_ELEMS;
    if (mf_live0) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ko = ks * 16 + frag_k;
        const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(Bs + (b_row[0] + frag_r) * LDS_LD + ko);
        const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(Bs + (b_row[1] + frag_r) * LDS_LD + ko);
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(As + (a_row0 + frag_r) * LDS_LD + ko);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
        if (mf_live1) {
          const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(As + (a_row0 + 32 + frag_r) * LDS_LD + ko);
          acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds column (lane & 31) and, for register r, row
  // 8*(r/4) + 4*(lane/32) + r%4 of each 32 x 32 accumulator.
  const int ccol = lane & 31;
  const int rsub = 4 * (lane >> 5);
#pragma unroll
  for (int mf = 0; mf < 2; ++mf) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = a_row0 + mf * 32 + 8 * (r >> 2) + rsub + (r & 3);
      if (rr >= rows) continue;
      const int64_t orow = row0 + rr;
      if (MODE == kGateUp) {
        const int hc = nt * 64 + 32 * wn + ccol;
        if (hc < a.b_rows) {
          const float g = acc[mf][0][r];
          const float u = acc[mf][1][r];
          const float hval = g / (1.0f + __expf(-g)) * u;
          reinterpret_cast<uint16_t*>(a.out)[orow * a.ldo + hc] = f32_to_bf16_u16(hval);
        }
      } else {
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const int col = nt * BN + b_row[nf] + ccol;
          if (col < a.b_rows) {
            if (MODE == kDown) {
              reinterpret_cast<uint16_t*>(a.out)[orow * a.ldo + col] = f32_to_bf16_u16(acc[mf][nf][r]);
            } else {
              float z = acc[mf][nf][r];
              if (a.offset) z += a.offset[col];
              reinterpret_cast<float*>(a.out)[orow * a.ldo + col] = z;
            }
          }
        }
      }
    }
  }
}

static hipError_t launch_gemm(int mode, const GemmArgs& a, int64_t max_m_tiles,
                              hipStream_t stream) {
  const int64_t work = max_m_tiles * a.n_tiles_n;
  if (work <= 0) return hipSuccess;
  const int64_t share = (work + kXcd - 1) / kXcd;
  const int64_t blocks = share * kXcd;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(256);
  switch (mode) {
    case kGateUp: hipLaunchKernelGGL(gemm_kernel<kGateUp>, grid, block, 0, stream, a); break;
    case kDown: hipLaunchKernelGGL(gemm_kernel<kDown>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(gemm_kernel<kRouter>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w_router,
                              const float* offset, int64_t N, int d, int E, float* Z,
                              hipStream_t stream) {
  GemmArgs a{};
  a.A = x; a.lda = d; a.gather = nullptr; a.gather_div = 1;
  a.tiles = nullptr; a.n_tiles = nullptr; a.rows_dense = N;
  a.B0 = w_router; a.B1 = nullptr; a.b_expert_stride = 0; a.b_rows = E; a.kdim = d;
  a.n_tiles_n = (E + BN - 1) / BN; a.out = Z; a.ldo = E; a.offset = offset;
  return launch_gemm(kRouter, a, (N + BM - 1) / BM, stream);
}

hipError_t launch_gateup(const uint16_t* x, const int32_t* sorted_src, int K,
                         const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                         int64_t rows_dense, const uint16_t* w_gate,
                         const uint16_t* w_up, int d, int h, uint16_t* H,
                         hipStream_t stream) {
  GemmArgs a{};
  a.A = x; a.lda = d; a.gather = tiles ? sorted_src : nullptr; a.gather_div = K;
  a.tiles = tiles; a.n_tiles = n_tiles; a.rows_dense = rows_dense;
  a.B0 = w_gate; a.B1 = w_up; a.b_expert_stride = (int64_t)h * d; a.b_rows = h; a.kdim = d;
  a.n_tiles_n = (h + 63) / 64; a.out = H; a.ldo = h; a.offset = nullptr;
  const int64_t mt = tiles ? max_tiles : (rows_dense + BM - 1) / BM;
  return launch_gemm(kGateUp, a, mt, stream);
}

hipError_t launch_down(const uint16_t* H, const int32_t* tiles, const int32_t* n_tiles,
                       int64_t max_tiles, int64_t rows_dense, const uint16_t* w_down,
                       int d, int h, uint16_t* Y, hipStream_t stream) {
  GemmArgs a{};
  a.A = H; a.lda = h; a.gather = nullptr; a.gather_div = 1;
  a.tiles = tiles; a.n_tiles = n_tiles; a.rows_dense = rows_dense;
  a.B0 = w_down; a.B1 = nullptr; a.b_expert_stride = (int64_t)d * h; a.b_rows = d; a.kdim = h;
  a.n_tiles_n = (d + BN - 1) / BN; a.out = Y; a.ldo = d; a.offset = nullptr;
  const int64_t mt = tiles ? max_tiles : (rows_dense + BM - 1) / BM;
  return launch_gemm(kDown, a, mt, stream);
}

}  // namespace moe
