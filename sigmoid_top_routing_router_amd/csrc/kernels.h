// Host-side launchers of the gfx950 kernels (internal to the library).
// Every launcher enqueues on `stream`, performs no allocation and no
// host/device synchronisation, and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#define MOE_KMAX_INTERNAL 8

namespace moe {

// ---------------------------------------------------------------- routing
// zero / zero_n: a buffer of zero_n words that the launch also clears (the
// first EQB histogram, when the routing gives the token bias of an update).
hipError_t launch_route(const float* Z, const float* beta, int64_t N, int E, int K,
                        int32_t* ids, float* S, float* alpha, float* margin,
                        hipStream_t stream, uint32_t* zero = nullptr, size_t zero_n = 0);
// The same with the bias centred on the fly from raw quantiles qraw (the
// last step of an exact quantile update): beta_e = fp32(fp64(-qraw_e) - mean)
// is used for the selection and stored to beta_out (required); beta is
// ignored.
hipError_t launch_route_centred(const float* Z, const float* beta, const float* qraw,
                                float* beta_out, int64_t N, int E, int K, int32_t* ids,
                                float* S, float* alpha, float* margin, hipStream_t stream,
                                uint32_t* zero = nullptr, size_t zero_n = 0);

// Selection fused into the router GEMM (RouterSel given to the router
// launchers below): every column tile of the router product writes, for
// each row, its K + 1 first entries in the selection order (biased score
// descending, expert ascending) to cand_s / cand_e [N][router_col_tiles(E)]
// [K + 1]; the first K + 1 entries of a row lie among them.
struct RouterSel {
  const float* beta;  // selection bias [E] or NULL (zero)
  float* cand_s;      // biased scores
  uint32_t* cand_e;   // their experts
  int K;
};
int router_col_tiles(int E);
// The merge of those lists: the same ids, S, alpha and margin as
// launch_route over Z with the same bias (any of the four may be NULL).
hipError_t launch_route_merge(const float* cand_s, const uint32_t* cand_e, int n_col_tiles,
                              const float* Z, int64_t N, int E, int K, int32_t* ids, float* S,
                              float* alpha, float* margin, hipStream_t stream,
                              uint32_t* zero = nullptr, size_t zero_n = 0);

// ---------------------------------------------------------------- EQB
// Workspace carved by the caller (all 256-byte aligned):
//   hist  [passes][E][256] uint32 (passes = key_bits / 8)
//   state [2*E + 4] uint32 (per-expert key prefix and remaining rank, counter)
//   qraw  [E] fp32 (raw quantiles)
struct EqbWork {
  uint32_t* hist;
  uint32_t* state;
  float* qraw;
};
size_t eqb_hist_bytes(int E, int key_bits);
// One-block centring of raw quantiles: beta_out = fp32(fp64(-qraw) - mean).
hipError_t launch_eqb_centre(const float* qraw, int E, float* beta_out, hipStream_t stream);
size_t eqb_state_bytes(int E);
// hist0_zeroed: the first pass's histogram (hist[0 .. E*256)) is already
// zero (cleared by the routing launch that gave alpha); else a fill clears it.
hipError_t launch_eqb(const float* Z, const float* alpha, int64_t N, int E, int K,
                      int key_bits, float* beta_out, float* quantile_out,
                      const EqbWork& w, hipStream_t stream, bool hist0_zeroed = false);
// The pieces of launch_eqb, for a batch that arrives in several parts: the
// histogram of one pass over one part (added into hist_pass = hist + pass*E*256;
// prefix = w.state), and the selection step of one pass over the summed
// histogram (rank from n_total, the rows of all parts; after the last pass
// the raw quantiles and the centred bias are written).
hipError_t launch_eqb_hist(const float* Z, const float* alpha, int64_t N, int E, int key_bits,
                           int pass, const uint32_t* prefix, uint32_t* hist_pass,
                           hipStream_t stream);
hipError_t launch_eqb_scan(const EqbWork& w, int E, int K, int key_bits, int pass,
                           int64_t n_total, float* beta_out, float* quantile_out,
                           hipStream_t stream);

// ---------------------------------------------------------------- grouping
// Stable counting sort of the (t,k) pairs by expert, plus the m-tile table of
// the grouped GEMMs (tiles of `bm` rows per expert).
struct PermWork {
  uint32_t* block_counts;  // [perm_count_rows(pairs)][E]
  int32_t* counts;         // [E]
  int32_t* offsets;        // [E+1]
  int32_t* sorted_src;     // [N*K]
  int32_t* src_pos;        // [N*K]
  int32_t* tiles;          // [max_tiles][4]: expert, first row, rows, pad
  int32_t* n_tiles;        // [1]
};
int64_t perm_count_rows(int64_t pairs);
int64_t perm_max_tiles(int64_t pairs, int E, int bm);
// Tiles hold bm rows; the last tile of a segment up to bm + xr rows.
// shared_rows > 0 (one-block path only): ceil(shared_rows / 16) more m-tiles
// of at most 16 rows, expert -1, over rows N*K .. N*K + shared_rows - 1
// (the shared expert folded into the weight-streaming products).
hipError_t launch_permute(const int32_t* ids, int64_t N, int E, int K, int bm, int xr,
                          const PermWork& w, hipStream_t stream, int shared_rows = 0);
// Expert loads only (no permutation): counts[E] must be a device buffer.
hipError_t launch_count(const int32_t* ids, int64_t pairs, int E, int32_t* counts,
                        hipStream_t stream);

// ---------------------------------------------------------------- GEMMs
// Router logits Z[N,E] = x[N,d] W_r[E,d]^T (+ offset[E]) in fp32; N*d*2 < 4 GiB.
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w_router,
                              const float* offset, int64_t N, int d, int E, float* Z,
                              hipStream_t stream, const RouterSel* sel = nullptr);
// Grouped SwiGLU gate/up: for every m-tile of the table, H rows =
// silu(X W_g^T) * (X W_u^T) (bf16).  When `tiles` is NULL the rows are the
// tokens 0..N-1 of one expert (shared expert), otherwise A rows are gathered
// through sorted_src / K.  x has x_rows rows; x_rows * d * 2 < 4 GiB.
// kblock_major: w_gate and w_up are [E][d/64][h][64] (moe_pack_gateup_weights)
// instead of [E][h][d].
hipError_t launch_gateup(const uint16_t* x, int64_t x_rows, const int32_t* sorted_src, int K,
                         const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                         int64_t rows_dense, const uint16_t* w_gate,
                         const uint16_t* w_up, int d, int h, uint16_t* H,
                         hipStream_t stream, bool kblock_major = false);
// Grouped down projection: Y rows = H rows W_d^T (bf16 out).  H has h_rows
// rows; h_rows * h * 2 < 4 GiB.
hipError_t launch_down(const uint16_t* H, int64_t h_rows, const int32_t* tiles, const int32_t* n_tiles,
                       int64_t max_tiles, int64_t rows_dense, const uint16_t* w_down,
                       int d, int h, uint16_t* Y, hipStream_t stream);
int gemm_bm();
// Rows beyond gemm_bm() that one grouped m-tile may hold (bf16 and E4M3).
int gemm_xrows();
// Router logits and the shared expert's gate/up in one launch (both read x).
hipError_t launch_router_shared_gateup(const uint16_t* x, int64_t N, int d,
                                       const uint16_t* w_router, const float* offset, int E,
                                       float* Z, const uint16_t* ws_gate,
                                       const uint16_t* ws_up, int hs, uint16_t* Hs,
                                       hipStream_t stream, const RouterSel* sel = nullptr);


// ---------------------------------------------------------------- combine
// y[t] = sh[t] + sum_k S[t,k] * Y[src_pos[t,k]]  (sh may be NULL)
hipError_t launch_combine(const uint16_t* sh, const uint16_t* Y, const float* S,
                          const int32_t* src_pos, int64_t N, int K, int d,
                          uint16_t* y, hipStream_t stream);

// ---------------------------------------------------------------- diagnostics
// Same layout as moe_route_stats_t of the public header.
struct RouteStatsDev {
  double max_vio;
  double intervention_rate;
  int64_t overlap;
  int64_t near_ties;
  int32_t max_load;
  int32_t min_load;
};
// Loads counts[E] of the routed ids [N,K]; MaxVio; the overlap with the
// unbiased top-K ids_u [N,K] (NULL: intervention rate NaN); the number of
// tokens with margin < tau (margin NULL: 0).  Device outputs only.
hipError_t launch_route_stats(const int32_t* ids, const int32_t* ids_u, const float* margin,
                              int64_t N, int E, int K, float tau, int32_t* counts,
                              RouteStatsDev* st, hipStream_t stream);

// ---------------------------------------------------------------- LEI
// Load-Error Injection on the score gradient of one microbatch: loads of the
// routed ids [N,K] into counts[E] (scratch), the per-expert injection into
// inj[E] (scratch; also copied to inj_out when given), then Gout = G + inj
// (G NULL: zero; Gout may equal G) and dZ = Gout * sigma'(Z).  Gout or dZ may
// be NULL; Z is read only for dZ.
hipError_t launch_lei(const float* Z, const int32_t* ids, const float* G, int64_t N, int E,
                      int K, float lam, float tau, float* Gout, float* dZ, float* inj_out,
                      int32_t* counts, float* inj, hipStream_t stream);

// ---------------------------------------------------------------- FP8
// Rows of X [N,C] bf16 (C % 128 == 0) -> E4M3 codes Q [N,C] and one fp32
// scale per 1 x 128 group, S [N, C/128].
hipError_t launch_quant_rows(const uint16_t* X, int64_t N, int C, uint8_t* Q, float* S,
                             hipStream_t stream);
// `count` matrices W [count][R][C] bf16 -> codes Q [count][R][C] and one fp32
// scale per 128 x 128 block, S [count][ceil(R/128)][ceil(C/128)].
hipError_t launch_quant_blocks(const uint16_t* W, int64_t count, int R, int C, uint8_t* Q,
                               float* S, hipStream_t stream);

// E4M3 GEMMs (d % 128 == 0, h % 128 == 0).  Weight scales are
// [E][rows/128][cols/128]; activation scales [rows][cols/128].  The gate/up
// GEMMs leave H as E4M3 codes [rows][h] with scales [rows][h/128] (quantised
// in the epilogue from the fp32 SiLU(g) * u).  kblock_major: the gate and up
// codes are [E][d/128][h][128] (moe_pack_gateup_weights on the codes viewed
// as 16-bit words) instead of [E][h][d].
hipError_t launch_gateup_fp8(const uint8_t* xq, const float* xs, int64_t x_rows,
                             const int32_t* sorted_src, int K, const int32_t* tiles,
                             const int32_t* n_tiles, int64_t max_tiles, int64_t rows_dense,
                             const uint8_t* wg, const float* sg, const uint8_t* wu,
                             const float* su, int d, int h, uint8_t* Hq, float* Hs,
                             hipStream_t stream, bool kblock_major = false);
hipError_t launch_down_fp8(const uint8_t* Hq, const float* Hs, int64_t h_rows,
                           const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                           int64_t rows_dense, const uint8_t* wd, const float* sd, int d, int h,
                           uint16_t* Y, hipStream_t stream);
hipError_t launch_router_shared_gateup_fp8(const uint16_t* x, const uint8_t* xq, const float* xs,
                                           int64_t N, int d, const uint16_t* w_router,
                                           const float* offset, int E, float* Z,
                                           const uint8_t* wsg, const float* ssg,
                                           const uint8_t* wsu, const float* ssu, int hs,
                                           uint8_t* Hsq, float* Hss, hipStream_t stream,
                                           const RouterSel* sel = nullptr);

// The shared expert as more m-tiles of the weight-streaming products
// (batches of at most 64 tokens with h_shared == h): the tile table's
// entries with expert -1 cover rows row0 .. row0 + N - 1 of H and Y (tokens
// 0 .. N - 1 of x, in order) with these row-major weights (E4M3: and
// scales).
struct SharedFold {
  const void* gate;
  const void* up;
  const void* down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  int64_t row0;
};
// Weight-streaming variants of the routed (grouped) products for batches of
// at most 64 tokens (every tile then holds at most 64 rows); same arguments
// and results as the launchers above, `tiles` required.
constexpr int64_t kSmallBatch = 64;
hipError_t launch_gateup_small(const uint16_t* x, int64_t x_rows, const int32_t* sorted_src,
                               int K, const int32_t* tiles, const int32_t* n_tiles,
                               int64_t max_tiles, int64_t rows_dense, const uint16_t* w_gate,
                               const uint16_t* w_up, int d, int h, uint16_t* H,
                               hipStream_t stream, bool kblock_major = false,
                               const SharedFold* sf = nullptr);
// Packs [E][rows][cols] bf16 (cols % 64 == 0) into [E][cols/64][rows][64].
hipError_t launch_pack_kblocks(const uint16_t* w, int64_t E, int rows, int cols, uint16_t* out,
                               hipStream_t stream);
hipError_t launch_down_small(const uint16_t* H, int64_t h_rows, const int32_t* tiles,
                             const int32_t* n_tiles, int64_t max_tiles, int64_t rows_dense,
                             const uint16_t* w_down, int d, int h, uint16_t* Y,
                             hipStream_t stream, const SharedFold* sf = nullptr);
hipError_t launch_gateup_fp8_small(const uint8_t* xq, const float* xs, int64_t x_rows,
                                   const int32_t* sorted_src, int K, const int32_t* tiles,
                                   const int32_t* n_tiles, int64_t max_tiles, int64_t rows_dense,
                                   const uint8_t* wg, const float* sg, const uint8_t* wu,
                                   const float* su, int d, int h, uint8_t* Hq, float* Hs,
                                   hipStream_t stream, bool kblock_major = false,
                                   const SharedFold* sf = nullptr);
hipError_t launch_down_fp8_small(const uint8_t* Hq, const float* Hs, int64_t h_rows,
                                 const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles,
                                 int64_t rows_dense, const uint8_t* wd, const float* sd, int d,
                                 int h, uint16_t* Y, hipStream_t stream,
                                 const SharedFold* sf = nullptr);

// Dense products of a batch of at most 64 tokens (router, shared expert),
// split over 64-row weight blocks and 256-wide k chunks; `part` holds
// dense_small_part_floats() fp32 partial sums.  x / H are bf16, or E4M3
// codes with 1 x 128 scales when fp8 (weights then codes with 128 x 128
// block scales); the gate/up result is H in bf16, or E4M3 codes + scales.
size_t dense_small_part_floats(int64_t N, int d, int E, int hs);
hipError_t launch_router_dense_small(const uint16_t* x, const uint16_t* w_router,
                                     const float* offset, int64_t N, int d, int E, float* Z,
                                     float* part, hipStream_t stream);
hipError_t launch_shared_gateup_dense_small(const void* x, const float* xs, int64_t N, int d,
                                            const void* wg, const float* sg, const void* wu,
                                            const float* su, int hs, bool fp8, void* H,
                                            float* Hs, float* part, hipStream_t stream);
hipError_t launch_shared_down_dense_small(const void* H, const float* Hs, int64_t N, int d,
                                          const void* wd, const float* sd, int hs, bool fp8,
                                          uint16_t* Y, float* part, hipStream_t stream);

// ---------------------------------------------------------------- misc
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, size_t n, hipStream_t stream);

// Raises a kernel's dynamic LDS limit to `bytes` once per device (the
// attribute has to be set before the first launch that needs more than the
// default).  `done` holds one bit per device id below 32; concurrent callers
// may both set it, which is harmless.
inline hipError_t set_lds_limit_once(const void* fn, int bytes, std::atomic<uint32_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = (dev >= 0 && dev < 32) ? (1u << dev) : 0u;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace moe
