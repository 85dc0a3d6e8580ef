/*
 * moe_mi355x.h - C ABI of the sigmoid top-K routed MoE layer for MI355X (gfx950).
 *
 * The layer follows "Kolibri Pre-Training from Scratch: UniBPE, Hybrid
 * Attention and Exact Quantile Balancing" (blog post; cited below as [KPT])
 * and "Kolibri 1 im Detail: hybride RNoPE-Attention, Sparse MoE und
 * FP8-Serving" (German architecture guide; cited as [K1D]).
 *
 * Notation: N tokens (T on the pages), d model width, E routed experts,
 * K experts per token, h routed hidden width, hs shared hidden width.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is device memory owned by the caller (normally a
 *    contiguous row-major torch tensor).  The library never allocates or
 *    frees memory and keeps no pointer after the call returns.
 *  - bfloat16 data is passed as raw 16-bit patterns (uint16_t).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without waiting.  There is no device-to-host copy
 *    inside any call.
 *  - Arguments are checked before anything is enqueued; a rejected call
 *    returns a non-zero status and touches no memory.
 *    moe_last_error_message() then describes the problem (thread-local).
 *  - Outputs are fully overwritten and must not alias inputs.  Workspace
 *    contents are undefined on entry and on exit; concurrent calls need
 *    distinct workspaces.
 *  - Results are deterministic run to run (no floating-point atomics).
 *  - Non-finite logits or inputs are outside the contract.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad flag, aliasing */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,  /* a size outside the limits stated below */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP launch error; see the message */
} moe_status_t;

/* Size limits of every entry point: 1 <= N <= 2^24, 1 <= K <= 8,
 * K < E <= 384, and for the layer also d % 64 == 0 (64 <= d <= 8192),
 * h % 32 == 0 (32 <= h <= 4096), hs % 32 == 0, n_shared in {0, 1}, and
 * N*d, N*K*h and N*hs each below 2^31 (every bf16 GEMM operand under 4 GiB;
 * e.g. N <= 838,860 at d = 2560, K = 6, h = 512).  A larger layer is rejected
 * with MOE_ERR_UNSUPPORTED_SHAPE. */
#define MOE_MAX_E 384
#define MOE_MAX_K 8

/* Flags of moe_problem_t.flags */
#define MOE_RECOMPUTE_BIAS 0x1u  /* route with beta_in, one exact quantile update, re-route */
#define MOE_KEY32 0x2u           /* quantile over fp32 keys instead of bf16 keys */
#define MOE_PACKED_GATEUP 0x4u   /* w_gate, w_up packed by moe_pack_gateup_weights */
/* Select the experts inside the router GEMM's epilogue ([KPT] §6.1 routing
 * equations, §7.1 token bias): every column tile of the router product also
 * writes each row's K + 1 first (biased score, expert) entries, and a merge
 * ranks them.  The outputs are the same as without the flag (a separate pass
 * over the stored logits, the default, which measured faster); batches of at
 * most 64 tokens and calls with logits_in ignore the flag. */
#define MOE_ROUTE_FUSED 0x8u

/*
 * moe_route - bias-corrected top-K selection and sigmoid mixture weights over
 * given logits.  [KPT] §6.1 routing equations: B = Z + 1 beta^T is used for
 * selection only; S = sigmoid(Z) of the unbiased logits, not renormalised
 * ([K1D] "Routing", steps 1 and 2).  Also emits the token bias of [KPT] §7.1,
 * alpha_t = -(the (K+1)-th largest entry of B_t).
 *
 *  logits       [N,E] fp32, row-major (Z).
 *  beta         [E] fp32 correction bias, or NULL for zero.
 *  topk_ids     [N,K] int32 out: per token, B descending, ties -> lower id.
 *  topk_weights [N,K] fp32 out: sigmoid(Z[t, id]) (evaluated in fp64).
 *  alpha        [N] fp32 out or NULL: -(B_(K+1)), with -0 read as +0.
 *  margin       [N] fp32 out or NULL: B_(K) - B_(K+1) (near-tie indicator).
 * Pointers 4-byte aligned.  Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, HIP.
 */
moe_status_t moe_route(const float* logits, const float* beta, int64_t N,
                       int32_t E, int32_t K, int32_t* topk_ids,
                       float* topk_weights, float* alpha, float* margin,
                       void* stream);

/*
 * moe_eqb_bias - one exact expert-bias update of Quantile Balancing.
 * [KPT] §7.1: beta_e = -Q_r(Z[:,e] + alpha), r = floor(N*K/E), then centred
 * (mean subtracted); Q_m is the (m+1)-th largest entry ([KPT] §1).  The
 * quantile is found exactly by radix selection over order-preserving integer
 * keys with 256-bin per-expert histograms ([KPT] §7.3): two passes over
 * 16-bit keys of the bf16-rounded values v = bf16(fp32(Z + alpha))
 * (key_bits = 16, the pages' form) or four passes over fp32 keys
 * (key_bits = 32).  Centring: fp64 sum in expert order / E, subtracted in
 * fp64, rounded to fp32.
 *
 *  logits       [N,E] fp32.
 *  beta_in      [E] fp32 or NULL: only used when alpha is NULL, to compute
 *               alpha = -(B_(K+1)) with B = Z + beta_in (as moe_route).
 *  alpha        [N] fp32 token bias or NULL.
 *  beta_out     [E] fp32 out: centred bias.
 *  quantile_out [E] fp32 out or NULL: the raw quantiles Q_r (beta_raw = -Q).
 *  workspace    device scratch of at least moe_eqb_workspace_bytes(N, E,
 *               key_bits) bytes, 256-byte aligned; 0 from the query means
 *               N < 1, E < 1 or key_bits not 16 / 32.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL, HIP.
 */
size_t moe_eqb_workspace_bytes(int64_t N, int32_t E, int32_t key_bits);
moe_status_t moe_eqb_bias(const float* logits, const float* beta_in,
                          const float* alpha, int64_t N, int32_t E, int32_t K,
                          int32_t key_bits, float* beta_out, float* quantile_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Exact quantile update over a batch that arrives in several parts
 * (microbatches), with the result of moe_eqb_bias on the whole batch.
 * [KPT] §7.3: the quantile of a distributed batch is exact when the
 * per-expert 256-bin histograms of each radix pass are summed over all parts
 * before the bin holding the wanted rank is chosen; the sum is independent of
 * how the batch is split (summing local quantiles instead would not be).
 * On one GPU the parts are added into one state buffer, in any order.
 *
 * Use, with passes = key_bits / 8:
 *   moe_eqb_begin(E, key_bits, state)                 zero the histograms
 *   for pass in 0 .. passes-1:
 *     for every part:  moe_eqb_accumulate(pass, Z_part, alpha_part, N_part, ...)
 *     moe_eqb_select(pass, n_total, E, K, ...)        n_total = sum of N_part
 * The last moe_eqb_select writes beta_out (centred, as moe_eqb_bias) and the
 * raw quantiles.  Calls are stream-ordered: all calls of one update go to one
 * stream (or are ordered by events).
 *
 *  state        device buffer of moe_eqb_state_bytes(E, key_bits) bytes,
 *               256-byte aligned, owned by the caller; it carries the update
 *               from moe_eqb_begin to the last moe_eqb_select.
 *  Z_part       [N_part, E] fp32 logits of one part; alpha_part [N_part] its
 *               token biases (alpha = -(B_(K+1)), e.g. from moe_route).
 *  n_total      the rows of all parts together (sets r = floor(n_total*K/E));
 *               a value other than the sum of N_part gives an unspecified bias.
 *  beta_out     [E] fp32, required at the last pass; quantile_out [E] or NULL.
 * Errors: INVALID_ARGUMENT (pass out of range, NULL or misaligned pointers),
 * UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL (state too small), HIP.
 */
size_t moe_eqb_state_bytes(int32_t E, int32_t key_bits);
moe_status_t moe_eqb_begin(int32_t E, int32_t key_bits, void* state, size_t state_bytes,
                           void* stream);
moe_status_t moe_eqb_accumulate(int32_t pass, const float* logits, const float* alpha,
                                int64_t N, int32_t E, int32_t key_bits, void* state,
                                size_t state_bytes, void* stream);
moe_status_t moe_eqb_select(int32_t pass, int64_t n_total, int32_t E, int32_t K,
                            int32_t key_bits, float* beta_out, float* quantile_out,
                            void* state, size_t state_bytes, void* stream);

/*
 * moe_route_stats - routing diagnostics of one batch, on the device.
 * [KPT] §6.2: MaxVio = max_e c_e / (K N / E) - 1 over the expert loads c_e.
 * [KPT] §9: intervention rate = mean_t (1 - |I^u_t ∩ I_t| / K), the share of
 * routed slots that the bias moved away from the router's own top-K I^u_t;
 * it approaches 1 - K/E when the bias decides the selection.  Near-ties are
 * tokens whose margin B_(K) - B_(K+1) is below tau (selections there may
 * differ under rounding).
 *
 *  topk_ids          [N,K] int32 routed ids (e.g. moe_route with the bias);
 *                    ids outside [0,E) are not counted.
 *  topk_ids_unbiased [N,K] int32 or NULL: the top-K of the logits alone
 *                    (moe_route with beta = NULL); NULL gives a NaN rate.
 *  margin            [N] fp32 or NULL (near_ties = 0).
 *  counts            [E] int32 out: the loads c_e.
 *  stats             one moe_route_stats_t out, in device memory, 8-byte
 *                    aligned.  The integer fields are exact; the rates are
 *                    formed in fp64 from them.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, HIP.
 */
typedef struct {
  double max_vio;            /* max_e c_e / (K N / E) - 1 */
  double intervention_rate;  /* 1 - overlap / (K N), or NaN */
  int64_t overlap;           /* sum_t |I^u_t ∩ I_t| */
  int64_t near_ties;         /* #{t : margin_t < tau} */
  int32_t max_load;          /* max_e c_e */
  int32_t min_load;          /* min_e c_e */
} moe_route_stats_t;
moe_status_t moe_route_stats(const int32_t* topk_ids, const int32_t* topk_ids_unbiased,
                             const float* margin, int64_t N, int32_t E, int32_t K, float tau,
                             int32_t* counts, moe_route_stats_t* stats, void* stream);

/*
 * moe_lei_backward - Load-Error Injection on the routing-score gradient of
 * one microbatch ([KPT] §8).  With the loads c_e of the microbatch's routed
 * ids, f_e = c_e / (K N / E), rho = f - 1, xi = ||rho||_inf / tau:
 *   grad_scores_out[t,e] = grad_scores[t,e] + lam * tanh(xi)/xi * rho_e
 * for every token and expert (the factor is 1 at xi = 0; the injection stays
 * below lam * tau), and through S = sigma(Z):
 *   grad_logits_out[t,e] = grad_scores_out[t,e] * sigma(Z)(1 - sigma(Z)).
 * The pages use lam = 1e-5, tau = 1.  rho, xi and the factor are formed in
 * fp64, the injection rounded once to fp32, the rest in fp32.
 *
 *  logits          [N,E] fp32 (required for grad_logits_out).
 *  topk_ids        [N,K] int32 routed ids of the microbatch (ids outside
 *                  [0,E) are not counted).
 *  grad_scores     [N,E] fp32 gradient with respect to the sigmoid scores,
 *                  or NULL (zero); grad_scores_out may be the same buffer.
 *  grad_scores_out [N,E] fp32 out or NULL; grad_logits_out [N,E] fp32 out or
 *                  NULL (at least one; it must not alias an input).
 *  injection_out   [E] fp32 out or NULL: lam * tanh(xi)/xi * rho_e.
 *  workspace       moe_lei_workspace_bytes(E) bytes, 256-byte aligned.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL, HIP.
 */
size_t moe_lei_workspace_bytes(int32_t E);
moe_status_t moe_lei_backward(const float* logits, const int32_t* topk_ids,
                              const float* grad_scores, int64_t N, int32_t E, int32_t K,
                              float lam, float tau, float* grad_scores_out,
                              float* grad_logits_out, float* injection_out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Problem description of moe_forward. */
typedef struct {
  int64_t N;          /* tokens */
  int32_t d;          /* model width */
  int32_t E;          /* routed experts */
  int32_t K;          /* experts per token */
  int32_t h;          /* routed expert hidden width */
  int32_t n_shared;   /* 0 or 1 always-on shared expert */
  int32_t h_shared;   /* shared expert hidden width */
  uint32_t flags;     /* MOE_RECOMPUTE_BIAS | MOE_KEY32 | MOE_PACKED_GATEUP | MOE_ROUTE_FUSED */
  const float* logit_offset; /* [E] fp32 or NULL: added to Z before the bias
                                (an input-side knob, not part of the method) */
  const float* logits_in;    /* [N,E] fp32 or NULL: use these logits instead
                                of computing x W_r^T */
} moe_problem_t;

/* Weights, all bfloat16 bits, row-major, 16-byte aligned.  Shapes follow
 * [K1D] "Routing" (SwiGLU expert: two d->h projections, SiLU(gate)*up, then
 * h->d, no biases). */
typedef struct {
  const uint16_t* w_router;  /* [E,d]  (may be NULL when logits_in is set) */
  const uint16_t* w_gate;    /* [E,h,d] */
  const uint16_t* w_up;      /* [E,h,d] */
  const uint16_t* w_down;    /* [E,d,h] */
  const uint16_t* ws_gate;   /* [n_shared,hs,d] */
  const uint16_t* ws_up;     /* [n_shared,hs,d] */
  const uint16_t* ws_down;   /* [n_shared,d,hs] */
} moe_weights_t;

/* Optional outputs of moe_forward; every field may be NULL. */
typedef struct {
  float* logits;          /* [N,E] Z (after logit_offset) */
  int32_t* topk_ids;      /* [N,K] final selection */
  float* topk_weights;    /* [N,K] */
  float* alpha;           /* [N] token bias of the first routing (beta_in) */
  float* margin;          /* [N] selection margin of the final routing */
  float* beta_out;        /* [E] centred bias (MOE_RECOMPUTE_BIAS only) */
  float* quantile_out;    /* [E] raw quantiles (MOE_RECOMPUTE_BIAS only) */
  int32_t* counts_before; /* [E] loads of the beta_in routing */
  int32_t* counts;        /* [E] loads of the final routing */
  int32_t* offsets;       /* [E+1] exclusive sums of counts */
  int32_t* sorted_src;    /* [N*K] pair index t*K+k, grouped by expert, t ascending */
  int32_t* src_pos;       /* [N,K] inverse of sorted_src */
} moe_aux_t;

/*
 * moe_forward - the MoE layer forward pass, [KPT] §6.1:
 *   y_t = f_shared(x_t) + sum_{e in I_t} S_{t,e} f_e(x_t)
 * with Z = x W_r^T (+ logit_offset) in fp32, I_t the top-K of Z + beta,
 * S = sigmoid(Z).  With MOE_RECOMPUTE_BIAS the batch is first routed with
 * beta_in, one exact quantile update computes the new bias over the batch
 * ([KPT] §7.1-§7.3) and the batch is routed again with it (the update the
 * running example of [KPT] §7.2 performs).  Tokens are grouped by expert with
 * a stable counting sort; the expert MLPs run as grouped bf16 MFMA GEMMs
 * with fp32 accumulation; the hidden activations and the per-pair expert
 * outputs are held in bf16; the combine accumulates in fp32.
 * The shared expert's two products run on a second,
 * library-owned non-blocking stream (one per device and host thread, created
 * on first use, default priority), forked from `stream` at the call's start
 * and joined back into it before the combine: `stream` still orders the whole
 * call, and capturing `stream` into a HIP graph captures both branches.
 * Graph capture: make one uncaptured call of the same entry point with the
 * same problem, on the same device and host thread, before capturing.  The first call on a thread creates the side
 * stream and its events, and the first call on a device sets the kernels' LDS
 * attributes and queries their occupancy; none of these are stream work, and
 * they are not meant to run under capture.
 *
 *  p        problem (sizes, flags, optional logits_in / logit_offset).
 *  w        weights (see moe_weights_t).
 *  x        [N,d] bf16 bits.
 *  beta_in  [E] fp32 or NULL (zero).
 *  y        [N,d] bf16 bits out.
 *  aux      optional outputs, or NULL.
 *  workspace/workspace_bytes: scratch of at least
 *           moe_forward_workspace_bytes(p), 256-byte aligned.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, WORKSPACE_TOO_SMALL, HIP.
 */
size_t moe_forward_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_forward(const moe_problem_t* p, const moe_weights_t* w,
                         const uint16_t* x, const float* beta_in, uint16_t* y,
                         moe_aux_t* aux, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Packed gate/up weights, for moe_forward, moe_forward_noalloc and
 * moe_forward_fp8 with MOE_PACKED_GATEUP.  The routed experts' gate and up
 * products of the SwiGLU in [K1D] (Routing section) read their weights 128
 * bytes of every row at a time; this layout keeps the pieces read together
 * next to each other.  It changes no value and no order of arithmetic: the
 * layer's output with packed weights is bit-identical to the row-major one.
 *
 * moe_pack_gateup_weights - `count` matrices of 16-bit words w
 *   [count,rows,cols] (row-major) -> out [count, cols/64, rows, 64], i.e.
 *   out[c][k][r][j] = w[c][r][64k + j].  For bf16 experts w is the layer's
 *   w_gate or w_up [E,h,d]; for E4M3 experts it is their codes [E,h,d]
 *   viewed as [E,h,d/2] words, so that each row's 128-code k-blocks stay
 *   whole: out is then the codes [E, d/128, h, 128] (the block scales are
 *   not packed).  cols % 64 == 0 (64 <= cols <= 65536),
 *   1 <= rows <= 65536, 0 <= count <= 65535; w and out are caller-owned
 *   device memory, 16-byte aligned, not overlapping.  Enqueues one kernel
 *   on `stream`; out is fully overwritten.  With MOE_PACKED_GATEUP set, the
 *   forward calls read w_gate and w_up in this layout (the shared expert
 *   and w_down stay row-major).
 * Errors: INVALID_ARGUMENT (NULL, misaligned or overlapping buffers),
 *   UNSUPPORTED_SHAPE, HIP.
 */
moe_status_t moe_pack_gateup_weights(const uint16_t* w, int64_t count, int32_t rows,
                                     int32_t cols, uint16_t* out, void* stream);

/*
 * FP8 (E4M3) experts, [K1D] FP8 section: expert weights stored as E4M3 in
 * 128 x 128 blocks with one fp32 scale per block, activations quantised on
 * the fly in 1 x 128 groups of a row; the router stays bf16.  The pages fix
 * the format but not the scale rule; here every group or block uses
 * s = fp32(amax) / 448 (448 = largest E4M3 value) and each value v becomes
 * the E4M3 code of min(max(fp32(v / s), -448), 448), rounded to nearest even;
 * an all-zero group gets s = 0 and zero codes.  A value is code * scale.
 *
 * moe_fp8_quantize_blocks - `count` bf16 matrices w [count,rows,cols] ->
 *   codes [count,rows,cols] (uint8) and scales
 *   [count, ceil(rows/128), ceil(cols/128)] fp32 (ragged edge blocks use
 *   their valid part).  1 <= rows, cols <= 65536, count >= 0.
 * moe_fp8_quantize_rows - bf16 rows x [n,cols] -> codes [n,cols] and scales
 *   [n, cols/128]; cols % 128 == 0 (128 <= cols <= 65536), n >= 0, x
 *   4-byte aligned.
 * Both enqueue one kernel on `stream`; outputs are fully overwritten.
 * Errors: INVALID_ARGUMENT (NULL or misaligned pointers), UNSUPPORTED_SHAPE, HIP.
 */
moe_status_t moe_fp8_quantize_blocks(const uint16_t* w, int64_t count, int32_t rows,
                                     int32_t cols, uint8_t* codes, float* scales, void* stream);
moe_status_t moe_fp8_quantize_rows(const uint16_t* x, int64_t n, int32_t cols, uint8_t* codes,
                                   float* scales, void* stream);

/* Weights of moe_forward_fp8.  Codes are E4M3 bytes, row-major, 16-byte
 * aligned; scales fp32 [.., rows/128, cols/128] as moe_fp8_quantize_blocks
 * writes them. */
typedef struct {
  const uint16_t* w_router;  /* [E,d] bf16 (may be NULL when logits_in is set) */
  const uint8_t* w_gate;     /* [E,h,d]   codes */
  const float* s_gate;       /* [E,h/128,d/128] */
  const uint8_t* w_up;       /* [E,h,d] */
  const float* s_up;         /* [E,h/128,d/128] */
  const uint8_t* w_down;     /* [E,d,h] */
  const float* s_down;       /* [E,d/128,h/128] */
  const uint8_t* ws_gate;    /* [n_shared,hs,d] */
  const float* ss_gate;      /* [n_shared,hs/128,d/128] */
  const uint8_t* ws_up;      /* [n_shared,hs,d] */
  const float* ss_up;        /* [n_shared,hs/128,d/128] */
  const uint8_t* ws_down;    /* [n_shared,d,hs] */
  const float* ss_down;      /* [n_shared,d/128,hs/128] */
} moe_fp8_weights_t;

/*
 * moe_forward_fp8 - moe_forward with E4M3 experts (routed and shared).
 * Routing, bias update, grouping and combine are those of moe_forward (the
 * same kernels; ids, weights, loads and grouping equal moe_forward's for
 * the same logits).  x is quantised per 1 x 128 group; each expert computes
 * G = X W_g^T and U = X W_u^T from the codes with fp32 accumulation, one
 * scale product per 128 k; H = SiLU(G) * U is quantised from its fp32 value
 * per 1 x 128 group; then H W_d^T, held in bf16 per pair; the combine
 * accumulates in fp32.  Requires d % 128 == 0, h % 128 == 0 and (with a
 * shared expert) hs % 128 == 0, besides the limits of moe_forward.
 * Arguments and errors as moe_forward; workspace of at least
 * moe_forward_fp8_workspace_bytes(p).  Stage timing covers it as well (the
 * quantisation of x is part of stage 0).
 */
size_t moe_forward_fp8_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_forward_fp8(const moe_problem_t* p, const moe_fp8_weights_t* w,
                             const uint16_t* x, const float* beta_in, uint16_t* y,
                             moe_aux_t* aux, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * moe_forward_noalloc - moe_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The same layer as moe_forward (same kernels, bit-equal
 * results) with its workspace in a fixed device array owned by the library:
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held until the process ends.
 * The caller passes inputs, outputs and aux buffers as for moe_forward.
 * The call allocates nothing and creates no stream or event: the shared
 * expert runs on `stream` (no side stream) and stage timing is not recorded.
 * A problem whose moe_forward_workspace_bytes(p) exceeds the array is
 * rejected with MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (at
 * d=2560, E=384, K=6, h=512 up to 1,483 tokens fit).  Every call on one GPU
 * uses that GPU's one array, whose contents the call treats as undefined on
 * entry and leaves as it ends: calls that overlap on one GPU (several
 * streams or threads) race, so order them on one stream.
 * Errors: as moe_forward.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_forward_noalloc(const moe_problem_t* p, const moe_weights_t* w,
                                 const uint16_t* x, const float* beta_in, uint16_t* y,
                                 moe_aux_t* aux, void* stream);

/*
 * Stage timing (a profiling aid).  moe_stage_timing(1): every moe_forward
 * call records a HIP timing event on its stream at each stage boundary;
 * moe_stage_timing(2): only the two events around stage 3 (the routed
 * gate/up GEMM), which disturb the stream least; 0 turns timing off.  Events
 * are created on first use and reused; no device memory is allocated.
 * moe_stage_times waits for the recorded events, writes the summed
 * milliseconds of each stage since the previous read into
 * ms[MOE_NUM_STAGES], the number of recorded calls into *calls, and clears
 * the record.  Stages: 0 router GEMM and shared-expert gate/up GEMM (one
 * launch), 1 routing (selection, token bias, quantile update, re-route,
 * loads), 2 grouping, 3 routed gate/up GEMM, 4 routed down GEMM, 5 shared
 * down GEMM, 6 weighted combine.  With the shared expert on the side stream
 * stage 0 is the router GEMM alone, the shared expert's
 * work overlaps stages 0-4 and stage 5 is the wait for it at the join.
 * Errors: INVALID_ARGUMENT (NULL outputs, enable outside 0..2), HIP.
 */
#define MOE_NUM_STAGES 7
moe_status_t moe_stage_timing(int32_t enable);
moe_status_t moe_stage_times(double* ms, int64_t* calls);
const char* moe_stage_name(int32_t stage);

/* Status name, e.g. "MOE_ERR_INVALID_ARGUMENT". */
const char* moe_status_string(moe_status_t s);
/* Detail of the last failed call on this thread ("" if none). */
const char* moe_last_error_message(void);
/* Version of this ABI (incremented on any incompatible change). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
