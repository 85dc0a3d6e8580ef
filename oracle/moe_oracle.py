"""CPU oracle for the sigmoid top-K routed MoE layer with Exact Quantile Balancing.

TEST INFRASTRUCTURE.  This module is the plain, slow, obviously correct
statement of what the layer computes.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it; the library's
product path never does, and this module imports nothing from the library.

Sources (cited by page title and section):
  [KPT]  "Kolibri Pre-Training from Scratch: UniBPE, Hybrid Attention and
         Exact Quantile Balancing" (blog post).
  [K1D]  "Kolibri 1 im Detail: hybride RNoPE-Attention, Sparse MoE und
         FP8-Serving" (German architecture guide).

Every step is the definition written out with NumPy (fp64 wherever the pages
leave the precision open), in the pages' notation: T tokens (N), E routed
experts, top-K, logits Z, correction bias beta, biased scores B, selections
I_t, mixture weights S, token bias alpha, quantile Q_m, fair share r.

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):
  * bf16 values are decoded by placing the 16 bits above 16 zero bits.
  * Selection order: B descending, ties to the lower expert id; -0 equals +0
    and is returned as +0.
  * alpha_t = -(the (K+1)-th largest B_t), margin_t = B_(K) - B_(K+1).
  * Quantile keys: v = fp32(Z + alpha) rounded to bf16 (round to nearest
    even) in 16-bit mode, v itself in 32-bit mode; r = floor(T*K/E).
  * Centring: the fp64 sum of beta_raw taken sequentially in expert order,
    divided by E, subtracted in fp64, rounded once to fp32.
  * Mixture weights: sigmoid evaluated in fp64, rounded once to fp32.
  * Grouping: a stable sort of the (t, k) pairs by expert; within an expert
    tokens ascend.
  * Expert MLPs in fp64 with no intermediate rounding.
  * FP8 experts: scale = fp32(amax / 448) per group, codes are the nearest
    E4M3 values of v / scale clamped to +-448; the hidden activations H are
    quantised per 1 x 128 group straight from fp64.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against the pages' worked example, closed forms, brute force on tiny inputs
or library routines.  The router GEMM and the SwiGLU layer have no printed
values on the pages; they are pinned by brute-force loops on tiny inputs and
by special cases (see the tests).
"""
from __future__ import annotations

from typing import Optional

import math
import time

import numpy as np

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------
# bfloat16 helpers
# ---------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits (uint16) -> float32: the 16 bits become the upper half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(F32)


def f32_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits with round-to-nearest, ties to even.

    Finite inputs only.  The low 16 bits are dropped after adding half an
    ulp of the kept part, minus one when the kept part is already even, so
    exact halves land on the even neighbour.
    """
    v = np.ascontiguousarray(v, dtype=F32)
    if not np.all(np.isfinite(v)):
        raise ValueError("bf16 rounding: non-finite input")
    u = v.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def _lap(timings: Optional[dict], key: str, t0: float) -> float:
    """Step timing for callers that ask for it: adds the seconds since t0 to
    timings[key] and returns the current time.  No arithmetic of the method."""
    t = time.perf_counter()
    if timings is not None:
        timings[key] = timings.get(key, 0.0) + (t - t0)
    return t


def _canon(a: np.ndarray) -> np.ndarray:
    """Map -0.0 to +0.0 (in IEEE round-to-nearest, -0 + +0 = +0)."""
    return (np.asarray(a, dtype=F32) + F32(0.0)).astype(F32)


# ---------------------------------------------------------------------------
# [KPT] §1 "Mathematical Setup": quantiles
# ---------------------------------------------------------------------------
def quantile(values, m: int):
    """Q_m(list): the (m+1)-th largest entry (entries with repeats count
    separately).  [KPT] §1, definition of Q_m."""
    a = np.sort(np.asarray(values).ravel())[::-1]
    if not 0 <= m < a.size:
        raise ValueError(f"Q_{m} of a list with {a.size} entries")
    return a[m]


# ---------------------------------------------------------------------------
# [KPT] §6.1 and [K1D] "Routing": router logits, selection, mixture weights
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_offset: Optional[np.ndarray] = None) -> np.ndarray:
    """Z = x W_r^T in fp64, rounded once to fp32 ([K1D] "Routing": the router
    emits FP32 logits of shape [N, 384]).  An optional per-expert offset (a
    workload knob, not part of the method) is then added in fp32."""
    z = (np.asarray(x, F64) @ np.asarray(w_router, F64).T).astype(F32)
    if logit_offset is not None:
        z = (z + np.asarray(logit_offset, F32)[None, :]).astype(F32)
    return z


def route(Z: np.ndarray, beta: Optional[np.ndarray], K: int):
    """Selection with the correction bias ([KPT] §6.1; [K1D] "Routing" step 1).

    B = Z + 1_T beta^T in fp32.  I_t = the K largest entries of row t of B,
    ordered by (B descending, expert id ascending).  Also returns the token
    bias alpha_t = -Q_K(B_t) ([KPT] §7.1: -(the (K+1)-th largest)) and the
    selection margin B_(K) - B_(K+1).
    Returns (ids [T,K] int32, alpha [T] fp32, margin [T] fp32).
    """
    Z = np.asarray(Z, F32)
    T, E = Z.shape
    if not 1 <= K < E:
        raise ValueError("need 1 <= K < E")
    b = np.zeros(E, F32) if beta is None else np.asarray(beta, F32)
    B = _canon(Z + b[None, :])
    # A stable sort of -B keeps equal values in ascending expert order.
    order = np.argsort(-B, axis=1, kind="stable")
    ids = order[:, :K].astype(np.int32)
    kth = np.take_along_axis(B, order[:, K - 1:K], axis=1)[:, 0]
    k1th = np.take_along_axis(B, order[:, K:K + 1], axis=1)[:, 0]
    alpha = (-k1th).astype(F32)
    margin = (kth - k1th).astype(F32)
    return ids, alpha, margin


def mixture_weights(Z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """S_{t,k} = sigma(Z_{t, I_tk}) from the unbiased logits, not renormalised
    ([KPT] §6.1 "Two details matter"; [K1D] "Routing" step 2).  Evaluated in
    fp64 and rounded once to fp32."""
    z = np.take_along_axis(np.asarray(Z, F32), np.asarray(ids, np.int64), axis=1)
    z64 = z.astype(F64)
    return (1.0 / (1.0 + np.exp(-z64))).astype(F32)


# ---------------------------------------------------------------------------
# [KPT] §7.1-§7.3: Exact Quantile Balancing
# ---------------------------------------------------------------------------
def eqb_keys_values(v: np.ndarray, key_bits: int) -> np.ndarray:
    """Values whose quantile EQB takes.  16-bit mode: v rounded to bfloat16
    ([KPT] §7.3: every bfloat16 value gets a 16-bit key); 32-bit mode: v."""
    v = _canon(v)
    if key_bits == 16:
        return _canon(bf16_to_f32(f32_to_bf16_rne(v)))
    if key_bits == 32:
        return v
    raise ValueError("key_bits must be 16 or 32")


def eqb_expert_bias(Z: np.ndarray, alpha: np.ndarray, K: int, key_bits: int = 16):
    """One expert-bias update of Quantile Balancing, taken exactly ([KPT] §7.1,
    §7.3): beta_e = -Q_r(Z_{:,e} + alpha), r = T*K/E, then centred.

    Returns (beta_new [E] fp32, Q [E] fp32, beta_raw [E] fp32).
    """
    Z = np.asarray(Z, F32)
    T, E = Z.shape
    r = (T * K) // E
    v = (Z + np.asarray(alpha, F32)[:, None]).astype(F32)
    u = eqb_keys_values(v, key_bits)
    Q = np.array([quantile(u[:, e], r) for e in range(E)], dtype=F32)
    beta_raw = (-Q).astype(F32)
    # Centre: the mean of the expert biases is subtracted ([KPT] §7.1, §7.2).
    acc = 0.0
    for e in range(E):
        acc += float(beta_raw[e])
    mean = acc / E
    beta_new = np.array([float(b) - mean for b in beta_raw], dtype=F64).astype(F32)
    return beta_new, Q, beta_raw


def eqb_expert_bias_parts(Z_parts, alpha_parts, K: int, key_bits: int = 16):
    """The update of eqb_expert_bias over a batch given in parts (microbatches,
    or the shards of a distributed batch).  [KPT] §7.3: the quantile that sets
    the bias is the one of the whole batch, exactly, however the rows are
    split; averaging per-part quantiles would not give it.  So the definition
    is the whole-batch update on the rows of all parts together.

    Returns (beta_new [E] fp32, Q [E] fp32, beta_raw [E] fp32).
    """
    Z = np.concatenate([np.asarray(z, F32) for z in Z_parts], axis=0)
    alpha = np.concatenate([np.asarray(a, F32) for a in alpha_parts], axis=0)
    return eqb_expert_bias(Z, alpha, K, key_bits)


# ---------------------------------------------------------------------------
# Grouping by expert (dispatch) and the expert MLPs
# ---------------------------------------------------------------------------
def group_by_expert(ids: np.ndarray, E: int):
    """Stable counting sort of the (t, k) pairs by expert.

    Returns counts c_e [E], offsets [E+1] (exclusive sums), sorted_src [T*K]
    (flat pair index t*K+k in expert order, tokens ascending within an
    expert) and src_pos [T,K] (the inverse: where pair (t,k) landed).
    """
    ids = np.asarray(ids, np.int64)
    T, K = ids.shape
    flat = ids.ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_src = np.argsort(flat, kind="stable").astype(np.int32)
    src_pos = np.empty(T * K, np.int32)
    src_pos[sorted_src] = np.arange(T * K, dtype=np.int32)
    return counts, offsets, sorted_src, src_pos.reshape(T, K)


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
           w_down: np.ndarray) -> np.ndarray:
    """One SwiGLU expert with no biases ([K1D] "Routing", expert paragraph):
    two d -> h projections, SiLU(gate) * up, then h -> d.  fp64 throughout.
    X [n,d], w_gate/w_up [h,d], w_down [d,h] -> [n,d]."""
    X = np.asarray(X, F64)
    G = X @ np.asarray(w_gate, F64).T
    U = X @ np.asarray(w_up, F64).T
    H = silu(G) * U
    return H @ np.asarray(w_down, F64).T


def moe_combine(x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                ids, S, token_subset=None, timings: Optional[dict] = None) -> np.ndarray:
    """y_t = f_shared(x_t) + sum_{e in I_t} S_{t,e} f_e(x_t) ([KPT] §6.1).

    Weights are float arrays of shape [E,h,d]/[E,h,d]/[E,d,h] (routed) and
    [n_shared,hs,d]/[n_shared,hs,d]/[n_shared,d,hs] (shared; n_shared may be
    0).  ``token_subset`` restricts the output to those tokens (rows of the
    result follow the subset).  Returns fp64 [T', d].  ``timings`` (a dict,
    optional) receives the seconds spent in the shared expert, the routed
    experts and the weighted sum.
    """
    t = time.perf_counter()
    x = np.asarray(x, F64)
    toks = np.arange(x.shape[0]) if token_subset is None else np.asarray(token_subset)
    xs = x[toks]
    ids_s = np.asarray(ids)[toks]
    S_s = np.asarray(S, F64)[toks]
    y = np.zeros_like(xs)
    t = _lap(timings, "combine", t)
    for s in range(ws_gate.shape[0]):
        f = swiglu(xs, ws_gate[s], ws_up[s], ws_down[s])
        t = _lap(timings, "shared_expert", t)
        y += f
        t = _lap(timings, "combine", t)
    E = w_gate.shape[0]
    for e in range(E):
        rows, slots = np.nonzero(ids_s == e)
        if rows.size == 0:
            continue
        t = _lap(timings, "combine", t)
        f = swiglu(xs[rows], w_gate[e], w_up[e], w_down[e])
        t = _lap(timings, "routed_experts", t)
        y[rows] += S_s[rows, slots][:, None] * f
        t = _lap(timings, "combine", t)
    return y


# ---------------------------------------------------------------------------
# Diagnostics: [KPT] §6.2 MaxVio, §9 intervention rate
# ---------------------------------------------------------------------------
def max_vio(counts: np.ndarray, T: int, K: int, E: int) -> float:
    """MaxVio = max_e [c_e / (K T / E) - 1]  ([KPT] §6.2)."""
    target = K * T / E
    return float(np.max(np.asarray(counts, F64) / target - 1.0))


def intervention_rate(ids_router: np.ndarray, ids_routed: np.ndarray) -> float:
    """I = mean_t (1 - |I^u_t ∩ I_t| / K) ([KPT] §9)."""
    a = np.asarray(ids_router)
    b = np.asarray(ids_routed)
    K = a.shape[1]
    overlap = np.array([len(set(a[t].tolist()) & set(b[t].tolist()))
                        for t in range(a.shape[0])], dtype=F64)
    return float(np.mean(1.0 - overlap / K))


def near_tie_count(margin: np.ndarray, tau: float) -> int:
    """Tokens whose selection margin B_(K) - B_(K+1) is below tau (the
    boundary cases where rounding may change the selection)."""
    return int(np.sum(np.asarray(margin, F64) < float(np.float32(tau))))


# ---------------------------------------------------------------------------
# Load-Error Injection ([KPT] §8): balance inside each microbatch
# ---------------------------------------------------------------------------
def lei_injection(ids: np.ndarray, E: int, lam: float, tau: float):
    """The per-expert term that LEI adds to every token's score gradient.

    f_e = c_e / (K |B| / E) with c_e the loads of the microbatch B, rho = f - 1,
    xi = ||rho||_inf / tau, scale = tanh(xi) / xi (1 at xi = 0 by continuity);
    the injection is lam * scale * rho_e.  fp64 throughout.

    Returns (rho [E] f64, xi, scale, injection [E] f64).
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    counts = np.bincount(ids.ravel(), minlength=E).astype(F64)
    f = counts / (K * T / E)
    rho = f - 1.0
    xi = float(np.max(np.abs(rho))) / tau
    scale = 1.0 if xi == 0.0 else math.tanh(xi) / xi
    return rho, xi, scale, lam * scale * rho


def lei_backward(Z: np.ndarray, ids: np.ndarray, G: Optional[np.ndarray], lam: float,
                 tau: float):
    """Score and logit gradients with LEI ([KPT] §8).

    G [T,E]: incoming gradient with respect to the sigmoid scores
    S_{t,e} = sigma(Z_{t,e}) (None: zero).  G'_{t,e} = G_{t,e} + injection_e
    for every token and expert; the logits receive G' * sigma(Z)(1 - sigma(Z))
    by the chain rule.  fp64.

    Returns (G' [T,E] f64, dZ [T,E] f64).
    """
    Z = np.asarray(Z, F64)
    T, E = Z.shape
    _, _, _, inj = lei_injection(ids, E, lam, tau)
    Gp = (np.zeros((T, E), F64) if G is None else np.asarray(G, F64)) + inj[None, :]
    s = 1.0 / (1.0 + np.exp(-Z))
    return Gp, Gp * s * (1.0 - s)


# ---------------------------------------------------------------------------
# FP8 experts ([K1D] FP8 section): E4M3 weights in 128 x 128 blocks with one
# fp32 scale each, activations quantised per 1 x 128 group of a row.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0  # largest finite E4M3 value ([KPT] §4.4)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal; 0x7F and 0xFF are NaN, there is no inf)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return (sign * v).astype(F64)


_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0..126, ascending


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code, ties to the even code (even mantissa), magnitudes
    above 448 saturated to 448; the sign is kept (so -0.0 -> 0x80)."""
    x = np.asarray(x, F64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _quantize_group(v: np.ndarray):
    """One group (any shape) of fp32 values: s = fp32(amax) / 448 in fp32, the
    codes of fp32(v / s) clamped to +-448 (an all-zero group: s = 0, codes 0)."""
    v = np.asarray(v, F32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    if amax == 0:
        return np.zeros(v.shape, np.uint8), np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    q = np.clip((v / s).astype(F32), -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(q), s


def quantize_weight_blocks(W: np.ndarray, block: int = 128):
    """[R, C] -> (codes [R, C] uint8, scales [ceil(R/b), ceil(C/b)] fp32),
    one scale per block x block tile."""
    W = np.asarray(W, F32)
    R, C = W.shape
    codes = np.zeros((R, C), np.uint8)
    scales = np.zeros(((R + block - 1) // block, (C + block - 1) // block), F32)
    for i in range(scales.shape[0]):
        for j in range(scales.shape[1]):
            blk = W[i * block:(i + 1) * block, j * block:(j + 1) * block]
            q, sc = _quantize_group(blk)
            codes[i * block:(i + 1) * block, j * block:(j + 1) * block] = q
            scales[i, j] = sc
    return codes, scales


def _quantize_group_f64(v: np.ndarray):
    """One group of fp64 values (the SwiGLU hidden activations H, which the
    oracle holds unrounded): s = fp32(amax / 448), an fp32 scale as every
    scale of the FP8 path; the codes of min(max(v / s, -448), 448) with v / s
    taken in fp64 (an all-zero group: s = 0, codes 0)."""
    v = np.asarray(v, F64)
    amax = float(np.max(np.abs(v))) if v.size else 0.0
    s = np.float32(amax / E4M3_MAX)
    if s == 0:
        return np.zeros(v.shape, np.uint8), np.float32(0)
    q = np.clip(v / F64(s), -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(q), s


def quantize_row_groups_f64(X: np.ndarray, group: int = 128):
    """As quantize_row_groups for fp64 rows (each 1 x group piece through
    _quantize_group_f64)."""
    X = np.asarray(X, F64)
    N, C = X.shape
    codes = np.zeros((N, C), np.uint8)
    scales = np.zeros((N, (C + group - 1) // group), F32)
    for j in range(scales.shape[1]):
        for n in range(N):
            q, sc = _quantize_group_f64(X[n, j * group:(j + 1) * group])
            codes[n, j * group:(j + 1) * group] = q
            scales[n, j] = sc
    return codes, scales


def quantize_row_groups(X: np.ndarray, group: int = 128):
    """[N, C] -> (codes [N, C] uint8, scales [N, ceil(C/g)] fp32), one scale
    per 1 x group piece of a row (the dynamic activation quantisation)."""
    X = np.asarray(X, F32)
    N, C = X.shape
    codes = np.zeros((N, C), np.uint8)
    scales = np.zeros((N, (C + group - 1) // group), F32)
    for j in range(scales.shape[1]):
        for n in range(N):
            q, sc = _quantize_group(X[n, j * group:(j + 1) * group])
            codes[n, j * group:(j + 1) * group] = q
            scales[n, j] = sc
    return codes, scales


_E4M3_ALL = e4m3_decode(np.arange(256, dtype=np.uint8))  # the value of every code


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    v = _E4M3_ALL[np.asarray(codes, np.uint8)]
    sc = np.repeat(np.repeat(np.asarray(scales, F64), block, axis=0), block, axis=1)
    return v * sc[:v.shape[0], :v.shape[1]]


def dequantize_row_groups(codes: np.ndarray, scales: np.ndarray, group: int = 128) -> np.ndarray:
    v = _E4M3_ALL[np.asarray(codes, np.uint8)]
    sc = np.repeat(np.asarray(scales, F64), group, axis=1)
    return v * sc[:, :v.shape[1]]


def swiglu_fp8(x_codes, x_scales, g_codes, g_scales, u_codes, u_scales, d_codes, d_scales):
    """One SwiGLU expert on FP8 operands ([K1D] FP8 section): G = X W_g^T and
    U = X W_u^T on the dequantised values, H = SiLU(G) * U, all in fp64; H,
    the activation entering the down projection, is quantised dynamically per
    1 x 128 group straight from fp64 (the pages name no other rounding of
    it); then H W_d^T on the dequantised values."""
    X = dequantize_row_groups(x_codes, x_scales)
    G = X @ dequantize_blocks(g_codes, g_scales).T
    U = X @ dequantize_blocks(u_codes, u_scales).T
    hq, hs = quantize_row_groups_f64(silu(G) * U)
    return dequantize_row_groups(hq, hs) @ dequantize_blocks(d_codes, d_scales).T


def quantize_expert_weights(w_gate, w_up, w_down, ws_gate, ws_up, ws_down) -> dict:
    """Block-quantise every expert matrix ([E,h,d]/[E,h,d]/[E,d,h] routed,
    [S,hs,d]/[S,hs,d]/[S,d,hs] shared) -> dict of codes and scales under the
    names w_gate/s_gate, w_up/s_up, w_down/s_down, ws_gate/ss_gate,
    ws_up/ss_up, ws_down/ss_down."""
    out = {}
    for name, W in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down),
                    ("ws_gate", ws_gate), ("ws_up", ws_up), ("ws_down", ws_down)):
        W = np.asarray(W, F32)
        pairs = [quantize_weight_blocks(m) for m in W]
        sname = "s" + name[1:] if name.startswith("w_") else "ss" + name[2:]
        out[name] = np.stack([c for c, _ in pairs]) if pairs else np.zeros((0,) + W.shape[1:], np.uint8)
        out[sname] = np.stack([sc for _, sc in pairs]) if pairs else \
            np.zeros((0, (W.shape[1] + 127) // 128, (W.shape[2] + 127) // 128), F32)
    return out


def moe_combine_fp8(x, q: dict, ids, S, token_subset=None) -> np.ndarray:
    """y_t = f_shared(x_t) + sum_{e in I_t} S_{t,e} f_e(x_t) ([KPT] §6.1) with
    FP8 experts ([K1D] FP8 section): the rows of x are quantised per 1 x 128
    group and every expert is ``swiglu_fp8`` on its tokens' codes, with the
    weights' codes and block scales in ``q`` (see quantize_expert_weights).
    Returns fp64 [T', d]."""
    x = np.asarray(x, F32)
    toks = np.arange(x.shape[0]) if token_subset is None else np.asarray(token_subset)
    xq, xs = quantize_row_groups(x[toks])
    ids_s = np.asarray(ids)[toks]
    S_s = np.asarray(S, F64)[toks]
    y = np.zeros((len(toks), x.shape[1]), F64)
    for s in range(q["ws_gate"].shape[0]):
        y += swiglu_fp8(xq, xs, q["ws_gate"][s], q["ss_gate"][s], q["ws_up"][s], q["ss_up"][s],
                        q["ws_down"][s], q["ss_down"][s])
    for e in range(q["w_gate"].shape[0]):
        rows, slots = np.nonzero(ids_s == e)
        if rows.size == 0:
            continue
        f = swiglu_fp8(xq[rows], xs[rows], q["w_gate"][e], q["s_gate"][e], q["w_up"][e],
                       q["s_up"][e], q["w_down"][e], q["s_down"][e])
        y[rows] += S_s[rows, slots][:, None] * f
    return y


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------
def moe_layer(x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
              beta_in, K: int, recompute_bias: bool = False, key_bits: int = 16,
              logit_offset=None, logits_in=None, token_subset=None,
              compute_output: bool = True, timings: Optional[dict] = None) -> dict:
    """Forward pass of one MoE layer as [KPT] §6.1 and §7.1 state it.

    x [T,d] and all weights are float arrays (decode bf16 bits with
    ``bf16_to_f32`` first).  With ``recompute_bias`` the batch is routed with
    beta_in, one EQB update computes beta_new over the batch (token bias from
    that routing, expert quantile, centring) and the batch is routed again
    with beta_new ([KPT] §7.2 repairs the toy collapse this way).  The
    ``logits_in`` argument replaces the router product by given logits.
    ``timings`` (a dict, optional) receives the seconds of each step: router,
    route (both routings and the mixture weights), eqb, permutation,
    shared_expert, routed_experts, combine.
    """
    t = time.perf_counter()
    Z = router_logits(x, w_router, logit_offset) if logits_in is None \
        else np.asarray(logits_in, F32)
    T, E = Z.shape
    out = {"logits": Z}
    t = _lap(timings, "router", t)
    ids0, alpha0, margin0 = route(Z, beta_in, K)
    out["counts_before"] = np.bincount(ids0.ravel(), minlength=E).astype(np.int32)
    beta = np.zeros(E, F32) if beta_in is None else np.asarray(beta_in, F32)
    t = _lap(timings, "route", t)
    if recompute_bias:
        beta_new, Q, beta_raw = eqb_expert_bias(Z, alpha0, K, key_bits)
        out.update(alpha=alpha0, beta_out=beta_new, quantile=Q, beta_raw=beta_raw)
        beta = beta_new
        t = _lap(timings, "eqb", t)
        ids, alpha, margin = route(Z, beta, K)
    else:
        ids, alpha, margin = ids0, alpha0, margin0
        out.update(alpha=alpha0)
    S = mixture_weights(Z, ids)
    t = _lap(timings, "route", t)
    counts, offsets, sorted_src, src_pos = group_by_expert(ids, E)
    out.update(topk_ids=ids, topk_weights=S, margin=margin, counts=counts,
               offsets=offsets, sorted_src=sorted_src, src_pos=src_pos,
               route_alpha=alpha)
    _lap(timings, "permutation", t)
    if compute_output:
        out["y"] = moe_combine(x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                               ids, S, token_subset, timings)
    return out
