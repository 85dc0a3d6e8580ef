"""MI355X (gfx950) sigmoid top-K routed MoE layer with Exact Quantile Balancing.

Thin binding over the C ABI of libmoe_mi355x.so (include/moe_mi355x.h):
``route``, ``eqb_bias`` and ``forward`` marshal torch tensors (device memory
and the current stream) into the library calls; every step of the layer runs
in the library's HIP kernels.  There is no CPU fallback: a missing library or
a non-GPU tensor raises.
"""
from __future__ import annotations

import contextlib
import ctypes as C
from dataclasses import dataclass, replace
from typing import Optional

from . import _lib
from ._lib import (MOE_KEY32, MOE_PACKED_GATEUP, MOE_RECOMPUTE_BIAS, MOE_ROUTE_FUSED, MoeAux,
                   MoeError,
                   MoeFp8Weights, MoeProblem, MoeWeights)

__all__ = ["route", "eqb_bias", "eqb_workspace_bytes", "EqbState", "eqb_bias_parts",
           "route_stats", "read_route_stats", "lei_backward", "forward",
           "forward_workspace_bytes", "fp8_quantize_blocks", "fp8_quantize_rows",
           "Fp8ExpertWeights", "quantize_experts", "forward_fp8", "forward_fp8_workspace_bytes",
           "ExpertWeights", "MoeError", "load_library", "stage_timing", "stage_times",
           "forward_noalloc", "pack_gateup", "pack_gateup_weights"]

AUX_FIELDS = [f for f, _ in MoeAux._fields_]


def load_library():
    return _lib.load()


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context of a call: with an explicit stream, the outputs and
    temporaries of the call are allocated on that stream, so torch's caching
    allocator does not hand their memory to other work before the call's
    kernels on that stream are done."""
    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _bf16():
    torch = _torch()
    return (torch.bfloat16, torch.uint16, torch.int16)


def route(logits, K: int, beta=None, stream=None):
    """Top-K selection on logits + beta, sigmoid weights of the unbiased
    logits.  Returns (ids int32 [N,K], weights fp32 [N,K], alpha fp32 [N],
    margin fp32 [N])."""
    torch = _torch()
    lib = _lib.load()
    logits = _dev(logits, "logits", torch.float32)
    N, E = logits.shape
    beta = _dev(beta, "beta", torch.float32, (E,))
    with _on(stream):
        dev = logits.device
        ids = torch.empty((N, K), dtype=torch.int32, device=dev)
        w = torch.empty((N, K), dtype=torch.float32, device=dev)
        alpha = torch.empty((N,), dtype=torch.float32, device=dev)
        margin = torch.empty((N,), dtype=torch.float32, device=dev)
        _lib.check(lib.moe_route(_ptr(logits), _ptr(beta), N, E, K, _ptr(ids), _ptr(w),
                                 _ptr(alpha), _ptr(margin), _stream(stream)))
    return ids, w, alpha, margin


def route_stats(topk_ids, E: int, topk_ids_unbiased=None, margin=None, tau: float = 1e-3,
                stream=None):
    """Routing diagnostics on the device (moe_route_stats): returns
    (counts [E] int32, stats) where stats is a 40-byte device tensor holding a
    moe_route_stats_t; read_route_stats(stats) copies it to a dict."""
    torch = _torch()
    lib = _lib.load()
    topk_ids = _dev(topk_ids, "topk_ids", torch.int32)
    N, K = topk_ids.shape
    topk_ids_unbiased = _dev(topk_ids_unbiased, "topk_ids_unbiased", torch.int32, (N, K))
    margin = _dev(margin, "margin", torch.float32, (N,))
    with _on(stream):
        counts = torch.empty((E,), dtype=torch.int32, device=topk_ids.device)
        stats = torch.empty((C.sizeof(_lib.MoeRouteStats) // 8,), dtype=torch.float64,
                            device=topk_ids.device)
        _lib.check(lib.moe_route_stats(_ptr(topk_ids), _ptr(topk_ids_unbiased), _ptr(margin), N, E,
                                       K, float(tau), _ptr(counts), _ptr(stats), _stream(stream)))
    return counts, stats


def read_route_stats(stats) -> dict:
    """Copy a moe_route_stats_t from the device (synchronises) into a dict."""
    raw = stats.cpu().numpy().tobytes()
    st = _lib.MoeRouteStats.from_buffer_copy(raw)
    return {f: getattr(st, f) for f, _ in _lib.MoeRouteStats._fields_}


def lei_backward(topk_ids, E: int, logits=None, grad_scores=None, lam: float = 1e-5,
                 tau: float = 1.0, scores_out: bool = True, logits_out: bool = True,
                 inplace: bool = False, stream=None):
    """Load-Error Injection on the score gradient of one microbatch
    (moe_lei_backward).  Returns (grad_scores' [N,E] or None,
    grad_logits [N,E] or None, injection [E]).  With inplace=True the
    injection is added into grad_scores itself."""
    torch = _torch()
    lib = _lib.load()
    topk_ids = _dev(topk_ids, "topk_ids", torch.int32)
    N, K = topk_ids.shape
    logits = _dev(logits, "logits", torch.float32, (N, E))
    grad_scores = _dev(grad_scores, "grad_scores", torch.float32, (N, E))
    with _on(stream):
        dev_ = topk_ids.device
        if inplace:
            if grad_scores is None:
                raise ValueError("inplace needs grad_scores")
            gout = grad_scores
        else:
            gout = torch.empty((N, E), dtype=torch.float32, device=dev_) if scores_out else None
        dz = torch.empty((N, E), dtype=torch.float32, device=dev_) if logits_out else None
        inj = torch.empty((E,), dtype=torch.float32, device=dev_)
        need = int(lib.moe_lei_workspace_bytes(E))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev_)
        _lib.check(lib.moe_lei_backward(_ptr(logits), _ptr(topk_ids), _ptr(grad_scores), N, E, K,
                                        float(lam), float(tau), _ptr(gout), _ptr(dz), _ptr(inj),
                                        _ptr(ws), ws.numel(), _stream(stream)))
    return gout, dz, inj


def eqb_workspace_bytes(N: int, E: int, key_bits: int = 16) -> int:
    return int(_lib.load().moe_eqb_workspace_bytes(N, E, key_bits))


def eqb_bias(logits, K: int, beta_in=None, alpha=None, key_bits: int = 16,
             workspace=None, stream=None):
    """One exact Quantile Balancing update.  Returns (beta_out [E],
    quantile [E]) in fp32."""
    torch = _torch()
    lib = _lib.load()
    logits = _dev(logits, "logits", torch.float32)
    N, E = logits.shape
    beta_in = _dev(beta_in, "beta_in", torch.float32, (E,))
    alpha = _dev(alpha, "alpha", torch.float32, (N,))
    with _on(stream):
        need = int(lib.moe_eqb_workspace_bytes(N, E, key_bits))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=logits.device)
        beta_out = torch.empty((E,), dtype=torch.float32, device=logits.device)
        q = torch.empty((E,), dtype=torch.float32, device=logits.device)
        _lib.check(lib.moe_eqb_bias(_ptr(logits), _ptr(beta_in), _ptr(alpha), N, E, K, key_bits,
                                    _ptr(beta_out), _ptr(q), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
    return beta_out, q


class EqbState:
    """Exact quantile update over a batch that arrives in parts
    (moe_eqb_begin / moe_eqb_accumulate / moe_eqb_select).  Owns the device
    state buffer; use: ``st = EqbState(E, K, n_total)``, then for every pass
    ``st.accumulate(pass_, Z_part, alpha_part)`` over all parts and
    ``st.select(pass_)``; the last select returns (beta_out, quantile)."""

    def __init__(self, E: int, K: int, n_total: int, key_bits: int = 16, device=None,
                 stream=None):
        torch = _torch()
        self.lib = _lib.load()
        self.E, self.K, self.n_total, self.key_bits = E, K, n_total, key_bits
        self.passes = key_bits // 8
        self.stream = stream
        nbytes = int(self.lib.moe_eqb_state_bytes(E, key_bits))
        if nbytes == 0:
            raise ValueError(f"unsupported E={E} / key_bits={key_bits}")
        self.state = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
        _lib.check(self.lib.moe_eqb_begin(E, key_bits, _ptr(self.state), nbytes,
                                          _stream(stream)))

    def accumulate(self, pass_: int, logits, alpha):
        torch = _torch()
        logits = _dev(logits, "logits", torch.float32)
        N, E = logits.shape
        if E != self.E:
            raise ValueError(f"logits have E={E}, state has E={self.E}")
        alpha = _dev(alpha, "alpha", torch.float32, (N,))
        _lib.check(self.lib.moe_eqb_accumulate(pass_, _ptr(logits), _ptr(alpha), N, E,
                                               self.key_bits, _ptr(self.state),
                                               self.state.numel(), _stream(self.stream)))

    def select(self, pass_: int):
        torch = _torch()
        last = pass_ == self.passes - 1
        beta = torch.empty((self.E,), dtype=torch.float32, device=self.state.device) if last else None
        q = torch.empty((self.E,), dtype=torch.float32, device=self.state.device) if last else None
        _lib.check(self.lib.moe_eqb_select(pass_, self.n_total, self.E, self.K, self.key_bits,
                                           _ptr(beta), _ptr(q), _ptr(self.state),
                                           self.state.numel(), _stream(self.stream)))
        return (beta, q) if last else None


def eqb_bias_parts(logits_parts, alpha_parts, K: int, key_bits: int = 16, stream=None):
    """moe_eqb_bias over the concatenation of the parts, computed part by part
    (histograms summed over the parts for every radix pass).  Returns
    (beta_out [E], quantile [E])."""
    n_total = sum(int(z.shape[0]) for z in logits_parts)
    E = int(logits_parts[0].shape[1])
    st = EqbState(E, K, n_total, key_bits, device=logits_parts[0].device, stream=stream)
    out = None
    for p in range(st.passes):
        for z, a in zip(logits_parts, alpha_parts):
            st.accumulate(p, z, a)
        out = st.select(p)
    return out


@dataclass
class ExpertWeights:
    """bf16 weights of one MoE layer (torch tensors on the GPU)."""
    w_router: object        # [E, d]
    w_gate: object          # [E, h, d]
    w_up: object            # [E, h, d]
    w_down: object          # [E, d, h]
    ws_gate: object = None  # [S, hs, d]
    ws_up: object = None    # [S, hs, d]
    ws_down: object = None  # [S, d, hs]
    packed: bool = False    # w_gate, w_up as [E, d/64, h, 64] (pack_gateup)


def _problem(N, d, E, K, h, n_shared, h_shared, flags, logit_offset, logits_in):
    return MoeProblem(N, d, E, K, h, n_shared, h_shared, flags,
                      _ptr(logit_offset), _ptr(logits_in))


def forward_workspace_bytes(N, d, E, K, h, n_shared=1, h_shared=None,
                            recompute_bias=False, key_bits=16) -> int:
    flags = (MOE_RECOMPUTE_BIAS if recompute_bias else 0) | (MOE_KEY32 if key_bits == 32 else 0)
    p = _problem(N, d, E, K, h, n_shared, h_shared or h, flags, None, None)
    return int(_lib.load().moe_forward_workspace_bytes(C.byref(p)))


def forward_fp8_workspace_bytes(N, d, E, K, h, n_shared=1, h_shared=None,
                                recompute_bias=False, key_bits=16) -> int:
    flags = (MOE_RECOMPUTE_BIAS if recompute_bias else 0) | (MOE_KEY32 if key_bits == 32 else 0)
    p = _problem(N, d, E, K, h, n_shared, h_shared or h, flags, None, None)
    return int(_lib.load().moe_forward_fp8_workspace_bytes(C.byref(p)))


def pack_gateup_weights(w, stream=None):
    """moe_pack_gateup_weights: bf16 [count, rows, cols] (cols % 64 == 0) ->
    [count, cols/64, rows, 64], out[c, k, r, j] = w[c, r, 64k + j]."""
    torch = _torch()
    w = _dev(w, "w", _bf16())
    if w.dim() != 3:
        raise ValueError("w must be [count, rows, cols]")
    cnt, R, Cc = w.shape
    with _on(stream):
        out = torch.empty((cnt, Cc // 64, R, 64), dtype=torch.bfloat16, device=w.device)
        _lib.check(_lib.load().moe_pack_gateup_weights(_ptr(w), cnt, R, Cc, _ptr(out),
                                                       _stream(stream)))
    return out


def pack_gateup(weights, stream=None):
    """The same layer (ExpertWeights or Fp8ExpertWeights) with its routed
    gate and up weights packed k-block-major (MOE_PACKED_GATEUP); forward()
    and forward_fp8() give bit-identical results with either form.  E4M3
    codes are packed as 16-bit words, so each row's 128-code k-blocks stay
    whole: [E, h, d] -> [E, d/128, h, 128]."""
    if weights.packed:
        return weights
    if isinstance(weights, Fp8ExpertWeights):
        torch = _torch()

        def pack_codes(c):
            c = _dev(c, "codes", torch.uint8)
            return pack_gateup_weights(c.view(torch.bfloat16), stream).view(torch.uint8)
        return replace(weights, w_gate=pack_codes(weights.w_gate),
                       w_up=pack_codes(weights.w_up), packed=True)
    return replace(weights, w_gate=pack_gateup_weights(weights.w_gate, stream),
                   w_up=pack_gateup_weights(weights.w_up, stream), packed=True)


def fp8_quantize_blocks(w, stream=None):
    """bf16 [count, R, C] (or [R, C]) -> (E4M3 codes uint8 of the same shape,
    fp32 scales [count, ceil(R/128), ceil(C/128)] (or without count)), one
    scale per 128 x 128 block."""
    torch = _torch()
    w = _dev(w, "w", _bf16())
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    if w3.dim() != 3:
        raise ValueError("w must be [R, C] or [count, R, C]")
    cnt, R, Cc = w3.shape
    with _on(stream):
        codes = torch.empty((cnt, R, Cc), dtype=torch.uint8, device=w.device)
        scales = torch.empty((cnt, (R + 127) // 128, (Cc + 127) // 128), dtype=torch.float32,
                             device=w.device)
        _lib.check(_lib.load().moe_fp8_quantize_blocks(_ptr(w3), cnt, R, Cc, _ptr(codes),
                                                       _ptr(scales), _stream(stream)))
    return (codes[0], scales[0]) if squeeze else (codes, scales)


def fp8_quantize_rows(x, stream=None):
    """bf16 rows [n, C] (C % 128 == 0) -> (codes uint8 [n, C], fp32 scales
    [n, C/128]), one scale per 1 x 128 group."""
    torch = _torch()
    x = _dev(x, "x", _bf16())
    n, Cc = x.shape
    with _on(stream):
        codes = torch.empty((n, Cc), dtype=torch.uint8, device=x.device)
        scales = torch.empty((n, Cc // 128), dtype=torch.float32, device=x.device)
        _lib.check(_lib.load().moe_fp8_quantize_rows(_ptr(x), n, Cc, _ptr(codes), _ptr(scales),
                                                     _stream(stream)))
    return codes, scales


@dataclass
class Fp8ExpertWeights:
    """E4M3 expert weights with 128 x 128 block scales (torch tensors on the
    GPU); the router stays bf16."""
    w_router: object                   # [E, d] bf16
    w_gate: object                     # [E, h, d] uint8 codes
    s_gate: object                     # [E, h/128, d/128] fp32
    w_up: object
    s_up: object
    w_down: object                     # [E, d, h]
    s_down: object                     # [E, d/128, h/128]
    ws_gate: object = None             # [S, hs, d]
    ss_gate: object = None
    ws_up: object = None
    ss_up: object = None
    ws_down: object = None             # [S, d, hs]
    ss_down: object = None
    packed: bool = False               # w_gate, w_up as [E, d/128, h, 128] (pack_gateup)


def quantize_experts(weights: ExpertWeights, stream=None) -> Fp8ExpertWeights:
    """Quantise the expert weights of a bf16 layer with the library's block
    quantiser; the router is kept as it is."""
    if weights.packed:
        raise ValueError("quantize_experts takes row-major weights, not packed ones")
    q = {}
    for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        t = getattr(weights, name)
        codes, scales = (None, None) if t is None else fp8_quantize_blocks(t, stream)
        q[name] = codes
        q["s" + name[1:] if name.startswith("w_") else "ss" + name[2:]] = scales
    return Fp8ExpertWeights(w_router=weights.w_router, **q)


def _aux_tensors(aux, N, E, K, device):
    torch = _torch()
    shapes = {"logits": ((N, E), torch.float32), "topk_ids": ((N, K), torch.int32),
              "topk_weights": ((N, K), torch.float32), "alpha": ((N,), torch.float32),
              "margin": ((N,), torch.float32), "beta_out": ((E,), torch.float32),
              "quantile_out": ((E,), torch.float32), "counts_before": ((E,), torch.int32),
              "counts": ((E,), torch.int32), "offsets": ((E + 1,), torch.int32),
              "sorted_src": ((N * K,), torch.int32), "src_pos": ((N, K), torch.int32)}
    aux_t = {}
    for name in aux:
        if name not in shapes:
            raise ValueError(f"unknown aux output {name!r}")
        shp, dt = shapes[name]
        aux_t[name] = torch.empty(shp, dtype=dt, device=device)
    return aux_t


def _run_forward(fp8, x, wstruct, N, d, E, K, h, n_shared, h_shared, beta_in, recompute_bias,
                 key_bits, logit_offset, logits_in, aux, workspace, out, stream, extra_flags=0):
    torch = _torch()
    lib = _lib.load()
    beta_in = _dev(beta_in, "beta_in", torch.float32, (E,))
    logit_offset = _dev(logit_offset, "logit_offset", torch.float32, (E,))
    logits_in = _dev(logits_in, "logits_in", torch.float32, (N, E))
    flags = (MOE_RECOMPUTE_BIAS if recompute_bias else 0) | (MOE_KEY32 if key_bits == 32 else 0)
    p = _problem(N, d, E, K, h, n_shared, h_shared, flags | extra_flags, logit_offset, logits_in)
    ws_fn = lib.moe_forward_fp8_workspace_bytes if fp8 else lib.moe_forward_workspace_bytes
    fwd = lib.moe_forward_fp8 if fp8 else lib.moe_forward
    need = int(ws_fn(C.byref(p)))
    if need == 0:  # rejected shape: the call reports why
        _lib.check(fwd(C.byref(p), None, None, None, None, None, None, 0, None))
    with _on(stream):
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        y = out if out is not None else torch.empty((N, d), dtype=torch.bfloat16, device=x.device)
        _dev(y, "out", _bf16(), (N, d))
        aux_t = _aux_tensors(aux, N, E, K, x.device)
        a = MoeAux(*[_ptr(aux_t.get(f)) for f in AUX_FIELDS]) if aux_t else None
        _lib.check(fwd(C.byref(p), C.byref(wstruct), _ptr(x), _ptr(beta_in), _ptr(y),
                       C.byref(a) if a is not None else None, _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return (y, aux_t) if aux else y


def _bf16_weights(x, weights: ExpertWeights):
    x = _dev(x, "x", _bf16())
    N, d = x.shape
    wg = _dev(weights.w_gate, "w_gate", _bf16())
    if weights.packed:
        if wg.dim() != 4 or wg.shape[1] * 64 != d or wg.shape[3] != 64:
            raise ValueError("packed w_gate must be [E, d/64, h, 64]")
        E, _, h, _ = wg.shape
        _dev(weights.w_up, "w_up", _bf16(), (E, d // 64, h, 64))
    else:
        E, h, _ = wg.shape
        _dev(weights.w_up, "w_up", _bf16(), (E, h, d))
    _dev(weights.w_down, "w_down", _bf16(), (E, d, h))
    if weights.w_router is not None:
        _dev(weights.w_router, "w_router", _bf16(), (E, d))
    n_shared = 0 if weights.ws_gate is None else int(weights.ws_gate.shape[0])
    h_shared = h if n_shared == 0 else int(weights.ws_gate.shape[1])
    if n_shared:
        _dev(weights.ws_gate, "ws_gate", _bf16(), (n_shared, h_shared, d))
        _dev(weights.ws_up, "ws_up", _bf16(), (n_shared, h_shared, d))
        _dev(weights.ws_down, "ws_down", _bf16(), (n_shared, d, h_shared))
    w = MoeWeights(_ptr(weights.w_router), _ptr(wg), _ptr(weights.w_up),
                   _ptr(weights.w_down), _ptr(weights.ws_gate), _ptr(weights.ws_up),
                   _ptr(weights.ws_down))
    return x, w, N, d, E, h, n_shared, h_shared


def forward(x, weights: ExpertWeights, K: int, beta_in=None, recompute_bias: bool = False,
            key_bits: int = 16, logit_offset=None, logits_in=None, aux=(),
            workspace=None, out=None, stream=None, route_fused: bool = False):
    """MoE layer forward.  x: [N, d] bf16.  Returns y [N, d] bf16, or
    (y, dict) when ``aux`` names optional outputs (see moe_aux_t).
    ``route_fused`` selects the experts inside the router GEMM's epilogue
    (MOE_ROUTE_FUSED; same outputs as the default separate pass)."""
    x, w, N, d, E, h, n_shared, h_shared = _bf16_weights(x, weights)
    flags = (MOE_PACKED_GATEUP if weights.packed else 0) | \
        (MOE_ROUTE_FUSED if route_fused else 0)
    return _run_forward(False, x, w, N, d, E, K, h, n_shared, h_shared, beta_in, recompute_bias,
                        key_bits, logit_offset, logits_in, aux, workspace, out, stream, flags)


def forward_noalloc(x, weights: ExpertWeights, K: int, beta_in=None,
                    recompute_bias: bool = False, key_bits: int = 16, logit_offset=None,
                    logits_in=None, aux=(), out=None, stream=None,
                    route_fused: bool = False):
    """moe_forward_noalloc: the layer forward with the library's fixed
    per-GPU scratch array as its workspace (for callers that cannot allocate
    device memory; problems needing more than 64 MiB of workspace are
    rejected).  Arguments and results as forward(); pass ``out`` and aux
    tensors from the caller to keep the call itself free of allocations."""
    torch = _torch()
    lib = _lib.load()
    x, w, N, d, E, h, n_shared, h_shared = _bf16_weights(x, weights)
    beta_in = _dev(beta_in, "beta_in", torch.float32, (E,))
    logit_offset = _dev(logit_offset, "logit_offset", torch.float32, (E,))
    logits_in = _dev(logits_in, "logits_in", torch.float32, (N, E))
    flags = (MOE_RECOMPUTE_BIAS if recompute_bias else 0) | (MOE_KEY32 if key_bits == 32 else 0)
    flags |= MOE_PACKED_GATEUP if weights.packed else 0
    flags |= MOE_ROUTE_FUSED if route_fused else 0
    p = _problem(N, d, E, K, h, n_shared, h_shared, flags, logit_offset, logits_in)
    with _on(stream):
        y = out if out is not None else torch.empty((N, d), dtype=torch.bfloat16, device=x.device)
        _dev(y, "out", _bf16(), (N, d))
        aux_t = aux if isinstance(aux, dict) else _aux_tensors(aux, N, E, K, x.device)
        a = MoeAux(*[_ptr(aux_t.get(f)) for f in AUX_FIELDS]) if aux_t else None
        _lib.check(lib.moe_forward_noalloc(C.byref(p), C.byref(w), _ptr(x), _ptr(beta_in),
                                           _ptr(y), C.byref(a) if a is not None else None,
                                           _stream(stream)))
    return (y, aux_t) if aux else y


def forward_fp8(x, weights: Fp8ExpertWeights, K: int, beta_in=None,
                recompute_bias: bool = False, key_bits: int = 16, logit_offset=None,
                logits_in=None, aux=(), workspace=None, out=None, stream=None,
                route_fused: bool = False):
    """MoE layer forward with E4M3 experts (moe_forward_fp8).  x: [N, d] bf16;
    weights from ``quantize_experts`` or given codes and scales."""
    torch = _torch()
    x = _dev(x, "x", _bf16())
    N, d = x.shape
    u8, f32 = torch.uint8, torch.float32
    wg = _dev(weights.w_gate, "w_gate", u8)
    if weights.packed:
        if wg.dim() != 4 or wg.shape[1] * 128 != d or wg.shape[3] != 128:
            raise ValueError("packed w_gate codes must be [E, d/128, h, 128]")
        E, _, h, _ = wg.shape
        _dev(weights.w_up, "w_up", u8, (E, d // 128, h, 128))
    else:
        E, h, _ = wg.shape
        _dev(weights.w_up, "w_up", u8, (E, h, d))
    _dev(weights.w_down, "w_down", u8, (E, d, h))
    for name, shp in (("s_gate", (E, h // 128, d // 128)), ("s_up", (E, h // 128, d // 128)),
                      ("s_down", (E, d // 128, h // 128))):
        _dev(getattr(weights, name), name, f32, shp)
    if weights.w_router is not None:
        _dev(weights.w_router, "w_router", _bf16(), (E, d))
    n_shared = 0 if weights.ws_gate is None else int(weights.ws_gate.shape[0])
    hs = h if n_shared == 0 else int(weights.ws_gate.shape[1])
    if n_shared:
        _dev(weights.ws_gate, "ws_gate", u8, (n_shared, hs, d))
        _dev(weights.ws_up, "ws_up", u8, (n_shared, hs, d))
        _dev(weights.ws_down, "ws_down", u8, (n_shared, d, hs))
        for name, shp in (("ss_gate", (n_shared, hs // 128, d // 128)),
                          ("ss_up", (n_shared, hs // 128, d // 128)),
                          ("ss_down", (n_shared, d // 128, hs // 128))):
            _dev(getattr(weights, name), name, f32, shp)
    w = MoeFp8Weights(*[_ptr(getattr(weights, f)) for f, _ in MoeFp8Weights._fields_])
    flags = (MOE_PACKED_GATEUP if weights.packed else 0) | \
        (MOE_ROUTE_FUSED if route_fused else 0)
    return _run_forward(True, x, w, N, d, E, K, h, n_shared, hs, beta_in, recompute_bias,
                        key_bits, logit_offset, logits_in, aux, workspace, out, stream, flags)


def stage_timing(enable=True):
    """Per-stage HIP-event timing of forward(): True or 1 = every stage,
    2 = only the routed gate/up GEMM (two events per call), False or 0 = off.
    Clears what was recorded."""
    mode = int(enable) if not isinstance(enable, bool) else (1 if enable else 0)
    _lib.check(_lib.load().moe_stage_timing(mode))


def stage_times():
    """(dict stage -> summed ms since the last read, number of calls)."""
    lib = _lib.load()
    ms = (C.c_double * _lib.NUM_STAGES)()
    calls = C.c_int64(0)
    _lib.check(lib.moe_stage_times(ms, C.byref(calls)))
    return {lib.moe_stage_name(i).decode(): ms[i] for i in range(_lib.NUM_STAGES)}, calls.value
