"""Packed gate/up weights (moe_pack_gateup_weights, MOE_PACKED_GATEUP).

The packed layout moves values, not arithmetic: the pack must equal the
reshape it documents, and the layer with packed weights must give exactly
the bits of the layer with row-major weights, on the tile engine (with
288-row tiles), on the weight-streaming kernels of small batches, through
the no-allocation entry point, at the full prefill and skewed sizes, and
with E4M3 experts (codes packed as 16-bit words).
No oracle is needed for that: both sides are the same library on the same
inputs (the row-major layer itself is held to the oracle elsewhere)."""
from dataclasses import replace

import numpy as np
import pytest

from synth import CONFIGS, make_inputs, scaled
from tests.gpu_util import bf16_dev, dev, say, weights_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


def test_pack_layout(M):
    import torch
    rng = np.random.default_rng(7)
    w = rng.integers(0, 1 << 16, size=(3, 40, 192), dtype=np.uint16)
    say("pack layout", w.shape)
    out = M.pack_gateup_weights(bf16_dev(w))
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    want = w.reshape(3, 40, 3, 64).transpose(0, 2, 1, 3)
    assert got.shape == (3, 3, 40, 64)
    assert np.array_equal(got, want)


def _both(M, cfg, noalloc=False):
    import torch
    L = make_inputs(cfg)
    W = weights_dev(L)
    P = M.pack_gateup(W)
    assert P.packed and P.w_gate.shape == (cfg.E, cfg.d // 64, cfg.h, 64)
    x = bf16_dev(L.x)
    beta = dev(L.beta_in)
    off = None if L.logit_offset is None else dev(L.logit_offset)
    fwd = M.forward_noalloc if noalloc else M.forward
    out = []
    for weights in (W, P):
        y, A = fwd(x, weights, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                   logit_offset=off, aux=("topk_ids", "counts"))
        torch.cuda.synchronize()
        out.append((y.view(torch.int16).cpu().numpy(), A["topk_ids"].cpu().numpy(),
                    A["counts"].cpu().numpy()))
    return out


def _same(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("name,N,noalloc", [("prefill", 300, False), ("prefill", 3000, False),
                                            ("prefill", 17, False), ("decode", None, False),
                                            ("prefill", 300, True)])
def test_forward_packed_is_bit_identical(M, name, N, noalloc):
    cfg = CONFIGS[name] if N is None else scaled(CONFIGS[name], N)
    say("packed vs row-major", cfg.name, cfg.N, "noalloc" if noalloc else "")
    a, b = _both(M, cfg, noalloc)
    _same(a, b)


@pytest.mark.parametrize("N,K,offset,d,h", [(1100, 2, None, 192, 160),
                                            (2900, 3, "zipf1.2", 128, 96),
                                            (1100, 2, None, 576, 352)])
def test_forward_packed_segment_tails(M, N, K, offset, d, h):
    """Segments just above a multiple of 256 rows (288-row tiles), with two to
    nine k-blocks in the gate/up stage loop (the cases of the row-major tail
    test)."""
    cfg = replace(CONFIGS["toy"], name=f"packed_tail_{N}_{K}_{d}", N=N, d=d, E=8, K=K, h=h,
                  h_shared=h, offset=offset, recompute_bias=offset is None, dtype="bf16")
    say("packed tails", cfg.N, cfg.d, cfg.h)
    a, b = _both(M, cfg)
    c = a[2]
    assert np.any((c % 256 > 0) & (c % 256 <= 32) & (c > 256))
    _same(a, b)


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_forward_packed_full_size(M, name):
    cfg = CONFIGS[name]
    say("packed vs row-major, full size", name, cfg.N)
    a, b = _both(M, cfg)
    _same(a, b)


def test_quantize_experts_refuses_packed_weights(M):
    L = make_inputs(CONFIGS["toy"])
    P = replace(weights_dev(L), packed=True)
    with pytest.raises(ValueError):
        M.quantize_experts(P)


def _both_fp8(M, cfg):
    import torch
    L = make_inputs(cfg)
    Q = M.quantize_experts(weights_dev(L))
    P = M.pack_gateup(Q)
    assert P.packed and P.w_gate.shape == (cfg.E, cfg.d // 128, cfg.h, 128)
    x = bf16_dev(L.x)
    beta = dev(L.beta_in)
    off = None if L.logit_offset is None else dev(L.logit_offset)
    out = []
    for weights in (Q, P):
        y, A = M.forward_fp8(x, weights, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                             logit_offset=off, aux=("topk_ids", "counts"))
        torch.cuda.synchronize()
        out.append((y.view(torch.int16).cpu().numpy(), A["topk_ids"].cpu().numpy(),
                    A["counts"].cpu().numpy()))
    return out


@pytest.mark.parametrize("name,N", [("prefill", 300), ("prefill", 17), ("prefill", None)])
def test_forward_fp8_packed_is_bit_identical(M, name, N):
    """E4M3 codes packed as 16-bit words (128-code k-blocks): the tile
    engine, the weight-streaming kernel (17 tokens) and the full prefill."""
    cfg = CONFIGS[name] if N is None else scaled(CONFIGS[name], N)
    say("fp8 packed vs row-major", cfg.name, cfg.N)
    a, b = _both_fp8(M, cfg)
    _same(a, b)
