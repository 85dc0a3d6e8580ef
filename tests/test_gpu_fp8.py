"""GPU parity of the FP8 (E4M3) path against the oracle ("Kolibri 1 im
Detail", FP8 section: 128 x 128 weight blocks with fp32 scales, activations
quantised per 1 x 128 group, router in bf16).

* moe_fp8_quantize_rows / moe_fp8_quantize_blocks: codes and scales
  bit-exact (both sides divide in fp32 and round to nearest even).
* moe_forward_fp8 on a synthetic E4M3 checkpoint: routing, loads and grouping
  bit-exact and equal to moe_forward's for the same logits; the layer output
  within 2e-2 relative L2 of the oracle's FP8 layer (fp64 on the dequantised
  operands, H quantised from fp64), pooled, and within 5e-2 for every token
  on its own (the E4M3 MFMA's block sums move a few H codes by one step;
  see Y_REL_L2_FP8_TOKEN), on all tokens, or on 256 seeded tokens at the
  full size."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import CONFIGS, make_fp8_experts, make_inputs, scaled
from tests.gpu_util import (S_RTOL, Y_REL_L2_FP8_TOKEN, bf16_dev, bits_equal, check_logits,
                            check_output, dev, host, say, weights_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


def _bf16_bits(rng, shape, kind):
    x = rng.standard_normal(shape).astype(np.float32)
    if kind == "outliers":
        x[..., ::97] *= 1e4
    elif kind == "tiny":
        x *= 1e-30
    from synth import to_bf16_bits
    b = to_bf16_bits(x)
    return b


@pytest.mark.parametrize("n,cols,kind", [(1, 128, "normal"), (257, 512, "normal"),
                                          (300, 2560, "outliers"), (64, 384, "tiny")])
def test_quantize_rows_bitexact(M, n, cols, kind):
    say("fp8 quantize rows", n, cols, kind)
    rng = np.random.default_rng(n + cols)
    xb = _bf16_bits(rng, (n, cols), kind)
    if n > 3:
        xb[3, 128:256] = 0            # an all-zero group
        xb[2, 0:128] = 0x8000         # -0.0 everywhere
    q, s = M.fp8_quantize_rows(bf16_dev(xb))
    rq, rs = O.quantize_row_groups(O.bf16_to_f32(xb))
    assert np.array_equal(host(q), rq), "codes differ"
    assert bits_equal(host(s), rs), "scales differ"


@pytest.mark.parametrize("n,cols,shift", [(37, 384, 1), (64, 256, 3), (300, 2560, 0)])
def test_quantize_rows_alignment(M, n, cols, shift):
    """x shifted by `shift` 4-byte words off a 16-byte boundary takes the
    wave-per-group kernel, an aligned x the 16-lane one; both must give the
    oracle's codes and scales."""
    import torch
    say("fp8 quantize rows alignment", n, cols, shift)
    rng = np.random.default_rng(7 * n + cols + shift)
    xb = _bf16_bits(rng, (n, cols), "outliers")
    xb[n // 2, :128] = 0
    flat = bf16_dev(np.concatenate([np.zeros(2 * shift, np.uint16), xb.reshape(-1)]))
    x = flat[2 * shift:].view(n, cols)
    assert x.data_ptr() % 16 == (4 * shift) % 16
    q, s = M.fp8_quantize_rows(x)
    rq, rs = O.quantize_row_groups(O.bf16_to_f32(xb))
    assert np.array_equal(host(q), rq), "codes differ"
    assert bits_equal(host(s), rs), "scales differ"
    torch.cuda.synchronize()


@pytest.mark.parametrize("count,R,C", [(1, 128, 128), (3, 300, 200), (2, 256, 384), (1, 1, 1)])
def test_quantize_blocks_bitexact(M, count, R, C):
    say("fp8 quantize blocks", count, R, C)
    rng = np.random.default_rng(count * 1000 + R + C)
    wb = _bf16_bits(rng, (count, R, C), "normal")
    q, s = M.fp8_quantize_blocks(bf16_dev(wb))
    q, s = host(q), host(s)
    for i in range(count):
        rq, rs = O.quantize_weight_blocks(O.bf16_to_f32(wb[i]))
        assert np.array_equal(q[i], rq), f"codes of matrix {i} differ"
        assert bits_equal(s[i], rs), f"scales of matrix {i} differ"


def test_quantize_blocks_full_size_sampled(M):
    """The routed gate weights of the Kolibri-shaped layer, [384, 512, 2560]:
    a seeded sample of 24 blocks against the oracle."""
    L = make_inputs(CONFIGS["prefill"])
    say("fp8 quantize blocks full size")
    q, s = M.fp8_quantize_blocks(bf16_dev(L.w_gate))
    q, s = host(q), host(s)
    rng = np.random.default_rng(5)
    for _ in range(24):
        e, bi, bj = int(rng.integers(384)), int(rng.integers(4)), int(rng.integers(20))
        blk = O.bf16_to_f32(L.w_gate[e, bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128])
        rq, rs = O.quantize_weight_blocks(blk)
        assert np.array_equal(q[e, bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128], rq)
        assert bits_equal(s[e, bi, bj], rs[0, 0])


_CACHE = {}


def _case_inputs(cfg):
    key = (cfg.name, cfg.N, cfg.n_shared)
    if key not in _CACHE:
        if len(_CACHE) > 1:
            _CACHE.clear()
        _CACHE[key] = (make_inputs(cfg), make_fp8_experts(cfg))
    return _CACHE[key]


def _fp8_dev(M, L, q, shared):
    W = M.Fp8ExpertWeights(w_router=bf16_dev(L.w_router),
                           **{k: dev(v) for k, v in q.items() if not k.startswith(("ws", "ss"))})
    if shared:
        for k in ("ws_gate", "ss_gate", "ws_up", "ss_up", "ws_down", "ss_down"):
            setattr(W, k, dev(q[k]))
    return W


def run_fp8_case(M, cfg, sample=None, use_logits_in=False):
    import torch
    L, q = _case_inputs(cfg)
    shared = cfg.n_shared > 0
    say("fp8 forward", cfg.name, cfg.N, "shared", shared, "sample", sample,
        "logits_in", use_logits_in)
    x = bf16_dev(L.x)
    xf = O.bf16_to_f32(L.x)
    wr = O.bf16_to_f32(L.w_router)
    logits_in = O.router_logits(xf, wr, L.logit_offset) if use_logits_in else None
    kw = dict(beta_in=dev(L.beta_in), recompute_bias=cfg.recompute_bias,
              logit_offset=None if use_logits_in else dev(L.logit_offset),
              logits_in=dev(logits_in), aux=M.AUX_FIELDS)
    y, A = M.forward_fp8(x, _fp8_dev(M, L, q, shared), cfg.K, **kw)
    torch.cuda.synchronize()
    y = O.bf16_to_f32(host(y))
    A = {k: host(v) for k, v in A.items()}
    # the same routing as the bf16 layer on the same logits
    _, Ab = M.forward(x, weights_dev(L), cfg.K, **kw)
    torch.cuda.synchronize()
    keys = ["logits", "topk_ids", "topk_weights", "alpha", "margin", "counts", "offsets",
            "sorted_src", "src_pos"] + (["beta_out", "quantile_out"] if cfg.recompute_bias else [])
    for k in keys:
        assert bits_equal(A[k], host(Ab[k])), f"{k} differs from the bf16 layer's"
    N = cfg.N
    rows = np.arange(N) if sample is None else np.sort(
        np.random.default_rng(cfg.seed).choice(N, sample, replace=False))
    if not use_logits_in:
        check_logits(A["logits"][rows], O.router_logits(xf[rows], wr, L.logit_offset))
    ref = O.moe_layer(x=xf, w_router=None, w_gate=None, w_up=None, w_down=None, ws_gate=None,
                      ws_up=None, ws_down=None, beta_in=L.beta_in, K=cfg.K,
                      recompute_bias=cfg.recompute_bias, logits_in=A["logits"],
                      compute_output=False)
    assert np.array_equal(A["topk_ids"], ref["topk_ids"])
    assert np.array_equal(A["sorted_src"], ref["sorted_src"])
    S_err = np.max(np.abs(A["topk_weights"].astype(np.float64) - ref["topk_weights"])
                   / np.abs(ref["topk_weights"]))
    assert S_err <= S_RTOL, S_err
    qo = dict(q)
    if not shared:
        for k in ("ws_gate", "ss_gate", "ws_up", "ss_up", "ws_down", "ss_down"):
            qo[k] = q[k][:0]
    yref = O.moe_combine_fp8(xf, qo, ref["topk_ids"], ref["topk_weights"], token_subset=rows)
    err, _ = check_output(y[rows], yref, f"fp8 forward {cfg.name}", Y_REL_L2_FP8_TOKEN)
    return err


SMALL = [("origin", 300), ("decode", 64), ("prefill", 65), ("prefill", 1), ("skewed", 600)]


@pytest.mark.parametrize("name,N", SMALL)
def test_forward_fp8_small(M, name, N):
    cfg = scaled(CONFIGS[name], N)
    run_fp8_case(M, cfg)


def test_forward_fp8_logits_in_and_no_shared(M):
    cfg = scaled(CONFIGS["origin"], 520)
    run_fp8_case(M, cfg, use_logits_in=True)
    run_fp8_case(M, replace(cfg, n_shared=0), sample=64)


def test_forward_fp8_small_batch_concentrated(M):
    """The weight-streaming E4M3 GEMMs with every token on experts 0 and 1
    (64 rows: four passes), and a batch of 17 tokens."""
    base = CONFIGS["toy"]
    for N in (64, 17):
        cfg = replace(base, name=f"fp8_small_collapse_{N}", N=N, d=256, E=8, K=2, h=256,
                      h_shared=128, recompute_bias=False, dtype="bf16")
        run_fp8_case(M, cfg)


# Loads just above a multiple of 256 rows: the last m-tile of a segment
# holds up to 288 rows (the extra-rows tile), a longer remainder gets a tile
# of its own.  Loads (oracle):
#  a) 282 251 286 280 286 257 271 287       - 288-row tiles, one 251
#  b) 533 533 508 531 527 512 530 526       - 256 + extra-rows tiles, one 252
#  c) 2891 2687 1817 719 393 108 59 26      - long segments, tails of both kinds
#  d) 1481 1221 799 452 250 132 91 74       - as c, d = 256 and h = 128
#  e) N = 900, d = h = 384: three 128-k stages (first, middle, last, no
#     steady state) in both products
# The other cases give 1 and 2 stages; the full-size prefill test 20 and 4.
@pytest.mark.parametrize("N,K,offset,d,h", [(1100, 2, None, 256, 256), (2100, 2, None, 128, 128),
                                            (2900, 3, "zipf1.2", 128, 256),
                                            (1500, 3, "zipf1.2", 256, 128),
                                            (900, 2, None, 384, 384)])
def test_forward_fp8_segment_tails(M, N, K, offset, d, h):
    cfg = replace(CONFIGS["toy"], name=f"fp8_tail_{N}_{K}_{d}_{h}", N=N, d=d, E=8, K=K, h=h,
                  h_shared=h, offset=offset, recompute_bias=offset is None, dtype="bf16")
    run_fp8_case(M, cfg)


def test_forward_fp8_prefill_full_sampled(M):
    """The Kolibri-shaped prefill batch (N=16384, E=384, K=6, d=2560, h=512),
    256 sampled tokens."""
    run_fp8_case(M, CONFIGS["prefill"], sample=256)


def test_forward_fp8_rejects_unaligned_width(M):
    cfg = CONFIGS["toy"]  # d = 64
    L = make_inputs(cfg)
    W = M.Fp8ExpertWeights(w_router=bf16_dev(L.w_router), w_gate=dev(np.zeros((4, 32, 64), np.uint8)),
                           s_gate=dev(np.zeros((4, 0, 0), np.float32)),
                           w_up=dev(np.zeros((4, 32, 64), np.uint8)),
                           s_up=dev(np.zeros((4, 0, 0), np.float32)),
                           w_down=dev(np.zeros((4, 64, 32), np.uint8)),
                           s_down=dev(np.zeros((4, 0, 0), np.float32)))
    with pytest.raises(M.MoeError, match="UNSUPPORTED_SHAPE"):
        M.forward_fp8(bf16_dev(L.x), W, cfg.K)


def test_fp8_mfma_block_sum_precision():
    """The assumption behind Y_REL_L2_FP8_TOKEN: gfx950's E4M3 MFMA sums the
    128 products of a block with an error of at most 2^-12 of their absolute
    sum (and not exactly: one product of 448 among 127 of 2^-9 loses part of
    the small ones).  Measured by tests/probes/fp8_block_sum (built by the
    package build)."""
    import json
    import os
    import subprocess
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = os.path.join(os.path.dirname(__file__), "probes", "fp8_block_sum")
    assert os.path.exists(exe), "tests/probes/fp8_block_sum is not built (run the package build)"
    say("fp8 MFMA block-sum precision probe")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    m = json.loads(r.stdout.strip().splitlines()[-1])
    say("fp8 MFMA block sum", m)
    assert 0.0 < m["max_err_over_abs_sum"] <= 2.0 ** -12, m
    assert m["one_large_block"] != m["exact"]
