"""GPU tests of the expert selection fused into the router GEMM.

Above 64 tokens, when the layer computes its own logits, every column tile of
the router product can also write, for each of its rows, its K + 1 first
entries in the selection order (biased score descending, expert ascending),
and a small merge ranks the union (MOE_ROUTE_FUSED, route_fused=True); by
default the layer selects in a pass of its own over the stored logits.  The two must
agree bit for bit in every routing output, the grouping and the layer
output; against the oracle (given the GPU's logits) the fused selection is
bit-exact, including rows whose biased scores tie exactly across many
experts, where a tile's candidate list overflows and the tile pops its
entries one at a time ("Kolibri Pre-Training from Scratch" §6.1 routing
equations, §7.1 token bias)."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import CONFIGS, make_inputs, scaled
from tests.gpu_util import S_RTOL, bf16_dev, bits_equal, dev, host, say, weights_dev

pytestmark = pytest.mark.gpu

ROUTING = ("logits", "topk_ids", "topk_weights", "alpha", "margin", "counts_before", "counts",
           "offsets", "sorted_src", "src_pos", "beta_out", "quantile_out")


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


def _both(M, L, cfg, W=None, beta=None, noalloc=False):
    import torch
    W = W or weights_dev(L)
    x = bf16_dev(L.x)
    b = dev(L.beta_in if beta is None else beta)
    fwd = M.forward_noalloc if noalloc else M.forward
    out = []
    for fused in (True, False):
        y, A = fwd(x, W, cfg.K, beta_in=b, recompute_bias=cfg.recompute_bias,
                   logit_offset=dev(L.logit_offset), aux=M.AUX_FIELDS, route_fused=fused)
        torch.cuda.synchronize()
        out.append((host(y), {k: host(v) for k, v in A.items()}))
    return out


def _same(fused, sep, cfg):
    """Bit-identical routing and output.  One exception: for E % 4 != 0 the
    separate pass runs the one-wave route kernel, whose weights come from an
    fp64 sigmoid, while the merge (like the 16-lane route kernel) uses the
    fp32 one; both are within 1e-6 of sigma(z), so there the weights and the
    output are compared within that bound."""
    (yf, Af), (ys, As) = fused, sep
    exact_w = cfg.E % 4 == 0
    for k in ROUTING:
        if not cfg.recompute_bias and k in ("beta_out", "quantile_out"):
            continue
        if k == "topk_weights" and not exact_w:
            rel = np.abs(Af[k].astype(np.float64) - As[k]) / np.abs(As[k].astype(np.float64))
            assert rel.max() <= S_RTOL, rel.max()
            continue
        assert bits_equal(Af[k], As[k]), k
    if exact_w:
        assert np.array_equal(yf, ys)
    else:
        a, b = O.bf16_to_f32(yf), O.bf16_to_f32(ys)
        assert np.linalg.norm(a - b) <= 1e-4 * np.linalg.norm(b)


def _oracle_routing(A, beta, cfg):
    """Selection of the GPU's logits by the oracle, bit-exact."""
    Zg = A["logits"]
    ids, alpha, margin = O.route(Zg, beta, cfg.K)
    if cfg.recompute_bias:
        # the token bias and the loads come from the first pass with beta_in
        assert bits_equal(A["alpha"], alpha)
        assert np.array_equal(A["counts_before"], np.bincount(ids.ravel(), minlength=cfg.E))
    else:
        assert np.array_equal(A["topk_ids"], ids)
        assert bits_equal(A["alpha"], alpha)
        assert bits_equal(A["margin"], margin)


CASES = [
    ("prefill", 500, None, True),    # two column tiles (256 + 128 columns), bias update
    ("prefill", 500, None, False),   # the merge gives the final routing
    ("origin", 300, None, False),    # E = 128: narrow router tiles, K = 8
    ("skewed", 1000, None, True),    # Zipf logit offsets
    ("prefill", 300, 259, False),    # E % 4 != 0; the last tile holds 3 columns < K + 1
    ("prefill", 300, 130, True),     # E % 4 != 0, one tile
    ("prefill", 257, 383, False),    # a single row in the last m-tile
]


@pytest.mark.parametrize("name,N,E,recompute", CASES)
def test_fused_selection_matches_separate_pass(M, name, N, E, recompute):
    cfg = replace(scaled(CONFIGS[name], N), recompute_bias=recompute)
    if E is not None:
        cfg = replace(cfg, E=E, name=f"{name}_E{E}")
    say("fused vs separate", cfg.name, N, cfg.E, "recompute", recompute)
    L = make_inputs(cfg)
    fused, sep = _both(M, L, cfg)
    _same(fused, sep, cfg)
    _oracle_routing(fused[1], L.beta_in, cfg)


def test_fused_selection_no_alloc_entry_point(M):
    """moe_forward_noalloc runs the router inside the launch that also does
    the shared expert's gate/up (one stream); its fused selection must agree
    with its separate pass and with the oracle."""
    cfg = scaled(CONFIGS["prefill"], 700)
    say("fused vs separate, no-allocation entry point")
    L = make_inputs(cfg)
    fused, sep = _both(M, L, cfg, noalloc=True)
    _same(fused, sep, cfg)
    _oracle_routing(fused[1], L.beta_in, cfg)


@pytest.mark.parametrize("groups,K,zero_bias", [(1, 6, True), (4, 6, True), (24, 8, True),
                                                (48, 6, False)])
def test_fused_selection_exact_ties(M, groups, K, zero_bias):
    """Router rows repeated so that each token's logits take only `groups`
    distinct values, each shared by 384 / groups experts (groups = 1: every
    score of a row ties; 4: 96-way ties, more than a tile's candidate list
    holds).  With a zero bias (or a bias constant over each group) the
    scores tie exactly; the order among tied scores is by expert."""
    base = replace(scaled(CONFIGS["prefill"], 300), K=K, recompute_bias=False,
                   name=f"ties_{groups}_{K}")
    L = make_inputs(base)
    E = base.E
    reps = E // groups
    w = L.w_router[np.arange(E) // reps]
    L = replace(L, w_router=np.ascontiguousarray(w))
    if zero_bias:
        beta = np.zeros(E, np.float32)
    else:
        beta = np.repeat(np.random.default_rng(7).normal(0, 0.1, groups).astype(np.float32), reps)
    say("ties", groups, "K", K, "zero bias", zero_bias)
    fused, sep = _both(M, L, base, beta=beta)
    _same(fused, sep, base)
    Zg = fused[1]["logits"]
    distinct = max(len(np.unique(r)) for r in Zg[:16])
    say("distinct logits per row (first 16 rows, max)", distinct)
    _oracle_routing(fused[1], beta, base)
