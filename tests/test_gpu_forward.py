"""GPU parity of moe_forward (the whole layer) against the oracle.

For every case: router logits within 1e-4 relative; given the GPU's logits,
the selections, token biases, margins, expert biases, quantiles, loads,
offsets and the permutation bit-exact; sigmoid weights within 1e-6; the
layer output within 2e-2 relative L2, pooled and for every token on its own
(on all tokens, or on a seeded sample of tokens at the full sizes).  Where
asked, a free-running comparison (the oracle on its own logits and its own
bias update): selections may differ only where the oracle's margin is below
the near-tie threshold plus twice the largest logit and bias differences,
and the output is within 2e-2 relative L2 of the oracle's own output."""
from dataclasses import replace

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import CONFIGS, make_inputs, scaled
from tests.gpu_util import (S_RTOL, Y_REL_L2, bf16_dev, bits_equal, check_logits, check_output,
                            dev, free_running_mismatch, host, oracle_weights, rel_l2, say,
                            weights_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


_CACHE = {}


def _inputs(cfg):
    key = (cfg.name, cfg.N, cfg.n_shared)
    if key not in _CACHE:
        if len(_CACHE) > 2:
            _CACHE.clear()
        _CACHE[key] = make_inputs(cfg)
    return _CACHE[key]


def run_case(M, cfg, key_bits=16, sample=None, free_running=False, use_logits_in=False):
    L = _inputs(cfg)
    say(cfg.name, cfg.N, "key_bits", key_bits, "sample", sample, "logits_in", use_logits_in)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    xf = O.bf16_to_f32(L.x)
    wr = O.bf16_to_f32(L.w_router)
    logits_in = None
    if use_logits_in:
        logits_in = O.router_logits(xf, wr, L.logit_offset)
    y, A = M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=cfg.recompute_bias,
                     key_bits=key_bits,
                     logit_offset=None if use_logits_in else dev(L.logit_offset),
                     logits_in=dev(logits_in), aux=M.AUX_FIELDS)
    import torch
    torch.cuda.synchronize()
    y = O.bf16_to_f32(host(y))
    A = {k: host(v) for k, v in A.items()}
    N = cfg.N
    rows = np.arange(N) if sample is None else np.sort(
        np.random.default_rng(cfg.seed).choice(N, sample, replace=False))

    # router logits
    Zg = A["logits"]
    if use_logits_in:
        assert bits_equal(Zg, logits_in)
    else:
        zref = O.router_logits(xf[rows], wr, L.logit_offset)
        check_logits(Zg[rows], zref)

    # selection, bias update and grouping on identical logits: bit-exact
    ref = O.moe_layer(x=xf, w_router=None, **oracle_weights(L), beta_in=L.beta_in, K=cfg.K,
                      recompute_bias=cfg.recompute_bias, key_bits=key_bits, logits_in=Zg,
                      compute_output=False)
    assert np.array_equal(A["topk_ids"], ref["topk_ids"])
    assert bits_equal(A["alpha"], ref["alpha"])
    assert bits_equal(A["margin"], ref["margin"])
    assert np.array_equal(A["counts_before"], ref["counts_before"])
    assert np.array_equal(A["counts"], ref["counts"])
    assert np.array_equal(A["offsets"], ref["offsets"])
    assert np.array_equal(A["sorted_src"], ref["sorted_src"])
    assert np.array_equal(A["src_pos"], ref["src_pos"])
    if cfg.recompute_bias:
        assert bits_equal(A["beta_out"], ref["beta_out"])
        assert bits_equal(A["quantile_out"], ref["quantile"])
    S_err = np.max(np.abs(A["topk_weights"].astype(np.float64) - ref["topk_weights"])
                   / np.abs(ref["topk_weights"]))
    assert S_err <= S_RTOL, S_err

    # experts and combine, (ii) the GPU's routing forced into the oracle (= the
    # oracle's on Zg): pooled and per-token relative L2 on the sampled tokens
    yref = O.moe_combine(xf, **oracle_weights(L), ids=ref["topk_ids"], S=ref["topk_weights"],
                         token_subset=rows)
    check_output(y[rows], yref, f"{cfg.name} forced ids")

    if free_running:
        # (i) the oracle on its own logits and its own bias update
        own = O.moe_layer(x=xf, w_router=wr, **oracle_weights(L), beta_in=L.beta_in, K=cfg.K,
                          recompute_bias=cfg.recompute_bias, key_bits=key_bits,
                          logit_offset=L.logit_offset, compute_output=False)
        fr = free_running_mismatch(own, A, Zg)
        diff = fr.pop("diff")
        say(cfg.name, "free-running", fr)
        assert fr["beyond_bound"] == 0, fr
        yown = O.moe_combine(xf, **oracle_weights(L), ids=own["topk_ids"],
                             S=own["topk_weights"], token_subset=rows)
        pooled = rel_l2(y[rows], yown)
        say(cfg.name, "free-running rel L2", f"{pooled:.3e}")
        assert pooled <= Y_REL_L2, pooled
        same = ~diff[rows]
        if same.any():
            check_output(y[rows][same], yown[same], f"{cfg.name} free-running, same selection")
    return y, A


# Small cases: several tiles and a ragged tail, oracle over every token.
SMALL = [
    ("toy", None),
    ("origin", 300),
    ("prefill", 500),
    ("decode", 64),
    ("prefill", 65),   # first size on the tile engine and the side stream
    ("skewed", 1000),
    ("prefill", 3000),  # 18,000 pairs: the count table (9 rows), filled by the final routing pass
]


@pytest.mark.parametrize("name,N", SMALL)
def test_forward_small(M, name, N):
    cfg = CONFIGS[name] if N is None else scaled(CONFIGS[name], N)
    if name == "toy":
        # the toy layer routes every token to experts 0 and 1 before the update
        _, A = run_case(M, cfg)
        assert A["counts_before"].tolist() == [4, 4, 0, 0]
    else:
        run_case(M, cfg, free_running=True)


def test_forward_key32_and_logits_in(M):
    cfg = scaled(CONFIGS["skewed"], 700)
    run_case(M, cfg, key_bits=32)
    run_case(M, cfg, use_logits_in=True)


def test_forward_tiny_shapes(M):
    base = CONFIGS["toy"]
    for N, E, K in ((1, 9, 8), (3, 5, 1), (130, 16, 4)):
        cfg = replace(base, name=f"tiny_{N}_{E}_{K}", N=N, E=E, K=K, offset=None,
                      recompute_bias=(N > 1), dtype="bf16")
        run_case(M, cfg)


def test_forward_small_batch_concentrated(M):
    """Batches of at most 64 tokens take the weight-streaming expert GEMMs.
    With the collapse offset every token picks experts 0 and 1, so those
    tiles hold all 64 rows (four 16-row passes); h = 96 leaves a half k-set
    in the down projection and a partly empty block of hidden columns."""
    base = CONFIGS["toy"]
    for N in (64, 17):
        cfg = replace(base, name=f"small_collapse_{N}", N=N, d=256, E=8, K=2, h=96,
                      h_shared=96, recompute_bias=False, dtype="bf16")
        _, A = run_case(M, cfg)
        assert A["counts"][0] == N and A["counts"][1] == N


# Expert loads just above a multiple of 256 rows: the last m-tile of such a
# segment holds up to 288 rows (the extra-rows tile), larger remainders get
# a tile of their own.  The loads of each case (from the oracle's routing):
#  a) 286 284 284 276 262 256 278 274      - single 288-row tiles, one 256
#  b) 542 520 502 530 534 508 507 557      - 256 + extra-rows tiles, 256+256+45
#  c) 2891 2687 1817 719 393 108 59 26     - many tiles, a 281-row last tile
#  d) 251 280 285 278 277 274 277 278
# d and h set the k loops (gate/up, down): 192/160 -> 3/3 stages with a 32-k
# tail in down, 64/160 -> 1/3, 128/96 -> 2/2 (b_rows = 128 leaves whole
# waves of the down tile without columns), 576/352 -> 9/6 (steady state).
@pytest.mark.parametrize("N,K,offset,d,h", [(1100, 2, None, 192, 160), (2100, 2, None, 64, 160),
                                            (2900, 3, "zipf1.2", 128, 96),
                                            (1100, 2, None, 576, 352)])
def test_forward_tail_rows(M, N, K, offset, d, h):
    cfg = replace(CONFIGS["toy"], name=f"tail_{N}_{K}_{d}", N=N, d=d, E=8, K=K, h=h,
                  h_shared=h, offset=offset, recompute_bias=offset is None, dtype="bf16")
    _, A = run_case(M, cfg)
    assert np.any((A["counts"] % 256 > 0) & (A["counts"] % 256 <= 32) & (A["counts"] > 256))


@pytest.mark.parametrize("E", [200, 136, 100])
def test_forward_router_column_tails(M, E):
    """The router GEMM alone (shared expert on the side stream) with column
    counts that fill no tile: E = 200 and 136 take one 256-wide tile whose
    waves own 64 columns each (E = 200: the last wave 8 live columns;
    E = 136: one wave 8, the last none); E = 100 takes the 256 x 128 tile,
    whose last 32-column block holds 4 live columns.  Logits, routing and
    output against the oracle."""
    cfg = replace(scaled(CONFIGS["prefill"], 700), E=E, name=f"router_tail_{E}")
    run_case(M, cfg)


@pytest.mark.parametrize("N,hs", [(50, None), (37, 1024)])
def test_forward_decode_shared_expert_paths(M, N, hs):
    """At most 64 tokens: with h_shared == h the shared expert runs as 16-row
    tiles (the last one ragged) inside the weight-streaming products; with a
    wider shared expert it keeps its own split-K products on the side
    stream.  Every token against the oracle."""
    base = scaled(CONFIGS["decode"], N)
    cfg = replace(base, h_shared=hs or base.h, name=f"decode_shared_{N}_{hs}")
    run_case(M, cfg, free_running=True)


def test_forward_without_shared_expert(M):
    cfg = replace(scaled(CONFIGS["prefill"], 200), n_shared=0, name="noshared")
    run_case(M, cfg)


def test_forward_zero_routed_weights_gives_shared_only(M):
    cfg = scaled(CONFIGS["prefill"], 256)
    L = _inputs(cfg)
    say("zero routed weights")
    W = weights_dev(L)
    W.w_down = W.w_down * 0
    y = O.bf16_to_f32(host(M.forward(bf16_dev(L.x), W, cfg.K, beta_in=dev(L.beta_in))))
    xf = O.bf16_to_f32(L.x)
    sh = O.swiglu(xf, O.bf16_to_f32(L.ws_gate[0]), O.bf16_to_f32(L.ws_up[0]),
                  O.bf16_to_f32(L.ws_down[0]))
    assert rel_l2(y, sh) <= Y_REL_L2


def test_forward_deterministic(M):
    cfg = scaled(CONFIGS["prefill"], 2048)
    L = _inputs(cfg)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    say("determinism")
    a = host(M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True))
    b = host(M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True))
    assert np.array_equal(a, b)


# Full sizes of the workloads (the benchmark's launch configuration).
@pytest.mark.parametrize("name,sample,free", [("origin", 256, True), ("decode", None, True),
                                              ("prefill", 256, True), ("skewed", 256, True)])
def test_forward_full_size(M, name, sample, free):
    run_case(M, CONFIGS[name], sample=sample, free_running=free)


def test_stage_timing_records_every_stage(M):
    cfg = scaled(CONFIGS["prefill"], 1024)
    L = _inputs(cfg)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    say("stage timing")
    M.stage_timing(True)
    for _ in range(3):
        M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True)
    times, calls = M.stage_times()
    M.stage_timing(False)
    assert calls == 3
    assert all(v > 0 for v in times.values()), times
    # nothing recorded while disabled
    M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True)
    M.stage_timing(True)
    times, calls = M.stage_times()
    M.stage_timing(False)
    assert calls == 0
    # light mode: only the routed gate/up GEMM is timed
    M.stage_timing(2)
    for _ in range(2):
        M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True)
    times, calls = M.stage_times()
    M.stage_timing(False)
    assert calls == 2 and times["gate_up"] > 0
    assert all(v == 0 for k, v in times.items() if k != "gate_up"), times
    # light mode also on the weight-streaming path (N <= 64) and with E4M3
    # experts
    small = scaled(CONFIGS["prefill"], 64)
    Ls = _inputs(small)
    Wq = M.quantize_experts(W)
    for run in (lambda: M.forward(bf16_dev(Ls.x), weights_dev(Ls), small.K,
                                  beta_in=dev(Ls.beta_in), recompute_bias=True),
                lambda: M.forward_fp8(x, Wq, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True)):
        M.stage_timing(2)
        run()
        times, calls = M.stage_times()
        M.stage_timing(False)
        assert calls == 1 and times["gate_up"] > 0, times
    # and full mode again after it times every stage
    M.stage_timing(True)
    M.forward(x, W, cfg.K, beta_in=dev(L.beta_in), recompute_bias=True)
    times, calls = M.stage_times()
    M.stage_timing(False)
    assert calls == 1 and all(v > 0 for v in times.values()), times
