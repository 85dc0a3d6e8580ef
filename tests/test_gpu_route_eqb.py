"""GPU parity of moe_route and moe_eqb_bias against the oracle on identical
logits: selections, token biases, margins, quantiles and biases bit-exact;
sigmoid weights within 1e-6 relative."""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import make_bias, make_logits
from tests.gpu_util import S_RTOL, bits_equal, dev, host, say

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden", "toy_routing_eqb.json")


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


def _route_case(M, Z, beta, K):
    ids, S, alpha, margin = M.route(dev(Z), K, dev(beta))
    ids, S, alpha, margin = host(ids), host(S), host(alpha), host(margin)
    ri, ra, rm = O.route(Z, beta, K)
    rs = O.mixture_weights(Z, ri)
    assert np.array_equal(ids, ri), f"ids differ in {np.sum(np.any(ids != ri, axis=1))} rows"
    assert bits_equal(alpha, ra)
    assert bits_equal(margin, rm)
    err = np.max(np.abs(S.astype(np.float64) - rs) / np.abs(rs))
    assert err <= S_RTOL, err
    return ids


ROUTE_CASES = [
    # seed, N, E, K, tie_fraction, with_beta
    (101, 1, 5, 2, 0.0, False),
    (102, 7, 9, 8, 0.5, True),
    (103, 1000, 384, 6, 0.0, True),
    (104, 1000, 384, 6, 0.8, True),
    (105, 4096, 128, 8, 0.0, True),
    (106, 333, 64, 8, 0.3, True),
    (107, 257, 100, 3, 0.9, True),
    (108, 129, 383, 1, 0.2, False),
    (109, 64, 65, 4, 0.0, True),
    (110, 301, 128, 1, 0.3, True),
    (111, 299, 192, 7, 0.6, True),
]


@pytest.mark.parametrize("seed,N,E,K,ties,with_beta", ROUTE_CASES)
def test_route_parity(M, seed, N, E, K, ties, with_beta):
    say("route", seed, N, E, K, ties, with_beta)
    Z = make_logits(seed, N, E, 1.0, tie_fraction=ties)
    beta = make_bias(seed + 1, E, 0.3 if ties == 0 else 0.25) if with_beta else None
    if beta is not None and ties > 0:
        beta = (np.round(beta * 8) / 8).astype(np.float32)
    _route_case(M, Z, beta, K)


@pytest.mark.parametrize("E,K", [(64, 6), (68, 8), (100, 6), (128, 8), (384, 6)])
def test_route_tied_candidates(M, E, K):
    """Rows whose largest scores tie across many experts, so that the
    candidate list of a row (scores at or above the bound from the lane
    maxima) holds K, K+1, 63, 64, 65 or all E entries: beyond 64 a wave
    selects by popping the row maximum instead, and the rows of that wave
    that did not overflow must come out the same.  Also whole rows of one
    value and rows of signed zeros."""
    say("route tied candidates", E, K)
    rng = np.random.default_rng(230 + E)
    counts = [K, K + 1, 63, 64, 65, E]
    N = 4 * len(counts) + 9
    Z = rng.standard_normal((N, E)).astype(np.float32)
    for t in range(N):
        kind = t % 8
        if kind < len(counts):
            m = min(counts[kind], E)
            Z[t, rng.choice(E, m, replace=False)] = 4.0
        elif kind == 6:
            Z[t] = 0.25
        else:
            Z[t] = np.where(rng.random(E) < 0.5, np.float32(-0.0), np.float32(0.0))
    _route_case(M, Z, None, K)
    beta = (np.round(make_bias(231 + E, E, 0.25) * 8) / 8).astype(np.float32)
    _route_case(M, Z - beta, beta, K)


def test_route_parity_full_size_skewed(M):
    """N=65536, E=384, K=6 at the launch size of the benchmark."""
    say("route full 65536x384")
    Z = make_logits(111, 65536, 384, 0.6)
    beta = make_bias(112, 384, 0.1)
    _route_case(M, Z, beta, 6)


def test_route_printed_toy_logits(M):
    g = json.load(open(GOLD))
    Z = np.array(g["logits"]["Z"], np.float32)
    say("route toy")
    ids = _route_case(M, Z, None, 2)
    assert [sorted(r) for r in ids.tolist()] == g["logits"]["top2_with_beta0"]
    beta = np.array(g["centring"]["beta"], np.float32)
    ids = _route_case(M, Z, beta, 2)
    assert [sorted(r) for r in ids.tolist()] == g["reroute"]["top2_sets"]


def test_route_is_deterministic(M):
    say("route determinism")
    Z = make_logits(121, 5000, 384, 1.0, tie_fraction=0.5)
    a = [host(t) for t in M.route(dev(Z), 6, None)]
    b = [host(t) for t in M.route(dev(Z), 6, None)]
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


# ---------------------------------------------------------------- EQB
def _eqb_case(M, Z, beta_in, K, key_bits, give_alpha):
    _, alpha, _ = O.route(Z, beta_in, K)
    bo, q = M.eqb_bias(dev(Z), K, beta_in=dev(beta_in),
                       alpha=dev(alpha) if give_alpha else None, key_bits=key_bits)
    bo, q = host(bo), host(q)
    rb, rq, _ = O.eqb_expert_bias(Z, alpha, K, key_bits)
    assert bits_equal(q, rq), f"quantiles differ at {np.nonzero(q != rq)[0][:10]}"
    assert bits_equal(bo, rb)
    return bo, q


EQB_CASES = [
    # seed, N, E, K, ties
    (201, 40, 8, 2, 0.0),
    (202, 1000, 384, 6, 0.0),
    (203, 1000, 384, 6, 0.9),
    (204, 4096, 128, 8, 0.3),
    (205, 777, 100, 5, 0.5),
    (206, 64, 384, 6, 0.0),
]


@pytest.mark.parametrize("key_bits", [16, 32])
@pytest.mark.parametrize("give_alpha", [True, False])
@pytest.mark.parametrize("seed,N,E,K,ties", EQB_CASES)
def test_eqb_parity(M, seed, N, E, K, ties, key_bits, give_alpha):
    say("eqb", seed, N, E, K, ties, key_bits, give_alpha)
    Z = make_logits(seed, N, E, 1.0, tie_fraction=ties)
    beta = make_bias(seed + 1, E, 0.1)
    _eqb_case(M, Z, beta, K, key_bits, give_alpha)


@pytest.mark.parametrize("key_bits", [16, 32])
def test_eqb_parity_full_size(M, key_bits):
    """N=65536, E=384, K=6 (r = 1024), with a Zipf-like skew in the logits."""
    say("eqb full", key_bits)
    Z = make_logits(211, 65536, 384, 0.6)
    p = np.arange(1, 385, dtype=np.float64) ** -1.2
    Z = (Z + (0.5 * np.log(p / p.sum())).astype(np.float32)[None, :]).astype(np.float32)
    beta = make_bias(212, 384, 0.1)
    bo, q = _eqb_case(M, Z, beta, 6, key_bits, give_alpha=False)
    # exactness invariant on the keys: #{u > Q} <= r < #{u >= Q}
    _, alpha, _ = O.route(Z, beta, 6)
    u = O.eqb_keys_values((Z + alpha[:, None]).astype(np.float32), key_bits)
    r = 65536 * 6 // 384
    assert ((u > q[None, :]).sum(0) <= r).all() and ((u >= q[None, :]).sum(0) > r).all()


def _signed_zero_logits(seed, N, E):
    """Columns with a block of ones, a cluster of signed zeros and values
    that round to a bfloat16 zero (+-1e-41) or to a negative bfloat16
    subnormal (-3e-39), and -1 below; the block of ones grows with the
    column (period 12) so that the wanted rank falls at different places of
    the cluster."""
    rng = np.random.default_rng(seed)
    pattern = np.array([0.0, -0.0, -1e-41, 1e-41, -3e-39], np.float32)
    Z = np.full((N, E), -1.0, np.float32)
    for e in range(E):
        ones = 2 * (e % 12)
        Z[:ones, e] = 1.0
        Z[ones:ones + 30, e] = pattern[rng.integers(0, 5, 30)]
        Z[:, e] = Z[rng.permutation(N), e]
    return Z


@pytest.mark.parametrize("key_bits", [16, 32])
def test_eqb_signed_zeros_and_subnormals(M, key_bits):
    """-0 and +0 are one value of the selection (bfloat16 keys also merge
    the values that round to -0); the quantile lands in the zero cluster."""
    say("eqb signed zeros", key_bits)
    N, E, K = 64, 8, 2  # r = 16
    Z = _signed_zero_logits(221, N, E)
    alpha = np.zeros(N, np.float32)
    alpha[::3] = -0.0
    bo, q = M.eqb_bias(dev(Z), K, alpha=dev(alpha), key_bits=key_bits)
    bo, q = host(bo), host(q)
    rb, rq, _ = O.eqb_expert_bias(Z, alpha, K, key_bits)
    assert bits_equal(q, rq), (q, rq)
    assert bits_equal(bo, rb)
    assert np.any(q == 0.0)


def _wide_span_logits(seed, N, E, K):
    """Every row's K largest logits are columns 0..K-1 (1 + |n|), its
    (K+1)-th is column K at exactly 0 (so alpha = -0 and v = Z), and the
    other columns are -s_e |n| with s_e log-uniform over 1e-30 .. 1: the
    quantiles then span about a hundred binades, more than a sum of E
    of them can hold exactly in fp64."""
    rng = np.random.default_rng(seed)
    Z = np.empty((N, E), np.float32)
    Z[:, :K] = 1.0 + np.abs(rng.standard_normal((N, K)))
    Z[:, K] = 0.0
    s = 10.0 ** rng.uniform(-30, 0, E - K - 1)
    Z[:, K + 1:] = -(s[None, :] * np.abs(rng.standard_normal((N, E - K - 1))))
    return Z.astype(np.float32)


@pytest.mark.parametrize("key_bits", [16, 32])
def test_eqb_centring_wide_exponent_span(M, key_bits):
    """Quantiles whose sum is not exact in fp64 in every order: the
    centring must then add them in expert order (the block-parallel sum is
    taken only when every partial sum is exact), bit for bit with the
    oracle; moe_eqb_bias (the one-block centring) and moe_forward (the final
    routing pass centres the biases itself) both."""
    N, E, K = 2048, 384, 6
    Z = _wide_span_logits(231, N, E, K)
    say("eqb wide exponent span", key_bits)
    _, alpha, _ = O.route(Z, None, K)
    assert np.all(alpha == 0.0)
    rb, rq, _ = O.eqb_expert_bias(Z, alpha, K, key_bits)
    nz = np.abs(rq[rq != 0].astype(np.float64))
    assert np.log2(nz.max()) - np.log2(nz.min()) > 60
    bo, q = M.eqb_bias(dev(Z), K, key_bits=key_bits)
    assert bits_equal(host(q), rq)
    assert bits_equal(host(bo), rb)
    # the layer with these logits given: its beta_out comes from the routing pass
    from synth import CONFIGS, make_inputs, scaled
    from tests.gpu_util import bf16_dev, weights_dev
    cfg = scaled(CONFIGS["prefill"], N)
    L = make_inputs(cfg)
    _, A = M.forward(bf16_dev(L.x), weights_dev(L), K, recompute_bias=True, key_bits=key_bits,
                     logits_in=dev(Z), aux=("beta_out", "quantile_out"))
    assert bits_equal(host(A["quantile_out"]), rq)
    assert bits_equal(host(A["beta_out"]), rb)


def test_route_signed_zeros(M):
    """Logits and biases with both zeros: -0 + -0 is the only -0 sum, and it
    ties with +0 (ids by expert order, alpha and margin bit-exact)."""
    say("route signed zeros")
    Z = _signed_zero_logits(222, 64, 8)
    beta = np.array([-0.0, 0.0, -0.0, 0.0, -0.0, -0.0, 0.0, 0.0], np.float32)
    for K in (1, 2, 5):
        _route_case(M, Z, beta, K)
    # the 384-wide kernel (16 lanes per row) on the same kind of data
    Z = _signed_zero_logits(223, 200, 384)
    beta = np.where(np.arange(384) % 2 == 0, -0.0, 0.0).astype(np.float32)
    _route_case(M, Z, beta, 6)


@pytest.mark.parametrize("E", [384, 100, 383])
def test_route_extreme_logits(M, E):
    """Very negative logits: mixture weights near the bottom of the fp32
    range (z around -100, where the weight is a subnormal float) and far
    below 1 but normal (z around -50), for the 16-lanes-per-row kernel
    (E = 384 and 100) and the one-wave kernel (E = 383)."""
    say("route extreme logits", E)
    rng = np.random.default_rng(224)
    Z = rng.standard_normal((200, E)).astype(np.float32)
    Z[:100] -= 100.0
    Z[100:] -= 50.0
    beta = make_bias(225, E, 0.1)
    _route_case(M, Z, beta, 6)


@pytest.mark.parametrize("key_bits", [16, 32])
def test_eqb_printed_toy(M, key_bits):
    g = json.load(open(GOLD))
    Z = np.array(g["logits"]["Z"], np.float32)
    say("eqb toy", key_bits)
    bo, q = _eqb_case(M, Z, None, 2, key_bits, give_alpha=False)
    assert (-q).tolist() == g["expert_bias"]["beta_raw"]
    assert bo.tolist() == g["centring"]["beta"]
