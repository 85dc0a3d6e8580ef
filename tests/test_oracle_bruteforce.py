"""The oracle against brute force, closed forms, library routines and special
cases on tiny inputs (no GPU).  Each case is chosen so that a plausible slip
in the oracle (a dropped term, a wrong sign or index, a transposed operand,
an unstable sort) fails it."""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import make_logits


# ---------------------------------------------------------------- bf16 helpers
def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 3,
        rng.standard_normal(2000).astype(np.float32) * 1e-30,
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, -3.0e38, 1e-45], np.float32),
    ])
    # exact halfway cases, even and odd kept parts
    base = rng.integers(0, 0x7F7F, 4000).astype(np.uint32) << 16
    halves = (base | 0x8000).view(np.float32)
    v = np.concatenate([v, halves, (base | 0x18000).view(np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f32_to_bf16_rne(v)
    assert np.array_equal(got, want)
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_to_f32(want).view(np.uint32), back.view(np.uint32))


def test_bf16_round_rejects_nonfinite():
    with pytest.raises(ValueError):
        O.f32_to_bf16_rne(np.array([np.inf], np.float32))


# ---------------------------------------------------------------- quantile
def test_quantile_counting_definition():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        a = rng.integers(-5, 6, n).astype(np.float32) / 2  # many repeats
        m = int(rng.integers(0, n))
        q = O.quantile(a, m)
        assert q in a
        assert (a > q).sum() <= m < (a >= q).sum()


def test_quantile_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.quantile([1.0, 2.0], 2)


# ---------------------------------------------------------------- routing
def _brute_route(Z, beta, K):
    T, E = Z.shape
    ids = np.zeros((T, K), np.int32)
    alpha = np.zeros(T, np.float32)
    margin = np.zeros(T, np.float32)
    for t in range(T):
        vals = []
        for e in range(E):
            b = np.float32(Z[t, e]) + np.float32(0 if beta is None else beta[e])
            b = float(np.float32(b))
            if b == 0.0:
                b = 0.0  # -0 -> +0
            vals.append((b, e))
        srt = sorted(vals, key=lambda p: (-p[0], p[1]))
        ids[t] = [e for _, e in srt[:K]]
        alpha[t] = np.float32(-srt[K][0])
        margin[t] = np.float32(np.float32(srt[K - 1][0]) - np.float32(srt[K][0]))
    return ids, alpha, margin


@pytest.mark.parametrize("seed,T,E,K,ties", [
    (1, 7, 9, 3, 0.0), (2, 5, 4, 2, 0.5), (3, 6, 16, 8, 0.9), (4, 3, 12, 1, 0.7),
    (5, 9, 33, 6, 0.3)])
def test_route_matches_full_sort(seed, T, E, K, ties):
    Z = make_logits(seed, T, E, 1.0, tie_fraction=ties)
    beta = make_logits(seed + 100, 1, E, 0.5, tie_fraction=ties)[0]
    for b in (None, beta):
        ids, alpha, margin = O.route(Z, b, K)
        bi, ba, bm = _brute_route(Z, b, K)
        assert np.array_equal(ids, bi)
        assert np.array_equal(alpha.view(np.uint32), ba.view(np.uint32))
        assert np.array_equal(margin.view(np.uint32), bm.view(np.uint32))


def test_route_all_equal_rows_and_signed_zero():
    Z = np.zeros((3, 6), np.float32)
    Z[1] = -0.0
    Z[2, 4] = -0.0
    ids, alpha, margin = O.route(Z, None, 3)
    assert ids.tolist() == [[0, 1, 2]] * 3
    assert np.all(margin == 0) and np.all(np.signbit(margin) == False)  # noqa: E712
    assert np.all(np.signbit(alpha))  # alpha = -(+0)


def test_mixture_weights_are_unbiased_sigmoids():
    Z = make_logits(9, 5, 10, 2.0)
    ids_a, _, _ = O.route(Z, None, 3)
    big = np.zeros(10, np.float32)
    big[7] = 100.0  # the bias forces expert 7 in, but must not change weights
    ids_b, _, _ = O.route(Z, big, 3)
    assert (ids_b == 7).any(axis=1).all()
    S = O.mixture_weights(Z, ids_b)
    for t in range(5):
        for k in range(3):
            z = float(Z[t, ids_b[t, k]])
            assert S[t, k] == np.float32(1.0 / (1.0 + math.exp(-z)))
    assert not np.allclose(S.sum(axis=1), 1.0)  # no renormalisation


# ---------------------------------------------------------------- EQB
@pytest.mark.parametrize("key_bits", [16, 32])
@pytest.mark.parametrize("seed,T,E,K,ties", [(21, 40, 8, 2, 0.0), (22, 64, 16, 3, 0.6),
                                             (23, 30, 5, 4, 0.9)])
def test_eqb_matches_columnwise_sort(seed, T, E, K, ties, key_bits):
    Z = make_logits(seed, T, E, 1.0, tie_fraction=ties)
    beta_in = make_logits(seed + 7, 1, E, 0.1)[0]
    _, alpha, _ = O.route(Z, beta_in, K)
    beta_new, Q, beta_raw = O.eqb_expert_bias(Z, alpha, K, key_bits)
    r = T * K // E
    for e in range(E):
        col = []
        for t in range(T):
            v = np.float32(np.float32(Z[t, e]) + np.float32(alpha[t]))
            if key_bits == 16:
                v = O.bf16_to_f32(O.f32_to_bf16_rne(np.array([v])))[0]
            col.append(float(v) + 0.0)
        col.sort(reverse=True)
        assert float(Q[e]) == col[r]
        # tie-proof exactness invariant: #{u > Q} <= r < #{u >= Q}
        assert sum(c > col[r] for c in col) <= r < sum(c >= col[r] for c in col)
    assert np.array_equal(beta_raw, -Q)
    # centring: constant shift, zero mean (to fp32 rounding)
    shift = beta_new.astype(np.float64) - beta_raw.astype(np.float64)
    assert np.ptp(shift) <= 4 * np.finfo(np.float32).eps * (1 + np.abs(beta_raw).max())
    assert abs(beta_new.astype(np.float64).mean()) <= 1e-6 * (1 + np.abs(beta_raw).max())


def test_eqb_centring_uses_sequential_fp64_sum():
    # values whose fp32 pairwise sum would differ; fp64 sequential sum is exact here
    Z = np.array([[1e7, 1.0, -1e7, 3.0]], np.float32)
    alpha = np.zeros(1, np.float32)
    beta_new, Q, beta_raw = O.eqb_expert_bias(Z, alpha, 1, 32)
    # r = floor(1*1/4) = 0 -> Q = the column maximum = the single entry
    assert Q.tolist() == Z[0].tolist()
    mean = (-1e7 - 1.0 + 1e7 - 3.0) / 4
    assert beta_new.tolist() == [np.float32(-z - mean) for z in Z[0].tolist()]


def test_eqb_sixteen_bit_mode_rounds_before_selecting():
    """16-bit keys select among bf16-rounded values (round to nearest even),
    which can change the quantile against 32-bit keys."""
    one = 1.0
    col = np.array([one + 2 ** -8,          # exact half ulp, kept part even -> 1.0
                    one + 3 * 2 ** -9,      # above half ulp -> 1.0078125
                    one + 2 ** -9,          # below half ulp -> 1.0
                    one + 2 ** -7 + 2 ** -8,  # exact half ulp, kept part odd -> 1.015625
                    0.5], np.float32)
    Z = np.stack([col, np.zeros_like(col)], axis=1)  # T=5, E=2
    alpha = np.zeros(5, np.float32)
    # K=1, E=2, T=5 -> r = 2: the third largest of column 0
    _, Q16, _ = O.eqb_expert_bias(Z, alpha, 1, 16)
    _, Q32, _ = O.eqb_expert_bias(Z, alpha, 1, 32)
    assert Q32[0] == np.float32(one + 2 ** -8)       # 1.0117, 1.0059, [1.0039], ...
    assert Q16[0] == np.float32(1.0)                 # 1.015625, 1.0078125, [1.0], 1.0, 0.5


# ---------------------------------------------------------------- grouping
@pytest.mark.parametrize("seed,T,E,K", [(31, 50, 7, 3), (32, 1, 5, 2), (33, 200, 40, 6)])
def test_grouping_matches_stable_sorted(seed, T, E, K):
    Z = make_logits(seed, T, E)
    ids, _, _ = O.route(Z, None, K)
    counts, offsets, sorted_src, src_pos = O.group_by_expert(ids, E)
    pairs = [(int(ids[t, k]), t, t * K + k) for t in range(T) for k in range(K)]
    want = [p[2] for p in sorted(pairs, key=lambda p: p[0])]  # Python sort is stable
    assert sorted_src.tolist() == want
    assert counts.sum() == T * K
    for e in range(E):
        seg = sorted_src[offsets[e]:offsets[e + 1]]
        assert len(seg) == counts[e]
        assert all(ids.ravel()[s] == e for s in seg)
        toks = [s // K for s in seg]
        assert toks == sorted(toks)
    assert np.array_equal(sorted_src[src_pos.ravel()], np.arange(T * K))


# ---------------------------------------------------------------- GEMMs / MLPs
def test_router_logits_match_loops():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    off = rng.standard_normal(4).astype(np.float32)
    Z = O.router_logits(x, w, off)
    for t in range(3):
        for e in range(4):
            s = sum(float(x[t, j]) * float(w[e, j]) for j in range(5))
            assert Z[t, e] == np.float32(np.float32(s) + off[e])


def test_swiglu_matches_loops_nonsquare():
    rng = np.random.default_rng(42)
    n, d, h = 3, 5, 2
    X = rng.standard_normal((n, d))
    Wg = rng.standard_normal((h, d))
    Wu = rng.standard_normal((h, d))
    Wd = rng.standard_normal((d, h))
    Y = O.swiglu(X, Wg, Wu, Wd)
    for i in range(n):
        Hrow = []
        for j in range(h):
            g = sum(X[i, c] * Wg[j, c] for c in range(d))
            u = sum(X[i, c] * Wu[j, c] for c in range(d))
            Hrow.append(g / (1 + math.exp(-g)) * u)
        for c in range(d):
            ref = sum(Hrow[j] * Wd[c, j] for j in range(h))
            assert abs(Y[i, c] - ref) <= 1e-12 * (1 + abs(ref))


def _tiny_layer(seed, T=6, d=8, E=5, K=2, h=3, S=1):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((T, d)), w_router=rng.standard_normal((E, d)),
                w_gate=rng.standard_normal((E, h, d)), w_up=rng.standard_normal((E, h, d)),
                w_down=rng.standard_normal((E, d, h)), ws_gate=rng.standard_normal((S, h, d)),
                ws_up=rng.standard_normal((S, h, d)), ws_down=rng.standard_normal((S, d, h)))


def test_layer_output_matches_loops():
    L = _tiny_layer(51)
    beta = np.array([0.3, -0.2, 0.0, 0.5, -0.1], np.float32)
    out = O.moe_layer(**L, beta_in=beta, K=2)
    T = L["x"].shape[0]
    for t in range(T):
        y = O.swiglu(L["x"][t:t + 1], L["ws_gate"][0], L["ws_up"][0], L["ws_down"][0])[0]
        for k in range(2):
            e = out["topk_ids"][t, k]
            z = float(out["logits"][t, e])
            w = 1 / (1 + math.exp(-z))
            y = y + w * O.swiglu(L["x"][t:t + 1], L["w_gate"][e], L["w_up"][e], L["w_down"][e])[0]
        assert np.allclose(out["y"][t], y, rtol=1e-6, atol=1e-9)


def test_layer_zero_routed_weights_gives_shared_only():
    L = _tiny_layer(52)
    L["w_down"] = np.zeros_like(L["w_down"])
    out = O.moe_layer(**L, beta_in=None, K=2)
    sh = O.swiglu(L["x"], L["ws_gate"][0], L["ws_up"][0], L["ws_down"][0])
    assert np.array_equal(out["y"], sh)


def test_layer_identical_experts_scale_by_weight_sum():
    L = _tiny_layer(53)
    for k in ("w_gate", "w_up", "w_down"):
        L[k] = np.repeat(L[k][:1], L[k].shape[0], axis=0)
    out = O.moe_layer(**L, beta_in=None, K=2)
    sh = O.swiglu(L["x"], L["ws_gate"][0], L["ws_up"][0], L["ws_down"][0])
    f = O.swiglu(L["x"], L["w_gate"][0], L["w_up"][0], L["w_down"][0])
    want = sh + out["topk_weights"].astype(np.float64).sum(axis=1)[:, None] * f
    assert np.allclose(out["y"], want, rtol=1e-12, atol=1e-12)


def test_layer_without_shared_expert_and_token_subset():
    L = _tiny_layer(54, S=0)
    out = O.moe_layer(**L, beta_in=None, K=2)
    sub = O.moe_layer(**L, beta_in=None, K=2, token_subset=[4, 1])
    assert np.allclose(sub["y"], out["y"][[4, 1]], rtol=1e-13, atol=1e-13)
    L1 = _tiny_layer(54, S=1)
    L1["ws_down"] = np.zeros_like(L1["ws_down"])
    out1 = O.moe_layer(**L1, beta_in=None, K=2)
    assert np.allclose(out1["y"], out["y"], rtol=1e-13, atol=1e-13)


def test_recompute_balances_a_collapsed_router():
    """With a +3 offset on experts 0 and 1 every token picks them; one exact
    update spreads the load (MaxVio falls)."""
    rng = np.random.default_rng(61)
    T, d, E, K = 64, 16, 8, 2
    x = rng.standard_normal((T, d))
    w = rng.standard_normal((E, d)) * 0.02
    off = np.zeros(E, np.float32)
    off[:2] = 3.0
    L = _tiny_layer(61, T=T, d=d, E=E, K=K)
    L.update(x=x, w_router=w)
    out = O.moe_layer(**L, beta_in=None, K=K, recompute_bias=True,
                      logit_offset=off, compute_output=False)
    assert out["counts_before"][:2].tolist() == [T, T]
    assert O.max_vio(out["counts"], T, K, E) < O.max_vio(out["counts_before"], T, K, E)


def test_near_tie_count_threshold_is_strict():
    m = np.array([0.0, 5e-4, np.float32(1e-3), 2e-3, 0.5], np.float32)
    assert O.near_tie_count(m, 1e-3) == 2
    assert O.near_tie_count(m, 0.0) == 0
    assert O.near_tie_count(m, 1.0) == 5
