"""The oracle against the values the pages print for the running example.

Every expected number comes from tests/golden/*.json, each entry citing the
page and section it was read from.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


TOY = _gold("toy_routing_eqb.json")
Z_TOY = np.array(TOY["logits"]["Z"], dtype=np.float32)
K_TOY = TOY["logits"]["K"]


def test_quantile_definition_example():
    q = TOY["quantile_example"]
    assert O.quantile(q["list"], q["m"]) == q["value"]


def test_toy_collapsed_routing_and_maxvio():
    ids, alpha, margin = O.route(Z_TOY, None, K_TOY)
    assert [sorted(r) for r in ids.tolist()] == TOY["logits"]["top2_with_beta0"]
    counts = np.bincount(ids.ravel(), minlength=4)
    assert counts.tolist() == TOY["logits"]["loads_with_beta0"]
    assert O.max_vio(counts, 4, K_TOY, 4) == TOY["maxvio_before"]["value"]


def test_toy_token_bias():
    _, alpha, _ = O.route(Z_TOY, None, K_TOY)
    assert alpha.tolist() == TOY["token_bias"]["alpha"]


@pytest.mark.parametrize("key_bits", [16, 32])
def test_toy_expert_bias_and_centring(key_bits):
    _, alpha, _ = O.route(Z_TOY, None, K_TOY)
    cols = (Z_TOY + alpha[:, None]).T
    assert cols.tolist() == TOY["expert_bias"]["columns_Z_plus_alpha"]
    beta_new, Q, beta_raw = O.eqb_expert_bias(Z_TOY, alpha, K_TOY, key_bits)
    assert beta_raw.tolist() == TOY["expert_bias"]["beta_raw"]
    assert (-Q).tolist() == TOY["expert_bias"]["beta_raw"]
    assert beta_new.tolist() == TOY["centring"]["beta"]
    # exactness: r = 2 positive entries per column of Z + alpha + beta_raw
    M = Z_TOY + alpha[:, None] + beta_raw[None, :]
    assert ((M > 0).sum(axis=0) == TOY["expert_bias"]["positives_per_column"]).all()
    assert M[:, 0].tolist() == TOY["expert_bias"]["column_e1_after"]


def test_toy_reroute_after_update():
    beta = np.array(TOY["centring"]["beta"], dtype=np.float32)
    B = Z_TOY + beta[None, :]
    assert B.tolist() == TOY["reroute"]["B"]
    ids, _, _ = O.route(Z_TOY, beta, K_TOY)
    assert [sorted(r) for r in ids.tolist()] == TOY["reroute"]["top2_sets"]
    counts = np.bincount(ids.ravel(), minlength=4)
    assert counts.tolist() == TOY["reroute"]["loads"]
    assert O.max_vio(counts, 4, K_TOY, 4) == TOY["reroute"]["maxvio_after"]


def test_toy_full_layer_path_matches_pages():
    """moe_layer with recompute on the printed logits reproduces the update."""
    E = 4
    out = O.moe_layer(x=np.zeros((4, 8)), w_router=np.zeros((E, 8)),
                      w_gate=np.zeros((E, 4, 8)), w_up=np.zeros((E, 4, 8)),
                      w_down=np.zeros((E, 8, 4)), ws_gate=np.zeros((0, 4, 8)),
                      ws_up=np.zeros((0, 4, 8)), ws_down=np.zeros((0, 8, 4)),
                      beta_in=None, K=K_TOY, recompute_bias=True,
                      logits_in=Z_TOY)
    assert out["counts_before"].tolist() == TOY["logits"]["loads_with_beta0"]
    assert out["beta_out"].tolist() == TOY["centring"]["beta"]
    assert out["counts"].tolist() == TOY["reroute"]["loads"]


def test_toy_unbiased_mixture_weights():
    mw = TOY["mixture_weights"]
    beta = np.array(TOY["centring"]["beta"], dtype=np.float32)
    ids, _, _ = O.route(Z_TOY, beta, K_TOY)
    S = O.mixture_weights(Z_TOY, ids)
    t = mw["token"]
    got = dict(zip(ids[t].tolist(), S[t].tolist()))
    assert sorted(got) == mw["experts"]
    for e, w in zip(mw["experts"], mw["weights_3dp"]):
        assert round(got[e], 3) == w
    assert round(sum(got.values()), 3) == mw["sum_3dp"]


def test_average_of_local_quantiles_is_not_the_global_quantile():
    a = TOY["average_of_quantiles"]
    qa = O.quantile(a["rank_a"], a["local_m"])
    qb = O.quantile(a["rank_b"], a["local_m"])
    assert [qa, qb] == a["local_quantiles"]
    assert (qa + qb) / 2 == a["average"]
    assert O.quantile(a["rank_a"] + a["rank_b"], a["global_m"]) == a["global"]
    # and the EQB update over the union uses the global value for expert e1
    _, alpha, _ = O.route(Z_TOY, None, K_TOY)
    _, Q, _ = O.eqb_expert_bias(Z_TOY, alpha, K_TOY)
    assert Q[0] == a["global"]


def test_eqb_over_parts_uses_the_global_quantile():
    """[KPT] §7.3 split: tokens t1, t2 on one rank and t3, t4 on the other.
    The update over the two parts reaches the printed global quantile 1.5 for
    e1 (not the 1.0 of averaged local quantiles) and the whole-batch biases."""
    a = TOY["average_of_quantiles"]
    parts = [Z_TOY[:2], Z_TOY[2:]]
    alphas = [O.route(z, None, K_TOY)[1] for z in parts]  # alpha is per token
    # the e1 column of v = Z + alpha on each rank is the printed one
    assert [float(v) for v in (parts[0][:, 0] + alphas[0])] == a["rank_a"]
    assert [float(v) for v in (parts[1][:, 0] + alphas[1])] == a["rank_b"]
    for kb in (16, 32):
        beta, Q, beta_raw = O.eqb_expert_bias_parts(parts, alphas, K_TOY, kb)
        assert Q[0] == a["global"]
        _, alpha, _ = O.route(Z_TOY, None, K_TOY)
        beta1, Q1, _ = O.eqb_expert_bias(Z_TOY, alpha, K_TOY, kb)
        assert np.array_equal(beta.view(np.uint32), beta1.view(np.uint32))
        assert np.array_equal(Q.view(np.uint32), Q1.view(np.uint32))


def _radix_select_desc(keys, rank, base, digits):
    """Test-only radix selection of the rank-th largest key (1-based),
    most significant digit first, as in the two-digit analogue."""
    cand = list(keys)
    prefix = 0
    for p in reversed(range(digits)):
        div = base ** p
        hist = {}
        for k in cand:
            hist[(k // div) % base] = hist.get((k // div) % base, 0) + 1
        above = 0
        for b in sorted(hist, reverse=True):
            if above + hist[b] >= rank:
                rank -= above
                cand = [k for k in cand if (k // div) % base == b]
                prefix = prefix * base + b
                break
            above += hist[b]
    assert len(set(cand)) == 1
    return cand[0]


def test_radix_walkthrough_two_digits():
    w = TOY["radix_walkthrough"]
    hist = {}
    for k in w["keys"]:
        hist[k // 10] = hist.get(k // 10, 0) + 1
    assert {str(k): v for k, v in hist.items()} == w["tens_bins"]
    key = _radix_select_desc(w["keys"], w["want_rank"], 10, 2)
    assert key == w["key"] and key / 10 == w["value"]


def test_radix_select_base256_matches_oracle_quantile_on_bf16_keys():
    """Base-256 two-pass selection over order-preserving 16-bit keys of bf16
    values returns the same value as the oracle's sort-defined quantile."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        n = int(rng.integers(2, 300))
        v = rng.standard_normal(n).astype(np.float32)
        if trial % 3 == 0:
            v = np.round(v * 4) / 4  # heavy ties and zeros
            v = v.astype(np.float32)
        u = O.eqb_keys_values(v, 16)
        bits = O.f32_to_bf16_rne(u).astype(np.int64)
        keys = np.where(bits & 0x8000, 0xFFFF - bits, bits | 0x8000)
        m = int(rng.integers(0, n))
        k = _radix_select_desc(keys.tolist(), m + 1, 256, 2)
        b = k - 0x8000 if k >= 0x8000 else 0xFFFF - k
        val = O.bf16_to_f32(np.array([b], np.uint16))[0]
        assert val == O.quantile(u, m)


def test_histogram_bytes():
    h = TOY["histogram_bytes"]
    assert h["bins"] * h["E"] * 4 == h["bytes"]


def test_intervention_rate_toy_and_random_routing_expectation():
    ir = TOY["intervention_rate"]
    beta = np.array(TOY["centring"]["beta"], dtype=np.float32)
    ids_u, _, _ = O.route(Z_TOY, None, K_TOY)
    ids_r, _, _ = O.route(Z_TOY, beta, K_TOY)
    assert O.intervention_rate(ids_u, ids_r) == ir["toy_value"]
    K, E = ir["kolibri_K"], ir["kolibri_E"]
    assert round(1 - K / E, 3) == ir["kolibri_expected_3dp"]
    # Monte Carlo: routed sets uniformly random -> E[I] = 1 - K/E
    rng = np.random.default_rng(3)
    T = 20000
    ids_u = np.tile(np.arange(K), (T, 1))
    ids_r = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    got = O.intervention_rate(ids_u, ids_r)
    sd = math.sqrt((K / E) / K / T)  # loose binomial-like bound
    assert abs(got - (1 - K / E)) < 6 * sd


def test_expert_weight_counts():
    g = _gold("expert_sizes.json")
    per = 3 * g["d"] * g["h"]
    assert per == g["weights_per_expert"]
    assert round(per * g["experts_touched_per_token"] / 1e6, 1) == g["weights_touched_per_token_millions_1dp"]
    assert round(per * g["experts_per_block"] / 1e9, 2) == g["weights_per_block_billions_2dp"]


LEI = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lei_check.json")))


def test_lei_printed_check():
    """[KPT] §8 numerical check on the collapsed running example."""
    ids, _, _ = O.route(Z_TOY, None, K_TOY)
    assert np.bincount(ids.ravel(), minlength=4).tolist() == LEI["loads"]
    rho, xi, scale, inj = O.lei_injection(ids, 4, LEI["lambda"], LEI["tau"])
    assert rho.tolist() == LEI["rho"]
    assert xi == LEI["xi"]
    assert round(scale, 4) == LEI["tanh_xi_over_xi_4dp"]
    assert np.allclose(inj, LEI["lambda"] * scale * np.array(LEI["rho"]), rtol=0, atol=0)
    # score gradients all receive the injection; the logit of (t1, e1) gets it
    # times sigma'(2.0)
    Gp, dZ = O.lei_backward(Z_TOY, ids, None, LEI["lambda"], LEI["tau"])
    assert np.array_equal(Gp, np.tile(inj, (4, 1)))
    t, e = LEI["token"], LEI["expert"]
    assert float(Z_TOY[t, e]) == 2.0
    sp = dZ[t, e] / inj[e]
    assert round(sp, 3) == LEI["sigma_prime_at_2_3dp"]
    assert abs(dZ[t, e] - LEI["lambda"] * LEI["tanh_xi_over_xi_4dp"]
               * LEI["sigma_prime_at_2_3dp"]) < 1e-9


def test_lei_bound_and_balanced_limit():
    """|injection| <= lam * tau * tanh(xi) < lam * tau however lopsided the
    loads ([KPT] §8); a perfectly balanced microbatch gets no injection and
    the scale is 1 (its continuous limit at xi = 0)."""
    rng = np.random.default_rng(5)
    for lam, tau, skew in ((1e-5, 1.0, 0.0), (1e-3, 0.25, 3.0), (0.5, 2.0, 8.0)):
        T, E, K = 512, 64, 4
        p = np.exp(-skew * np.arange(E) / E)
        p /= p.sum()
        ids = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)])
        rho, xi, scale, inj = O.lei_injection(ids, E, lam, tau)
        assert np.max(np.abs(inj)) <= lam * tau * math.tanh(xi) * (1 + 1e-12)
        assert np.max(np.abs(inj)) < lam * tau
        assert np.isclose(xi, np.max(np.abs(rho)) / tau)
    ids = np.tile(np.arange(4), (8, 1)).reshape(-1, 2)  # every expert loaded equally
    rho, xi, scale, inj = O.lei_injection(ids, 4, 1e-5, 1.0)
    assert xi == 0.0 and scale == 1.0 and not inj.any()
    # small imbalance: tanh(xi)/xi = 1 - xi^2/3 + O(xi^4), the injection ~ lam * rho
    _, xi, scale, _ = O.lei_injection(np.array([[0, 1]] * 999 + [[0, 2]]), 1000, 1.0, 1e6)
    assert 0 < xi < 1e-3 and abs(scale - (1 - xi * xi / 3)) < xi ** 4
