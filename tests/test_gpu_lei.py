"""GPU parity of moe_lei_backward (Load-Error Injection) against the oracle:
the per-expert injection within 1e-6 relative (fp64 formed, fp32 rounded),
score gradients within one fp32 rounding of the fp64 sum, logit gradients
within 1e-5 relative to the largest logit gradient of the row (fp32 sigma');
the printed numerical check of the running example and the bound lam*tau."""
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import make_bias, make_logits
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

LEI = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lei_check.json")))
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "toy_routing_eqb.json")))


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


def _check(M, Z, ids, G, lam, tau, inplace=False):
    N, E = Z.shape
    Gd = dev(G) if G is not None else None
    gout, dz, inj = M.lei_backward(dev(ids), E, dev(Z), Gd, lam, tau, inplace=inplace)
    gout = host(Gd if inplace else gout).astype(np.float64)
    dz, inj = host(dz).astype(np.float64), host(inj).astype(np.float64)
    _, _, _, rinj = O.lei_injection(ids, E, lam, tau)
    Gf = None if G is None else G.astype(np.float32)
    rG, rdZ = O.lei_backward(Z, ids, Gf, lam, tau)
    assert np.all(np.abs(inj - rinj) <= 1e-6 * np.abs(rinj) + 1e-30)
    # fp32 sum of fp32 operands: within one rounding of the fp64 value
    assert np.all(np.abs(gout - rG) <= 2 ** -23 * np.abs(rG) + 1e-6 * np.abs(rinj).max() + 1e-30)
    scale = np.maximum(np.abs(rdZ).max(axis=1, keepdims=True), 1e-30)
    assert np.all(np.abs(dz - rdZ) <= 1e-5 * scale)
    return inj, gout, dz


def test_lei_printed_check(M):
    Z = np.array(GOLD["logits"]["Z"], np.float32)
    ids, _, _ = O.route(Z, None, 2)
    say("lei toy")
    inj, gout, dz = _check(M, Z, ids.astype(np.int32), None, LEI["lambda"], LEI["tau"])
    assert np.round(inj / LEI["lambda"], 4).tolist() == [
        r * LEI["tanh_xi_over_xi_4dp"] for r in LEI["rho"]]
    t, e = LEI["token"], LEI["expert"]
    assert abs(dz[t, e] - LEI["lambda"] * LEI["tanh_xi_over_xi_4dp"]
               * LEI["sigma_prime_at_2_3dp"]) < 1e-9


@pytest.mark.parametrize("seed,N,E,K,lam,tau,with_g,inplace", [
    (501, 3000, 384, 6, 1e-5, 1.0, True, False),
    (502, 3000, 384, 6, 1e-2, 0.5, False, False),
    (503, 777, 100, 5, 1e-3, 2.0, True, True),
    (504, 1, 9, 8, 1e-5, 1.0, True, False),
    (505, 16384, 384, 6, 1e-5, 1.0, True, True),
])
def test_lei_parity(M, seed, N, E, K, lam, tau, with_g, inplace):
    say("lei", seed, N, E, K, lam, tau, with_g, inplace)
    Z = make_logits(seed, N, E, 2.0)
    # skewed selections so that rho and xi are far from zero
    off = np.linspace(1.0, -1.0, E).astype(np.float32)
    ids, _, _ = O.route((Z + off).astype(np.float32), make_bias(seed + 1, E, 0.1), K)
    G = (np.random.default_rng(seed).standard_normal((N, E)) * 1e-4).astype(np.float32) \
        if with_g else None
    inj, _, _ = _check(M, Z, ids.astype(np.int32), G, lam, tau, inplace)
    _, xi, _, _ = O.lei_injection(ids, E, lam, tau)
    assert np.max(np.abs(inj)) <= lam * tau * math.tanh(xi) * (1 + 1e-6)
