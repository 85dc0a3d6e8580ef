"""GPU parity of moe_route_stats (routing diagnostics) against the oracle:
loads, extreme loads, slot overlap and near-tie counts exact; MaxVio exact
(one fp64 division of exact integers); the intervention rate within 1e-12
(the oracle averages per-token fractions, the kernel divides the integer
sum).  The printed running example pins MaxVio and the intervention rate."""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import make_bias, make_logits
from tests.gpu_util import dev, host, say

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


def _stats_case(M, Z, beta, K, tau=1e-3):
    N, E = Z.shape
    ids, _, _, margin = M.route(dev(Z), K, dev(beta))
    ids_u, _, _, _ = M.route(dev(Z), K, None)
    counts, st = M.route_stats(ids, E, ids_u, margin, tau)
    counts, st = host(counts), M.read_route_stats(st)
    ri, _, rm = O.route(Z, beta, K)
    ru, _, _ = O.route(Z, None, K)
    rc = np.bincount(ri.ravel(), minlength=E)
    assert np.array_equal(counts, rc)
    assert st["max_load"] == rc.max() and st["min_load"] == rc.min()
    overlap = sum(len(set(ri[t]) & set(ru[t])) for t in range(N))
    assert st["overlap"] == overlap
    assert st["near_ties"] == O.near_tie_count(rm, tau)
    assert st["max_vio"] == O.max_vio(rc, N, K, E)
    assert abs(st["intervention_rate"] - O.intervention_rate(ru, ri)) <= 1e-12
    return st


@pytest.mark.parametrize("seed,N,E,K,ties,bstd", [
    (401, 1, 9, 8, 0.0, 0.1), (402, 1000, 384, 6, 0.0, 0.1), (403, 4096, 128, 8, 0.5, 0.3),
    (404, 777, 100, 5, 0.9, 1.0), (405, 65536, 384, 6, 0.0, 0.1)])
def test_route_stats_parity(M, seed, N, E, K, ties, bstd):
    say("route stats", seed, N, E, K, ties, bstd)
    Z = make_logits(seed, N, E, 1.0, tie_fraction=ties)
    _stats_case(M, Z, make_bias(seed + 1, E, bstd), K)


def test_route_stats_printed_example(M):
    """Collapsed routing: MaxVio 1.0 before the update and 0 after; the
    intervention rate of the updated bias on the four tokens is printed."""
    g = json.load(open(GOLD))
    Z = np.array(g["logits"]["Z"], np.float32)
    say("route stats toy")
    before = _stats_case(M, Z, np.zeros(4, np.float32), 2)
    assert before["max_vio"] == g["maxvio_before"]["value"]
    after = _stats_case(M, Z, np.array(g["centring"]["beta"], np.float32), 2)
    assert after["max_vio"] == g["reroute"]["maxvio_after"]
    assert after["intervention_rate"] == g["intervention_rate"]["toy_value"]


def test_route_stats_random_bias_signature(M):
    """A bias much larger than the logits decides the selection: with random
    per-token winners the rate approaches 1 - K/E (E=384, K=6: 0.984)."""
    import torch
    say("route stats signature")
    rng = np.random.default_rng(7)
    N, E, K = 20000, 384, 6
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(N)]).astype(np.int32)
    ids_u = np.tile(np.arange(K, dtype=np.int32), (N, 1))
    counts, st = M.route_stats(torch.from_numpy(ids).cuda(), E, torch.from_numpy(ids_u).cuda())
    st = M.read_route_stats(st)
    assert abs(st["intervention_rate"] - O.intervention_rate(ids_u, ids)) <= 1e-12
    assert abs(st["intervention_rate"] - (1 - K / E)) < 0.003
    assert np.isnan(M.read_route_stats(M.route_stats(torch.from_numpy(ids).cuda(), E)[1])
                    ["intervention_rate"])
