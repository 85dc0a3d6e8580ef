"""GPU parity of the exact quantile update over a batch given in parts
(moe_eqb_begin / moe_eqb_accumulate / moe_eqb_select) against the oracle:
quantiles and biases bit-exact, equal to the whole-batch update however the
rows are split, including the printed two-rank split of the running example."""
import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import make_bias, make_logits
from tests.gpu_util import bits_equal, dev, host, say

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


def _parts_case(M, Z, beta, K, key_bits, sizes):
    assert sum(sizes) == Z.shape[0]
    bounds = np.cumsum([0] + list(sizes))
    Zp = [Z[bounds[i]:bounds[i + 1]] for i in range(len(sizes))]
    # token biases per part (alpha is per row, so parts see their own rows)
    ap = [O.route(z, beta, K)[1] for z in Zp]
    bo, q = M.eqb_bias_parts([dev(z) for z in Zp], [dev(a) for a in ap], K, key_bits)
    bo, q = host(bo), host(q)
    rb, rq, _ = O.eqb_expert_bias_parts(Zp, ap, K, key_bits)
    assert bits_equal(q, rq), "quantiles differ"
    assert bits_equal(bo, rb), "biases differ"
    # the same as the whole-batch entry point on the GPU
    whole_b, whole_q = M.eqb_bias(dev(Z), K, beta_in=dev(beta), key_bits=key_bits)
    assert bits_equal(host(whole_b), bo) and bits_equal(host(whole_q), q)
    return bo, q


PARTS_CASES = [
    # seed, N, E, K, ties, sizes
    (301, 3000, 384, 6, 0.0, [1, 700, 1299, 1000]),
    (302, 3000, 384, 6, 0.7, [3000]),
    (303, 2048, 128, 8, 0.3, [512, 512, 512, 512]),
    (304, 999, 100, 5, 0.5, [333, 1, 1, 664]),
    (305, 65, 65, 4, 0.0, [64, 1]),
]


@pytest.mark.parametrize("key_bits", [16, 32])
@pytest.mark.parametrize("seed,N,E,K,ties,sizes", PARTS_CASES)
def test_eqb_parts_parity(M, seed, N, E, K, ties, sizes, key_bits):
    say("eqb parts", seed, N, E, K, ties, sizes, key_bits)
    Z = make_logits(seed, N, E, 1.0, tie_fraction=ties)
    beta = make_bias(seed + 1, E, 0.1)
    _parts_case(M, Z, beta, K, key_bits, sizes)


@pytest.mark.parametrize("key_bits", [16, 32])
def test_eqb_parts_printed_split(M, key_bits):
    """Tokens t1, t2 on one part and t3, t4 on the other: the update reaches
    the printed global quantile 1.5 for e1 and the printed biases."""
    g = json.load(open(GOLD))
    Z = np.array(g["logits"]["Z"], np.float32)
    say("eqb parts toy", key_bits)
    bo, q = _parts_case(M, Z, np.zeros(4, np.float32), 2, key_bits, [2, 2])
    assert float(q[0]) == g["average_of_quantiles"]["global"]
    assert (-q).tolist() == g["expert_bias"]["beta_raw"]
    assert bo.tolist() == g["centring"]["beta"]


def test_eqb_parts_full_size(M):
    """The skewed batch (N=65536, E=384, K=6) in 16 parts of 4096 rows."""
    say("eqb parts full")
    Z = make_logits(311, 65536, 384, 0.6)
    p = np.arange(1, 385, dtype=np.float64) ** -1.2
    Z = (Z + (0.5 * np.log(p / p.sum())).astype(np.float32)[None, :]).astype(np.float32)
    beta = make_bias(312, 384, 0.1)
    _parts_case(M, Z, beta, 6, 16, [4096] * 16)
