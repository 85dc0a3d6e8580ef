"""moe_forward_noalloc (the layer with the library's fixed per-GPU scratch
array as workspace) against moe_forward, through the C ABI: two calls in a
row, the second with a smaller batch (the array keeps the first call's
contents), every output and aux field bit-equal to moe_forward's on the same
inputs; a problem that needs more than the array is rejected before any GPU
work.  Calls on one GPU share the array, so the test runs them in order on
one stream."""
import numpy as np
import pytest

from synth import CONFIGS, make_inputs, scaled
from tests.gpu_util import bf16_dev, dev, host, say, weights_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sigmoid_top_routing_router_amd as M
    M.load_library()
    return M


def _check(M, cfg):
    import torch
    L = make_inputs(cfg)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    kw = dict(beta_in=dev(L.beta_in), recompute_bias=cfg.recompute_bias,
              logit_offset=dev(L.logit_offset))
    say("no-alloc forward", cfg.name, cfg.N)
    need = M.forward_workspace_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared,
                                     cfg.h_shared, cfg.recompute_bias)
    assert need <= 64 << 20
    y_ref, A_ref = M.forward(x, W, cfg.K, aux=M.AUX_FIELDS, **kw)
    # the caller passes every output, so the call allocates nothing
    y = torch.full((cfg.N, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    aux = {k: torch.full_like(v, 3) for k, v in A_ref.items()}
    M.forward_noalloc(x, W, cfg.K, aux=aux, out=y, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), host(y_ref)), "y differs from moe_forward"
    for k, v in A_ref.items():
        if k in ("beta_out", "quantile_out") and not cfg.recompute_bias:
            continue
        assert np.array_equal(host(aux[k]), host(v)), f"{k} differs from moe_forward"


def test_noalloc_matches_forward_twice_second_smaller(M):
    # 1200 tokens: tile engine, shared expert in order on the caller's stream;
    # then 48 tokens: the small-batch kernels
    _check(M, scaled(CONFIGS["prefill"], 1200))
    _check(M, scaled(CONFIGS["decode"], 48))


def test_noalloc_rejects_a_problem_above_the_array(M):
    import torch
    cfg = CONFIGS["prefill"]  # 16384 tokens need about 0.7 GB of workspace
    L = make_inputs(scaled(cfg, 8))
    W = weights_dev(L)
    x = torch.zeros((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")
    say("no-alloc rejects", cfg.N)
    with pytest.raises(M.MoeError, match="WORKSPACE_TOO_SMALL"):
        M.forward_noalloc(x, W, cfg.K, recompute_bias=True)
