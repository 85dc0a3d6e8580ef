"""moe_forward under HIP graph capture: the whole layer (router, routing with
the bias update, grouping, experts, combine) is captured once on a stream and
replayed; every replay, with eager work and synchronisations in between, is
bit-identical to the eager call (the path is deterministic, uses fill kernels
instead of memsets and never synchronises with the host)."""
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


@pytest.mark.parametrize("name,N", [("prefill", 3000), ("decode", None), ("skewed", 2048)])
def test_forward_graph_replay_matches_eager(M, name, N):
    import torch
    cfg = CONFIGS[name] if N is None else scaled(CONFIGS[name], N)
    say("graph", cfg.name, cfg.N)
    L = make_inputs(cfg)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    beta = dev(L.beta_in)
    off = dev(L.logit_offset)
    ws = torch.empty(M.forward_workspace_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared,
                                               cfg.h_shared, cfg.recompute_bias),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((cfg.N, cfg.K), dtype=torch.int32, device="cuda")

    def run():
        M.forward(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                  logit_offset=off, workspace=ws, out=y)

    run()  # warm up (kernel attributes, occupancy queries) outside the capture
    torch.cuda.synchronize()
    ref = host(y).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        ws.fill_(0xA5)  # the replay must not depend on workspace contents
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref), f"replay {rep} differs"
        run()  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref)
