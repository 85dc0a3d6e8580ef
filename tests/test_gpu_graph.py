"""moe_forward under HIP graph capture: the whole layer (router, routing with
the bias update, grouping, experts, combine) is captured once on a stream and
replayed; every replay, with eager work and synchronisations in between, is
bit-identical to the eager call (the path is deterministic, uses fill kernels
instead of memsets and never synchronises with the host).  With bf16 and
with E4M3 experts; above 64 tokens the capture also records the shared
expert's branch on the library's side stream."""
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


@pytest.mark.parametrize("name,N,fp8", [("prefill", 3000, False), ("decode", None, False),
                                        ("skewed", 2048, False), ("prefill", 3000, True),
                                        ("decode", None, True)])
def test_forward_graph_replay_matches_eager(M, name, N, fp8):
    import torch
    cfg = CONFIGS[name] if N is None else scaled(CONFIGS[name], N)
    say("graph", cfg.name, cfg.N, "fp8" if fp8 else "bf16")
    L = make_inputs(cfg)
    W = weights_dev(L)
    fwd, ws_fn = M.forward, M.forward_workspace_bytes
    if fp8:
        W = M.quantize_experts(W)
        fwd, ws_fn = M.forward_fp8, M.forward_fp8_workspace_bytes
    x = bf16_dev(L.x)
    beta = dev(L.beta_in)
    off = dev(L.logit_offset)
    ws = torch.empty(ws_fn(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared, cfg.h_shared,
                           cfg.recompute_bias),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")

    def run():
        fwd(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
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


def test_forward_threads_and_streams(M):
    """Above 64 tokens the shared expert runs on a library-owned side stream
    per device and host thread, forked from the caller's stream and joined
    back before the combine.  Two host threads, each on its own stream with
    its own workspace, and calls on the default stream must all give the
    single-call result, every call only ordered by its own stream."""
    import threading

    import torch
    cfg = scaled(CONFIGS["prefill"], 1500)
    say("threads and streams", cfg.name, cfg.N)
    L = make_inputs(cfg)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    beta = dev(L.beta_in)
    off = dev(L.logit_offset)
    nbytes = M.forward_workspace_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared,
                                       cfg.h_shared, cfg.recompute_bias)

    def call(ws, y):
        M.forward(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                  logit_offset=off, workspace=ws, out=y)

    ws0 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y0 = torch.empty((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")
    call(ws0, y0)
    torch.cuda.synchronize()
    ref = host(y0).copy()

    outs, errors = [None, None], []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            y = torch.empty((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")
            with torch.cuda.stream(s):
                for _ in range(3):
                    y.zero_()
                    call(ws, y)
            s.synchronize()
            outs[i] = host(y).copy()
        except Exception as e:  # reported below, on the test's thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for _ in range(3):
        y0.zero_()
        call(ws0, y0)  # the main thread keeps working on the default stream
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert np.array_equal(host(y0), ref)
    for i in range(2):
        assert np.array_equal(outs[i], ref), f"thread {i} differs"


def test_explicit_stream_argument(M):
    """forward, eqb_bias and lei_backward with stream= a stream that is not
    the current one: the binding allocates the outputs and temporaries of the
    call on that stream, so the caching allocator cannot hand their memory to
    work on the current stream while the call's kernels still run.  The
    current stream is kept busy with allocations and writes of the same sizes
    meanwhile; every result must equal the plain call's."""
    import torch
    cfg = scaled(CONFIGS["prefill"], 1500)
    say("explicit stream argument", cfg.name, cfg.N)
    L = make_inputs(cfg)
    W = weights_dev(L)
    x = bf16_dev(L.x)
    beta = dev(L.beta_in)
    kw = dict(beta_in=beta, recompute_bias=True, aux=("logits", "topk_ids"))
    y_ref, A = M.forward(x, W, cfg.K, **kw)
    Z = A["logits"]
    b_ref, q_ref = M.eqb_bias(Z, cfg.K, beta_in=beta)
    g_ref = M.lei_backward(A["topk_ids"], cfg.E, logits=Z)
    torch.cuda.synchronize()
    refs = [host(y_ref), host(b_ref), host(q_ref)] + [host(t) for t in g_ref]
    nbytes = M.forward_workspace_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared,
                                       cfg.h_shared, True)
    s = torch.cuda.Stream()
    for rep in range(3):
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda._sleep(2_000_000)  # the current stream runs behind the side stream
        y, _ = M.forward(x, W, cfg.K, stream=s, **kw)
        b, q = M.eqb_bias(Z, cfg.K, beta_in=beta, stream=s)
        g = M.lei_backward(A["topk_ids"], cfg.E, logits=Z, stream=s)
        # work on the current stream that would reuse freed temporaries
        junk = [torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(2)]
        del junk
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        got = [host(y), host(b), host(q)] + [host(t) for t in g]
        for i, (a, r) in enumerate(zip(got, refs)):
            assert np.array_equal(a, r), f"result {i} differs on repetition {rep}"
