#!/usr/bin/env python3
"""Throughput of the MoE layer forward pass on one MI355X.

One step = one call of moe_forward over a resident batch: router logits,
selection, one exact quantile update of the expert bias and re-routing
(when the workload asks for it), grouping by expert, routed and shared
SwiGLU experts and the weighted combine.  The default workload is the
Kolibri-shaped prefill batch (N=16384 tokens, d=2560, E=384, K=6, hidden
512, one shared expert, EQB update on).

Prints one JSON line.  `value` is tokens per second over exactly --steps
timed steps (inputs already in HBM, bracketed by device synchronisation).
The `roofline` entry covers the dominant kernel (the routed gate/up GEMM),
timed with HIP events on the library's stream during the same timed steps;
`cpu_baseline` times the CPU oracle on the same layer (median of 3 runs,
per-step seconds, a single-thread run of the routing steps) and `parity`
records the GPU's outputs of one call against the oracle's on that batch.
`extras` holds the skewed (N=65536, Zipf offsets) and decode (N=64)
workloads measured in the same run after the headline.
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# The CPU baseline's BLAS uses the cores this process may run on (a value
# already set in the environment is kept); set before numpy is imported.
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(host_threads()))

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
_CSRC = os.path.join(ROOT, "sigmoid_top_routing_router_amd", "csrc")


def roofline_kernel(n_tokens, fp8):
    """The kernel the roofline object covers (the routed gate/up GEMM of the
    path the layer takes): (name as rocprofv3 reports it, sources it is built
    from).  Batches of at most 64 tokens take the weight-streaming kernel."""
    if n_tokens <= 64:
        return (f"skinny_kernel<0, {'true' if fp8 else 'false'}>",
                [os.path.join(_CSRC, f) for f in ("skinny_gemm.hip", "gemm_args.h")])
    return ("gemm_fp8_kernel<0>" if fp8 else "gemm_kernel<0, true>",
            [os.path.join(_CSRC, f) for f in ("grouped_gemm.hip", "gemm_args.h")])


def traffic_key(workload, fp8):
    return workload + ("_fp8" if fp8 else "")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(sources) -> str:
    """Hash of a kernel's sources (a traffic record holds for them only)."""
    h = hashlib.sha256()
    for path in sources:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gateup_algorithmic(cfg, counts, fp8=False):
    """Flops and bytes the routed gate/up GEMM must do or move: every pair
    row times both d x h projections; each active expert's gate and up
    weights once, x once, H written once (bf16; with FP8 experts: E4M3 codes
    plus one fp32 scale per 128 x 128 weight block and per 1 x 128 group of
    x and of H).  Batches of at most 64 tokens whose shared expert has the
    routed width run that expert inside the same launch (its tiles follow
    the routed ones): its gate and up weights and its N rows of H count
    too."""
    pairs = cfg.N * cfg.K
    experts = int((counts > 0).sum())
    rows = pairs
    if cfg.N <= 64 and cfg.n_shared == 1 and cfg.h_shared == cfg.h:
        experts += 1
        rows += cfg.N
    flops = 2.0 * rows * (2 * cfg.h) * cfg.d
    if fp8:
        bytes_ = (experts * 2 * (cfg.h * cfg.d + (cfg.h // 128) * (cfg.d // 128) * 4)
                  + cfg.N * cfg.d * (1 + 4 / 128) + rows * cfg.h * (1 + 4 / 128))
    else:
        bytes_ = experts * 2 * cfg.h * cfg.d * 2 + cfg.N * cfg.d * 2 + rows * cfg.h * 2
    return flops, bytes_


def traffic_for(workload, n_tokens, fp8):
    """Recorded HBM bytes per launch of the roofline kernel, or None when no
    record exists or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    ent = t.get(traffic_key(workload, fp8))
    name, sources = roofline_kernel(n_tokens, fp8)
    if not ent or ent.get("kernel_name") != name or \
            ent.get("source_sha256_16") != kernel_source_hash(sources):
        return None
    return ent.get("bytes_per_launch")


COPY_KERNEL = "copyBuffer"


def _counter_means(csv_dir, counter, kernel):
    """Mean per-dispatch value of `counter` (KiB) for `kernel` and the
    largest plain copy in one rocprofv3 --pmc output directory.  Where the
    same kernel also runs a smaller product (the E4M3 tile serves the shared
    expert too), only the dispatches of the largest grid count: the routed
    launch, sized for the worst-case tile table."""
    import csv
    import glob
    gu, cp = [], []
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                if kernel in r["Kernel_Name"]:
                    gu.append((int(r["Grid_Size"]), float(r["Counter_Value"])))
                elif COPY_KERNEL in r["Kernel_Name"]:
                    cp.append(float(r["Counter_Value"]))
    if not gu or not cp:
        raise SystemExit(f"{csv_dir}: no {counter} rows for {kernel} or the copy")
    big = max(g for g, _ in gu)
    vals = [v for g, v in gu if g == big]
    return sum(vals) / len(vals), max(cp), len(vals)


def record_traffic(workload, n_tokens, fp8, fetch_dir, write_dir, copy_mib):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, each with --calibrate-copy-mib) into HBM bytes per launch of
    the roofline kernel (the routed gate/up GEMM of that path).  Each counter
    is scaled by the factor that makes it read the known size of the
    calibration copy (copy_mib MiB read and written)."""
    known_kib = copy_mib * 1024.0
    name, sources = roofline_kernel(n_tokens, fp8)
    f_gu, f_cp, n_f = _counter_means(fetch_dir, "FETCH_SIZE", name)
    w_gu, w_cp, n_w = _counter_means(write_dir, "WRITE_SIZE", name)
    f_scale, w_scale = known_kib / f_cp, known_kib / w_cp
    fetch_b = f_gu * f_scale * 1024.0
    write_b = w_gu * w_scale * 1024.0
    t = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    key = traffic_key(workload, fp8)
    t[key] = {
        "kernel": "routed gate/up GEMM (" + name + ")",
        "kernel_name": name,
        "bytes_per_launch": fetch_b + write_b,
        "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "fetch_kib_raw_mean": f_gu, "write_kib_raw_mean": w_gu,
        "launches": [n_f, n_w],
        "copy_calibration": {"copy_mib": copy_mib, "fetch_kib": f_cp, "write_kib": w_cp,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "source_sha256_16": kernel_source_hash(sources),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t[key]))


def _blas_info():
    """(threads of the BLAS pool, vendor string) from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        pools = []
    if not pools:
        return host_threads(), "unknown"
    threads = max(int(i.get("num_threads", 1)) for i in pools)
    vendor = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in pools)
    return threads, vendor


def cpu_baseline(cfg, L, gpu, runs=3):
    """The CPU baseline leg: the oracle (untuned) on the same inputs.

    * Timing: the whole layer (every step) on the whole batch, `runs` runs,
      median; the per-step seconds of the median run; routing, the quantile
      update and the permutation once more on one thread (on the logits of
      the first run, so the router product is not part of it).  Weight
      decoding to float is excluded.
    * Parity record of the same run: the GPU's outputs of one call on these
      inputs (`gpu`: logits, selections, margins, bias, y) against the
      oracle's, (i) free-running (the oracle on its own logits and bias) and
      (ii) with the GPU's logits given to the oracle (routing compared bit
      for bit, output per token)."""
    import numpy as np
    from oracle import moe_oracle as O
    threads, vendor = _blas_info()
    w = {k: O.bf16_to_f32(getattr(L, k)) for k in
         ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    x = O.bf16_to_f32(L.x)
    kw = dict(beta_in=L.beta_in, K=cfg.K, recompute_bias=cfg.recompute_bias)
    times, steps, own = [], [], None
    for r in range(runs):
        tm = {}
        t0 = time.perf_counter()
        out = O.moe_layer(x=x, **w, logit_offset=L.logit_offset, timings=tm, **kw)
        times.append(time.perf_counter() - t0)
        steps.append(tm)
        if own is None:
            own = out
        log(f"cpu baseline run {r}: {times[-1]:.2f} s")
    med = int(np.argsort(times)[len(times) // 2])
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            tm1 = {}
            O.moe_layer(x=x, **w, logits_in=own["logits"], compute_output=False, timings=tm1,
                        **kw)
    except ImportError:  # pragma: no cover
        tm1 = None
    base = {"value": cfg.N / times[med], "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle, whole layer (all steps) on the whole {cfg.name} batch "
                      f"(N={cfg.N}), median of {runs} runs "
                      f"({', '.join(f'{t:.2f}' for t in times)} s)",
            "runs_s": [round(t, 3) for t in times],
            "steps_s": {k: round(v, 4) for k, v in steps[med].items()},
            "blas": vendor, "threads_env": os.environ.get("OMP_NUM_THREADS")}
    if tm1 is not None:
        t_route = sum(tm1.get(k, 0.0) for k in ("route", "eqb", "permutation"))
        base["single_thread"] = {"what": "routing (both passes, mixture weights), quantile "
                                         "update and permutation on one thread",
                                 "seconds": round(t_route, 4),
                                 "tokens_per_s": cfg.N / t_route,
                                 "steps_s": {k: round(v, 4) for k, v in tm1.items()}}

    # ---- parity record (not timed)
    def per_token(a, b):
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)

    y_gpu = O.bf16_to_f32(gpu["y"])
    Zg = gpu["logits"]
    diff = np.any(np.sort(own["topk_ids"], 1) != np.sort(gpu["topk_ids"], 1), axis=1)
    dz = np.max(np.abs(Zg.astype(np.float64) - own["logits"]), axis=1)
    dbeta = float(np.max(np.abs(gpu["beta_out"].astype(np.float64) - own["beta_out"]))) \
        if cfg.recompute_bias else 0.0
    margin = own["margin"].astype(np.float64)
    allow = 1e-3 + 2.0 * (dz + dbeta)
    rms = np.sqrt(np.mean(own["logits"].astype(np.float64) ** 2, axis=1, keepdims=True))
    zrel = float(np.max(np.abs(Zg - own["logits"]) / np.maximum(np.abs(own["logits"]), rms)))
    pt_free = per_token(y_gpu, own["y"])
    same = ~diff
    forced = O.moe_layer(x=x, **w, logits_in=Zg, **kw)
    pt_forced = per_token(y_gpu, forced["y"])
    bit = {k: bool(np.array_equal(np.asarray(gpu[k]).view(np.uint32) if gpu[k].dtype == np.float32
                                  else gpu[k],
                                  np.asarray(forced[k]).view(np.uint32)
                                  if np.asarray(forced[k]).dtype == np.float32 else forced[k]))
           for k in ("topk_ids", "margin", "counts", "sorted_src")
           + (("beta_out",) if cfg.recompute_bias else ())}
    parity = {
        "tokens": cfg.N,
        "logits_max_rel_err": zrel,
        "free_running": {
            "selection_mismatches": int(diff.sum()),
            "near_ties_margin_below_1e-3": int(np.sum(margin < 1e-3)),
            "max_abs_dbeta": dbeta, "max_abs_dlogit": float(dz.max()),
            "mismatches_beyond_bound": int(np.sum(diff & ~(margin < allow))),
            "y_rel_l2": float(np.linalg.norm(y_gpu - own["y"]) / np.linalg.norm(own["y"])),
            "y_worst_token_rel_l2_same_selection": float(pt_free[same].max()) if same.any() else 0.0,
        },
        "gpu_logits_given": {
            "bit_exact": bit,
            "y_rel_l2": float(np.linalg.norm(y_gpu - forced["y"]) / np.linalg.norm(forced["y"])),
            "y_worst_token_rel_l2": float(pt_forced.max()),
            "tokens_above_2e-2": int(np.sum(pt_forced > 2e-2)),
        },
    }
    return base, parity


def run_extra(M, torch, name, steps, warmup, packed=True, route_fused=False):
    """Another workload of the same layer shape in the same run: step time
    and tokens/s (`steps` timed steps between device synchronisations), and
    the stage times of `steps` further steps (HIP events between stages).
    skewed: the routed expert GEMMs (gate/up + down) as a fraction of the
    bf16 MFMA peak.  decode: the whole layer as GB/s of its algorithmic
    bytes (every touched expert's three matrices once, the shared expert,
    the router, x and y)."""
    import numpy as np
    from synth import CONFIGS, make_inputs
    cfg = CONFIGS[name]
    L = make_inputs(cfg)

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    W = M.ExpertWeights(bf16(L.w_router), bf16(L.w_gate), bf16(L.w_up), bf16(L.w_down),
                        bf16(L.ws_gate), bf16(L.ws_up), bf16(L.ws_down))
    if packed:
        W = M.pack_gateup(W)  # untimed, as at weight-loading time
        torch.cuda.synchronize()
    x = bf16(L.x)
    beta = torch.from_numpy(L.beta_in).cuda()
    off = None if L.logit_offset is None else torch.from_numpy(L.logit_offset).cuda()
    ws = torch.empty(M.forward_workspace_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared,
                                               cfg.h_shared, cfg.recompute_bias),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")
    del L

    def step():
        M.forward(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                  logit_offset=off, workspace=ws, out=y, route_fused=route_fused)

    _, aux = M.forward(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                       logit_offset=off, workspace=ws, out=y, aux=("counts",),
                       route_fused=route_fused)
    counts = aux["counts"].cpu().numpy()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    M.stage_timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    st, calls = M.stage_times()
    M.stage_timing(False)
    st = {k: v / max(calls, 1) for k, v in st.items()}
    out = {"config": cfg.describe(), "steps": steps, "ms_per_step": 1e3 * dt,
           "tokens_per_s": cfg.N / dt,
           "stages_ms": {k: round(v, 4) for k, v in st.items()},
           "max_over_mean_load": float(counts.max() / counts.mean())}
    pairs = cfg.N * cfg.K
    if name == "skewed":
        fl = 2.0 * pairs * 3 * cfg.h * cfg.d
        t = (st["gate_up"] + st["down"]) * 1e-3
        out["routed_gemm"] = {"flops": fl, "ms": 1e3 * t, "tflops": fl / t / 1e12,
                              "mfma_frac": fl / t / 1e12 / PEAK_BF16_TFLOPS,
                              "gate_up_mfma_frac": 2.0 * pairs * 2 * cfg.h * cfg.d
                              / (st["gate_up"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                              "down_mfma_frac": 2.0 * pairs * cfg.h * cfg.d
                              / (st["down"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    if name == "decode":
        touched = int((counts > 0).sum())
        nbytes = ((touched * 3 * cfg.h * cfg.d + cfg.n_shared * 3 * cfg.h_shared * cfg.d
                   + cfg.E * cfg.d) * 2 + 2 * cfg.N * cfg.d * 2)
        out["layer_hbm"] = {"algorithmic_bytes": nbytes, "experts_touched": touched,
                            "gbs": nbytes / dt / 1e9,
                            "frac": nbytes / dt / 1e9 / PEAK_HBM_GBS}
    log(name, json.dumps(out))
    return out


def bench_parts(M, torch, cfg, Z, beta, iters):
    """Standalone timing of the routing steps through the C-ABI: moe_route
    (selection, weights, token bias) and moe_eqb_bias (one exact quantile
    update: histogram zeroing, two radix passes over the logits, scans,
    centring) on the workload's own logits.  Each sample brackets one call
    with HIP events on the current stream.  "warm": a spin kernel before the
    first event keeps the GPU busy while the host enqueues, so the events
    time the call alone, with the logits possibly in the 256 MB MALL.
    "cold": a read of a 1 GiB device buffer before each sample evicts the
    caches (with clean lines, so no write-back of the flush lands inside the
    sample), and the logits come from HBM.  Reports median, p10 and p90 over `iters` samples,
    and GB/s of the algorithmic bytes: (4E + 8K + 8) per token for
    moe_route (logits read; ids, weights, alpha, margin written) and
    2 (4E + 4) per token for moe_eqb_bias (logits and alpha read once per
    radix pass)."""
    import ctypes
    import numpy as np
    from sigmoid_top_routing_router_amd import _lib
    lib = _lib.load()
    N, E, K = cfg.N, cfg.E, cfg.K
    dev = Z.device
    ids = torch.empty((N, K), dtype=torch.int32, device=dev)
    w = torch.empty((N, K), dtype=torch.float32, device=dev)
    alpha = torch.empty((N,), dtype=torch.float32, device=dev)
    margin = torch.empty((N,), dtype=torch.float32, device=dev)
    beta_out = torch.empty((E,), dtype=torch.float32, device=dev)
    q = torch.empty((E,), dtype=torch.float32, device=dev)
    ws_n = max(int(lib.moe_eqb_workspace_bytes(N, E, 16)), 256)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    scratch = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def call_route():
        _lib.check(lib.moe_route(p(Z), p(beta), N, E, K, p(ids), p(w), p(alpha), p(margin), st))

    def call_eqb():
        _lib.check(lib.moe_eqb_bias(p(Z), p(beta), p(alpha), N, E, K, 16, p(beta_out), p(q),
                                    p(ws), ws_n, st))

    parts = [("moe_route", call_route, (4 * E + 8 * K + 8) * N),
             ("moe_eqb_bias", call_eqb, 2 * (4 * E + 4) * N)]
    call_route()  # alpha for the quantile update
    torch.cuda.synchronize()
    out = []
    for name, fn, nbytes in parts:
        for mode in ("warm", "cold"):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(iters)]
            for e0, e1 in ev:
                if mode == "cold":
                    scratch.max()
                else:
                    torch.cuda._sleep(100000)
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            us = np.array([1e3 * e0.elapsed_time(e1) for e0, e1 in ev])
            med = float(np.median(us))
            out.append({"part": name, "mode": mode, "median_us": round(med, 2),
                        "p10_us": round(float(np.percentile(us, 10)), 2),
                        "p90_us": round(float(np.percentile(us, 90)), 2),
                        "bytes": nbytes, "gbs": round(nbytes / med / 1e3, 1),
                        "hbm_frac": round(nbytes / med / 1e3 / PEAK_HBM_GBS, 3)})
            log(json.dumps(out[-1]))
    del scratch
    return out


def library_ceilings(torch):
    """Reference points of this GPU measured with the vendor libraries through
    torch (hipBLASLt GEMMs, the runtime's copy): dense bf16 GEMMs, the routed
    GEMMs' shapes as plain dense or batched products (no gather, uniform
    experts), and a device copy.  Context for the kernels' fractions of the
    datasheet peaks; none of it is part of the layer."""
    dev = "cuda"
    torch.manual_seed(0)

    def timed(fn, it, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(it):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / it

    out = {}
    for m, n, k, what in [(8192, 8192, 8192, "square"),
                          (16384, 16384, 4096, "large"),
                          (65536, 2560, 512, "the down projection's shape (k 512, n 2560) as one "
                                             "dense GEMM of 65,536 rows"),
                          (16384, 1024, 2560, "gate/up of one 16,384-token shared expert")]:
        A = torch.randn(m, k, device=dev, dtype=torch.bfloat16)
        B = torch.randn(k, n, device=dev, dtype=torch.bfloat16)
        ms = timed(lambda: A @ B, 20, 5)
        out[f"gemm_bf16_{m}x{n}x{k}"] = {"what": what, "ms": round(ms, 4),
                                         "tflops": round(2 * m * n * k / ms / 1e9, 1),
                                         "frac": round(2 * m * n * k / ms / 1e9 / PEAK_BF16_TFLOPS, 3)}
        log(json.dumps(out))
        del A, B
    E, rows = 384, 1024
    A = torch.randn(E, rows, 2560, device=dev, dtype=torch.bfloat16)
    B = torch.randn(E, 2560, 1024, device=dev, dtype=torch.bfloat16)
    ms = timed(lambda: torch.bmm(A, B), 5, 2)
    fl = 2 * E * rows * 1024 * 2560
    out["bmm_bf16_384x1024x1024x2560"] = {
        "what": "gate/up of 384 experts with 1,024 rows each, batched, no gather",
        "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
        "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 3)}
    del A, B
    X = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    Y = torch.empty_like(X)
    ms = timed(lambda: Y.copy_(X), 10, 2)
    out["copy_2GiB"] = {"what": "device copy, bytes read + written", "ms": round(ms, 4),
                        "gbs": round(2 * X.numel() / ms / 1e6, 1),
                        "frac": round(2 * X.numel() / ms / 1e6 / PEAK_HBM_GBS, 3)}
    del X, Y
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["origin", "prefill", "decode", "skewed"])
    ap.add_argument("--cpu-runs", type=int, default=3,
                    help="runs of the CPU oracle (median reported)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the skewed and decode workloads measured after the headline")
    ap.add_argument("--row-major", action="store_true",
                    help="routed gate/up weights in the row-major layout instead of the "
                         "packed one (moe_pack_gateup_weights)")
    ap.add_argument("--fp8", action="store_true",
                    help="E4M3 experts (moe_forward_fp8) quantised from the same bf16 weights")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling hardware byte counters)")
    ap.add_argument("--inference", action="store_true",
                    help="route with the given bias only (no quantile update in the step), "
                         "the layer as inference runs it")
    ap.add_argument("--route-fused", action="store_true",
                    help="select the experts inside the router GEMM's epilogue "
                         "(MOE_ROUTE_FUSED) instead of in a pass of their own")
    ap.add_argument("--parts", action="store_true",
                    help="instead of the layer: time moe_route and moe_eqb_bias alone on the "
                         "workload's logits (warm and cold, median/p10/p90 of --steps samples)")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the layer: time vendor-library GEMMs of related shapes "
                         "and a device copy on this GPU (reference points for the fractions)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: write the routed gate/up HBM bytes per launch from two "
                         "rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) of "
                         "this script run with --calibrate-copy-mib")
    args = ap.parse_args()
    if args.record_traffic:
        from synth import CONFIGS
        record_traffic(args.workload, CONFIGS[args.workload].N, args.fp8, *args.record_traffic,
                       args.calibrate_copy_mib or 1024)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer has no multi-GPU path "
              "(no expert or data sharding across devices); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sigmoid_top_routing_router_amd as M
    from synth import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.ceilings:
        print(json.dumps({"metric": "vendor-library reference points", "gpu":
                          torch.cuda.get_device_name(0), "results": library_ceilings(torch)}))
        return
    M.load_library()
    cfg = CONFIGS[args.workload]
    if args.inference:
        from dataclasses import replace
        cfg = replace(cfg, recompute_bias=False)
    log("workload", cfg.describe())
    L = make_inputs(cfg)
    log("inputs ready")

    def bf16(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    W = M.ExpertWeights(bf16(L.w_router), bf16(L.w_gate), bf16(L.w_up), bf16(L.w_down),
                        bf16(L.ws_gate), bf16(L.ws_up), bf16(L.ws_down))
    fwd, ws_fn = M.forward, M.forward_workspace_bytes
    if args.route_fused:
        fwd = functools.partial(fwd, route_fused=True)
    if args.fp8:
        # E4M3 experts quantised from the bf16 weights by the library (untimed)
        W = M.quantize_experts(W)
        torch.cuda.synchronize()
        fwd, ws_fn = M.forward_fp8, M.forward_fp8_workspace_bytes
        if args.route_fused:
            fwd = functools.partial(fwd, route_fused=True)
    if not args.row_major:
        # the routed gate/up weights in the library's packed layout, as a
        # deployment stores them (untimed; the results are bit-identical)
        W = M.pack_gateup(W)
        torch.cuda.synchronize()
        log("gate/up weights packed")
    x = bf16(L.x)
    beta = torch.from_numpy(L.beta_in).cuda()
    off = None if L.logit_offset is None else torch.from_numpy(L.logit_offset).cuda()
    ws_bytes = ws_fn(cfg.N, cfg.d, cfg.E, cfg.K, cfg.h, cfg.n_shared, cfg.h_shared,
                     cfg.recompute_bias)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.N, cfg.d), dtype=torch.bfloat16, device="cuda")

    def step():
        fwd(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
            logit_offset=off, workspace=ws, out=y)

    if args.parts:
        _, aux = fwd(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                     logit_offset=off, workspace=ws, out=y, aux=("logits",))
        del ws, y
        parts = bench_parts(M, torch, cfg, aux["logits"], beta, max(args.steps, 20))
        print(json.dumps({"metric": "routing steps alone (HIP events per call)",
                          "config": cfg.describe(), "samples": max(args.steps, 20),
                          "parts": parts}), flush=True)
        return

    # loads of the final routing (for the algorithmic byte count) and the
    # outputs the parity record compares with the oracle, untimed
    aux_names = ("counts", "counts_before", "logits", "topk_ids", "margin", "sorted_src") \
        + (("beta_out",) if cfg.recompute_bias else ())
    _, aux = fwd(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                 logit_offset=off, workspace=ws, out=y, aux=aux_names)
    gpu_out = {k: v.cpu().numpy() for k, v in aux.items()}
    gpu_out["y"] = y.view(torch.int16).cpu().numpy().view(np.uint16)
    del aux
    counts = gpu_out["counts"]
    counts_before = gpu_out["counts_before"]
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {n} bytes done")
    log("first call done; warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timed steps")

    # Stage breakdown (every stage boundary timed), untimed steps
    M.stage_timing(True)
    for _ in range(max(3, min(args.steps, 10))):
        step()
    torch.cuda.synchronize()
    stages, calls = M.stage_times()
    stage_ms = {k: v / max(calls, 1) for k, v in stages.items()}
    log("stage ms", json.dumps({k: round(v, 4) for k, v in stage_ms.items()}))

    # Timed steps: only the two events around the routed gate/up GEMM are
    # recorded (for its roofline), so the stream is barely disturbed
    M.stage_timing(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gu_times, gu_calls = M.stage_times()
    M.stage_timing(False)
    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / args.steps
    tokens_s = cfg.N * args.steps / elapsed
    gateup_ms = gu_times["gate_up"] / max(gu_calls, 1)

    flops, bytes_ = gateup_algorithmic(cfg, counts, args.fp8)
    peak_mfma = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    t_gu = gateup_ms * 1e-3
    t_mfma = flops / (peak_mfma * 1e12)
    t_hbm = bytes_ / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": bytes_ / t_gu / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_gu / 1e12, "peak": peak_mfma,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the traffic records are taken with the default (packed) layout and the
    # quantile update inside the step (other loads move other bytes)
    roof["traffic"] = None if (args.row_major or args.inference) else \
        traffic_for(args.workload, cfg.N, args.fp8)
    kname, _ = roofline_kernel(cfg.N, args.fp8)
    roof["kernel"] = kname + (" (routed gate/up GEMM, weight-streaming)" if cfg.N <= 64 else
                              " (routed gate/up GEMM, E4M3)" if args.fp8 else
                              " (routed gate/up GEMM)")
    roof["per_launch"] = {"flops": flops, "bytes": bytes_, "avg_ms": gateup_ms,
                          "tflops": flops / t_gu / 1e12, "gbs": bytes_ / t_gu / 1e9,
                          "mfma_frac": flops / t_gu / 1e12 / peak_mfma}

    layer_flops = 2.0 * cfg.N * cfg.E * cfg.d + 2.0 * cfg.N * cfg.K * 3 * cfg.h * cfg.d \
        + 2.0 * cfg.N * cfg.n_shared * 3 * cfg.h_shared * cfg.d
    out = {
        "metric": "MoE layer fwd tokens/s at E=384,K=6,d=2560 (1 GPU); % MFMA / HBM roofline",
        "value": tokens_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 experts (bf16 router)" if args.fp8 else "bf16",
        "data": "synthetic (seeded normal inputs and random-init weights of the layer shape)",
        "config": {**cfg.describe(), "parallelism": "none (1 GPU)",
                   **({"experts": "e4m3, 128x128 block scales, 1x128 activation groups"}
                      if args.fp8 else {}),
                   "gate_up_weights": "row-major" if args.row_major else
                   "packed k-block-major (moe_pack_gateup_weights, untimed)",
                   "selection": "fused into the router GEMM (merge kernel after it)"
                   if args.route_fused else "separate pass over the logits"},
        "layer_tflops": layer_flops / (ms_step * 1e-3) / 1e12,
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "loads": {"max_over_mean_before": float(counts_before.max() / counts_before.mean()),
                  "max_over_mean_after": float(counts.max() / counts.mean())},
        "roofline": roof,
    }
    if not args.no_extras and args.workload == "prefill" and not args.fp8 \
            and not args.inference:
        del ws, y, x, W
        torch.cuda.empty_cache()
        out["extras"] = {n: run_extra(M, torch, n, s, 3, not args.row_major,
                                         args.route_fused)
                         for n, s in (("skewed", 10), ("decode", 50))}
    if not args.no_cpu_baseline and not args.fp8:
        log("cpu baseline ...")
        out["cpu_baseline"], out["parity"] = cpu_baseline(cfg, L, gpu_out, args.cpu_runs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
