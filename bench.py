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
`cpu_baseline` times the CPU oracle on a bounded sample of the same layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
GEMM_SRC = [os.path.join(ROOT, "sigmoid_top_routing_router_amd", "csrc", f)
            for f in ("grouped_gemm.hip", "gemm_args.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the tile engine's sources (the kernel the traffic record covers)."""
    h = hashlib.sha256()
    for path in GEMM_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gateup_algorithmic(cfg, counts, fp8=False):
    """Flops and bytes the routed gate/up GEMM must do or move: every pair
    row times both d x h projections; each active expert's gate and up
    weights once, x once, H written once (bf16; with FP8 experts: E4M3 codes
    plus one fp32 scale per 128 x 128 weight block and per 1 x 128 group of
    x and of H)."""
    pairs = cfg.N * cfg.K
    flops = 2.0 * pairs * (2 * cfg.h) * cfg.d
    active = int((counts > 0).sum())
    if fp8:
        bytes_ = (active * 2 * (cfg.h * cfg.d + (cfg.h // 128) * (cfg.d // 128) * 4)
                  + cfg.N * cfg.d * (1 + 4 / 128) + pairs * cfg.h * (1 + 4 / 128))
    else:
        bytes_ = active * 2 * cfg.h * cfg.d * 2 + cfg.N * cfg.d * 2 + pairs * cfg.h * 2
    return flops, bytes_


def traffic_for(workload):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    ent = t.get(workload)
    if not ent or ent.get("source_sha256_16") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


ROUTED_GATEUP = "gemm_kernel<0, true>"
COPY_KERNEL = "copyBuffer"


def _counter_means(csv_dir, counter):
    """Mean per-dispatch value of `counter` (KiB) for the routed gate/up kernel
    and the largest plain copy in one rocprofv3 --pmc output directory."""
    import csv
    import glob
    gu, cp = [], []
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                if ROUTED_GATEUP in r["Kernel_Name"]:
                    gu.append(float(r["Counter_Value"]))
                elif COPY_KERNEL in r["Kernel_Name"]:
                    cp.append(float(r["Counter_Value"]))
    if not gu or not cp:
        raise SystemExit(f"{csv_dir}: no {counter} rows for the routed gate/up kernel or the copy")
    return sum(gu) / len(gu), max(cp), len(gu)


def record_traffic(workload, fetch_dir, write_dir, copy_mib):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, each with --calibrate-copy-mib) into HBM bytes per launch of
    the routed gate/up GEMM.  Each counter is scaled by the factor that makes
    it read the known size of the calibration copy (copy_mib MiB read and
    written)."""
    known_kib = copy_mib * 1024.0
    f_gu, f_cp, n_f = _counter_means(fetch_dir, "FETCH_SIZE")
    w_gu, w_cp, n_w = _counter_means(write_dir, "WRITE_SIZE")
    f_scale, w_scale = known_kib / f_cp, known_kib / w_cp
    fetch_b = f_gu * f_scale * 1024.0
    write_b = w_gu * w_scale * 1024.0
    t = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    t[workload] = {
        "kernel": "routed gate/up GEMM (" + ROUTED_GATEUP + ")",
        "bytes_per_launch": fetch_b + write_b,
        "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "fetch_kib_raw_mean": f_gu, "write_kib_raw_mean": w_gu,
        "launches": [n_f, n_w],
        "copy_calibration": {"copy_mib": copy_mib, "fetch_kib": f_cp, "write_kib": w_cp,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "source_sha256_16": kernel_source_hash(),
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    print(json.dumps(t[workload]))


def cpu_baseline(cfg, L, sample_tokens):
    """The oracle (untuned) timed on a bounded sample: the whole layer for
    the first `sample_tokens` tokens of the same inputs (the quantile update
    runs over that sample batch).  Weight decoding to float is excluded."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    n = min(sample_tokens, cfg.N)
    w = {k: O.bf16_to_f32(getattr(L, k)) for k in
         ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    x = O.bf16_to_f32(L.x[:n])
    t0 = time.perf_counter()
    O.moe_layer(x=x, **w, beta_in=L.beta_in, K=cfg.K, recompute_bias=cfg.recompute_bias,
                logit_offset=L.logit_offset)
    dt = time.perf_counter() - t0
    what = "the whole batch" if n == cfg.N else f"the first {n} of {cfg.N} tokens"
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle, whole layer (all steps) on {what} of the {cfg.name} "
                      f"workload, one run of {dt:.1f} s"}


def bench_parts(M, torch, cfg, Z, beta, iters):
    """Standalone timing of the routing steps through the C-ABI: moe_route
    (selection, weights, token bias) and moe_eqb_bias (one exact quantile
    update: histogram zeroing, two radix passes over the logits, scans,
    centring) on the workload's own logits.  Each sample brackets one call
    with HIP events on the current stream.  "warm": a spin kernel before the
    first event keeps the GPU busy while the host enqueues, so the events
    time the call alone, with the logits possibly in the 256 MB MALL.
    "cold": a 1 GiB device fill before each sample evicts the caches, so the
    logits come from HBM.  Reports median, p10 and p90 over `iters` samples,
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
    ws_n = max(int(lib.moe_eqb_workspace_bytes(N, E, K, 16)), 256)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
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
                    scratch.fill_(1)
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["origin", "prefill", "decode", "skewed"])
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="E4M3 experts (moe_forward_fp8) quantised from the same bf16 weights")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling hardware byte counters)")
    ap.add_argument("--inference", action="store_true",
                    help="route with the given bias only (no quantile update in the step), "
                         "the layer as inference runs it")
    ap.add_argument("--parts", action="store_true",
                    help="instead of the layer: time moe_route and moe_eqb_bias alone on the "
                         "workload's logits (warm and cold, median/p10/p90 of --steps samples)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: write the routed gate/up HBM bytes per launch from two "
                         "rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) of "
                         "this script run with --calibrate-copy-mib")
    args = ap.parse_args()
    if args.fp8 and (args.record_traffic or args.calibrate_copy_mib):
        ap.error("--fp8 has no traffic record")
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic, args.calibrate_copy_mib or 1024)
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
    if args.fp8:
        # E4M3 experts quantised from the bf16 weights by the library (untimed)
        W = M.quantize_experts(W)
        torch.cuda.synchronize()
        fwd, ws_fn = M.forward_fp8, M.forward_fp8_workspace_bytes
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

    # loads of the final routing (for the algorithmic byte count), untimed
    _, aux = fwd(x, W, cfg.K, beta_in=beta, recompute_bias=cfg.recompute_bias,
                 logit_offset=off, workspace=ws, out=y, aux=("counts", "counts_before"))
    counts = aux["counts"].cpu().numpy()
    counts_before = aux["counts_before"].cpu().numpy()
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
    roof["traffic"] = None if args.fp8 else traffic_for(args.workload)
    if cfg.N <= 64:  # batches of at most 64 tokens take the weight-streaming kernel
        roof["kernel"] = (f"skinny_kernel<0, {'true' if args.fp8 else 'false'}> "
                          "(routed gate/up GEMM, weight-streaming)")
    else:
        roof["kernel"] = ("gemm_fp8_kernel<0> (routed gate/up GEMM, E4M3)" if args.fp8
                          else "gemm_kernel<0, true> (routed gate/up GEMM)")
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
                      if args.fp8 else {})},
        "layer_tflops": layer_flops / (ms_step * 1e-3) / 1e12,
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "loads": {"max_over_mean_before": float(counts_before.max() / counts_before.mean()),
                  "max_over_mean_after": float(counts.max() / counts.mean())},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(cfg, L, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
