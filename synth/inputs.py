"""Seeded synthetic inputs for the MoE layer workloads.

Both sides of every parity check (the CPU oracle and the HIP library) receive
the same bit patterns from here.  This module only draws random numbers and
stores them; none of the layer's arithmetic lives here.

Recipe
------
* Root: ``SeedSequence(cfg.seed)``, spawned into 8 tensor streams in the fixed
  order [x, w_router, beta, w_gate, w_up, w_down, shared, spare].
* Every tensor is drawn in slabs; slab ``i`` uses child ``i`` of its stream's
  SeedSequence, with a PCG64 generator and float32 standard normals, so the
  draw does not depend on how many threads fill it.  Slabs: one expert for the
  expert weights, 4096 rows for x, the whole tensor otherwise.  The shared
  stream is split into 3 children (gate, up, down), each drawn per shared
  expert.
* x ~ N(0, x_std^2), weights ~ N(0, w_std^2), beta ~ N(0, beta_std^2); the
  products with the std are taken in float32, then rounded to bfloat16 with
  round-to-nearest-even (torch's CPU conversion) and stored as raw uint16
  bits.  The toy workload keeps float32 values as well.
* FP8 experts (``make_fp8_experts``): a synthetic E4M3 checkpoint drawn
  from ``SeedSequence([cfg.seed, 8])`` spawned into 6 streams [gate, up, down,
  shared gate, shared up, shared down], one child per expert.  Each code has a
  uniform sign, an exponent field in 9..15 with probabilities
  (.05 .10 .15 .25 .25 .15 .05) and a uniform 3-bit mantissa (magnitudes 4 to
  448, the NaN pattern replaced by 448); each 128 x 128 block scale is
  float32(w_std / 100 * exp(0.3 z)), z standard normal.
* Logit offsets (an input knob, added to the logits before the bias):
  "toy_collapse" adds +3 to experts 0 and 1 so that routing collapses onto
  them as in the running example; "zipf1.2" adds float32(0.5*ln p_e) with
  p_e proportional to (e+1)^-1.2, expert-id order.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import LayerConfig

X_SLAB_ROWS = 4096
_STREAMS = ["x", "w_router", "beta", "w_gate", "w_up", "w_down", "shared", "spare"]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round-to-nearest-even, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal(seed_seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed_seq))
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray            # [N, d]   bf16 bits (uint16)
    w_router: np.ndarray     # [E, d]   bf16 bits
    beta_in: np.ndarray      # [E]      float32
    w_gate: np.ndarray       # [E, h, d] bf16 bits
    w_up: np.ndarray         # [E, h, d] bf16 bits
    w_down: np.ndarray       # [E, d, h] bf16 bits
    ws_gate: np.ndarray      # [S, hs, d] bf16 bits
    ws_up: np.ndarray        # [S, hs, d] bf16 bits
    ws_down: np.ndarray      # [S, d, hs] bf16 bits
    logit_offset: Optional[np.ndarray]  # [E] float32 or None
    f32: Optional[dict] = None  # float32 originals (toy workload only)


def _expert_tensor(ss: np.random.SeedSequence, E: int, rows: int, cols: int,
                   std: float, keep_f32: bool):
    out = np.empty((E, rows, cols), dtype=np.uint16)
    f32 = np.empty((E, rows, cols), dtype=np.float32) if keep_f32 else None
    kids = ss.spawn(E)

    def fill(e):
        a = _normal(kids[e], (rows, cols), std)
        out[e] = to_bf16_bits(a)
        if f32 is not None:
            f32[e] = a

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    return out, f32


_FP8_EXP_FIELDS = np.arange(9, 16)
_FP8_EXP_P = np.array([0.05, 0.10, 0.15, 0.25, 0.25, 0.15, 0.05])


def _fp8_tensor(ss: np.random.SeedSequence, E: int, rows: int, cols: int, std: float):
    codes = np.empty((E, rows, cols), dtype=np.uint8)
    scales = np.empty((E, -(-rows // 128), -(-cols // 128)), dtype=np.float32)
    kids = ss.spawn(E)

    def fill(e):
        g = np.random.Generator(np.random.PCG64(kids[e]))
        sign = g.integers(0, 2, (rows, cols), dtype=np.uint8)
        ef = g.choice(_FP8_EXP_FIELDS, size=(rows, cols), p=_FP8_EXP_P).astype(np.uint8)
        man = g.integers(0, 8, (rows, cols), dtype=np.uint8)
        man[(ef == 15) & (man == 7)] = 6
        codes[e] = (sign << 7) | (ef << 3) | man
        scales[e] = (std / 100.0 * np.exp(0.3 * g.standard_normal(scales.shape[1:]))).astype(
            np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    return codes, scales


def make_fp8_experts(cfg: LayerConfig) -> dict:
    """Synthetic E4M3 expert weights of cfg's shapes: codes and 128 x 128
    block scales under the names w_gate/s_gate, w_up/s_up, w_down/s_down,
    ws_gate/ss_gate, ws_up/ss_up, ws_down/ss_down."""
    st = np.random.SeedSequence([cfg.seed, 8]).spawn(6)
    out = {}
    shapes = [("w_gate", "s_gate", cfg.E, cfg.h, cfg.d), ("w_up", "s_up", cfg.E, cfg.h, cfg.d),
              ("w_down", "s_down", cfg.E, cfg.d, cfg.h),
              ("ws_gate", "ss_gate", cfg.n_shared, cfg.h_shared, cfg.d),
              ("ws_up", "ss_up", cfg.n_shared, cfg.h_shared, cfg.d),
              ("ws_down", "ss_down", cfg.n_shared, cfg.d, cfg.h_shared)]
    for ss, (cn, sn, E, r, c) in zip(st, shapes):
        out[cn], out[sn] = _fp8_tensor(ss, E, r, c, cfg.w_std)
    return out


def logit_offset_for(cfg: LayerConfig) -> Optional[np.ndarray]:
    if cfg.offset is None:
        return None
    if cfg.offset == "toy_collapse":
        off = np.zeros(cfg.E, dtype=np.float32)
        off[:2] = 3.0
        return off
    if cfg.offset == "zipf1.2":
        w = np.array([(e + 1) ** -1.2 for e in range(cfg.E)], dtype=np.float64)
        p = w / w.sum()
        return np.array([0.5 * math.log(v) for v in p], dtype=np.float32)
    raise ValueError(f"unknown offset kind {cfg.offset!r}")


def make_inputs(cfg: LayerConfig) -> LayerInputs:
    root = np.random.SeedSequence(cfg.seed)
    s = dict(zip(_STREAMS, root.spawn(len(_STREAMS))))
    keep = cfg.dtype == "fp32"

    # x, in slabs of X_SLAB_ROWS rows
    n_slabs = max(1, -(-cfg.N // X_SLAB_ROWS))
    kids = s["x"].spawn(n_slabs)
    x = np.empty((cfg.N, cfg.d), dtype=np.uint16)
    x32 = np.empty((cfg.N, cfg.d), dtype=np.float32) if keep else None

    def fill_x(i):
        r0 = i * X_SLAB_ROWS
        r1 = min(cfg.N, r0 + X_SLAB_ROWS)
        a = _normal(kids[i], (r1 - r0, cfg.d), cfg.x_std)
        x[r0:r1] = to_bf16_bits(a)
        if x32 is not None:
            x32[r0:r1] = a

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill_x, range(n_slabs)))

    wr32 = _normal(s["w_router"].spawn(1)[0], (cfg.E, cfg.d), cfg.w_std)
    w_router = to_bf16_bits(wr32)
    if cfg.beta_std > 0:
        beta = _normal(s["beta"].spawn(1)[0], (cfg.E,), cfg.beta_std)
    else:
        beta = np.zeros(cfg.E, dtype=np.float32)

    w_gate, g32 = _expert_tensor(s["w_gate"], cfg.E, cfg.h, cfg.d, cfg.w_std, keep)
    w_up, u32 = _expert_tensor(s["w_up"], cfg.E, cfg.h, cfg.d, cfg.w_std, keep)
    w_down, d32 = _expert_tensor(s["w_down"], cfg.E, cfg.d, cfg.h, cfg.w_std, keep)

    sg, su, sd = s["shared"].spawn(3)
    S = cfg.n_shared
    ws_gate, sg32 = _expert_tensor(sg, S, cfg.h_shared, cfg.d, cfg.w_std, keep)
    ws_up, su32 = _expert_tensor(su, S, cfg.h_shared, cfg.d, cfg.w_std, keep)
    ws_down, sd32 = _expert_tensor(sd, S, cfg.d, cfg.h_shared, cfg.w_std, keep)

    f32 = None
    if keep:
        f32 = dict(x=x32, w_router=wr32, w_gate=g32, w_up=u32, w_down=d32,
                   ws_gate=sg32, ws_up=su32, ws_down=sd32)
    return LayerInputs(cfg, x, w_router, beta, w_gate, w_up, w_down,
                       ws_gate, ws_up, ws_down, logit_offset_for(cfg), f32)


def make_logits(seed: int, N: int, E: int, std: float = 1.0,
                tie_fraction: float = 0.0) -> np.ndarray:
    """Free-standing float32 logits [N, E] for routing and quantile cases.

    ``tie_fraction`` > 0 snaps that fraction of the entries onto a coarse grid
    (multiples of 1/8), which plants exact ties, repeated values and zeros of
    both signs.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    z = g.standard_normal((N, E), dtype=np.float32) * np.float32(std)
    if tie_fraction > 0:
        m = g.random((N, E)) < tie_fraction
        snapped = (np.round(z * 8.0) / 8.0).astype(np.float32)
        z = np.where(m, snapped, z).astype(np.float32)
        neg0 = g.random((N, E)) < tie_fraction * 0.05
        z = np.where(neg0, np.float32(-0.0), z).astype(np.float32)
    return np.ascontiguousarray(z)


def make_bias(seed: int, E: int, std: float = 0.1) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return g.standard_normal(E, dtype=np.float32) * np.float32(std)
