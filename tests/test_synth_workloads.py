"""Seeded workloads: determinism, shapes, and what each workload must show
through the oracle (toy collapse, Zipf skew)."""
import numpy as np

from oracle import moe_oracle as O
from synth import CONFIGS, make_inputs, scaled


def test_toy_inputs_deterministic_and_shaped():
    cfg = CONFIGS["toy"]
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for k in ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.x.shape == (4, 64) and a.w_gate.shape == (4, 32, 64)
    assert a.w_down.shape == (4, 64, 32) and a.ws_down.shape == (1, 64, 32)
    assert a.f32["x"].shape == (4, 64)
    assert np.array_equal(a.beta_in, np.zeros(4, np.float32))


def test_toy_collapse_and_one_update_fp32_and_bf16():
    cfg = CONFIGS["toy"]
    L = make_inputs(cfg)
    for src in ("f32", "bf16"):
        if src == "f32":
            w = L.f32
        else:
            w = {k: O.bf16_to_f32(getattr(L, k)) for k in
                 ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
        out = O.moe_layer(**w, beta_in=L.beta_in, K=cfg.K, recompute_bias=True,
                          logit_offset=L.logit_offset)
        assert out["counts_before"].tolist() == [4, 4, 0, 0]
        assert O.max_vio(out["counts_before"], 4, 2, 4) == 1.0
        # exactness on the bf16-rounded quantile keys: #{u > Q} <= r < #{u >= Q}
        Z = out["logits"]
        u = O.eqb_keys_values((Z + out["alpha"][:, None]).astype(np.float32), 16)
        Q = out["quantile"][None, :]
        assert ((u > Q).sum(axis=0) <= 2).all() and ((u >= Q).sum(axis=0) > 2).all()
        assert out["counts"].sum() == 8
        assert O.max_vio(out["counts"], 4, 2, 4) < 1.0


def test_zipf_offset_shape_and_range():
    cfg = scaled(CONFIGS["skewed"], 64)
    from synth.inputs import logit_offset_for
    off = logit_offset_for(cfg)
    assert off.shape == (384,) and off.dtype == np.float32
    assert np.all(np.diff(off) < 0)
    assert -0.71 < off[0] < -0.69 and -4.28 < off[-1] < -4.26


def test_slab_drawing_independent_of_batch_size():
    a = make_inputs(scaled(CONFIGS["origin"], 8))
    b = make_inputs(scaled(CONFIGS["origin"], 4))
    assert np.array_equal(a.x[:4], b.x)
    assert np.array_equal(a.w_gate, b.w_gate)
