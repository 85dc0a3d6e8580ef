"""The oracle's FP8 (E4M3) codec and quantisers against the format's
definition, torch's own E4M3 conversion and the error bounds of rounding.
[K1D] FP8 section: weights in 128 x 128 blocks with one fp32 scale each,
activations quantised per 1 x 128 group; 448 is the largest E4M3 value
([KPT] §4.4)."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def test_decode_table():
    v = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # codes 0..126 ascending
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -9 and pos[7] == 7 * 2.0 ** -9
    assert pos[8] == 2.0 ** -6 and v[0x38] == 1.0 and pos[126] == 448.0
    assert np.array_equal(v[0x80:0xFF], -pos)             # sign bit
    # exponent steps: within a binade the spacing is 1/8 of its start
    for e in range(1, 15):
        start = 2.0 ** (e - 7)
        assert np.allclose(np.diff(pos[8 * e:8 * e + 8]), start / 8)


def test_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(126):
        mid = (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert O.e4m3_encode(np.array([mid]))[0] == even
        eps = (pos[c + 1] - pos[c]) * 1e-3
        assert O.e4m3_encode(np.array([mid - eps]))[0] == c
        assert O.e4m3_encode(np.array([mid + eps]))[0] == c + 1
    assert O.e4m3_encode(np.array([1e6, -1e6, -0.0]))[[0, 1, 2]].tolist() == [0x7E, 0xFE, 0x80]


def test_encode_matches_torch_e4m3fn_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 1e-3]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), t)


def test_row_group_quantisation_bounds():
    rng = np.random.default_rng(12)
    X = (rng.standard_normal((37, 300)) * np.exp(rng.standard_normal((37, 1)))).astype(np.float32)
    X[3, 128:256] = 0.0                                    # an all-zero group
    q, s = O.quantize_row_groups(X, 128)
    assert s.shape == (37, 3) and s[3, 1] == 0 and not q[3, 128:256].any()
    D = O.dequantize_row_groups(q, s, 128)
    for n in range(37):
        for j in range(3):
            x = X[n, j * 128:(j + 1) * 128].astype(np.float64)
            d = D[n, j * 128:(j + 1) * 128]
            if s[n, j] == 0:
                continue
            assert np.float32(np.abs(x).max() / np.float32(448)) == s[n, j]
            # the largest magnitude lands on +-448 exactly
            assert np.max(np.abs(O.e4m3_decode(q[n, j * 128:(j + 1) * 128]))) == 448.0
            # half a step of E4M3 (relative 2^-4 for normals, 2^-10 absolute
            # in units of s for subnormals), plus the fp32 rounding of x / s
            tol = np.maximum(np.abs(x) * 2.0 ** -4, s[n, j] * 2.0 ** -10) * (1 + 1e-6)
            assert np.all(np.abs(d - x) <= tol)


def test_row_group_quantisation_of_fp64_values():
    """H is quantised from fp64: the scale is fp32(amax / 448), the largest
    magnitude of a group lands on +-448, every value is within half an E4M3
    step (normal) or half a subnormal step of the scale, and values that are
    exactly a code times the scale come back unchanged."""
    rng = np.random.default_rng(14)
    X = rng.standard_normal((29, 384)) * np.exp(2 * rng.standard_normal((29, 1)))
    X[4, :128] = 0.0
    X[5, 128:256] *= 1e-7                                  # deep in the subnormals
    X[5, 128] = 3.0
    q, s = O.quantize_row_groups_f64(X, 128)
    assert s.dtype == np.float32 and s[4, 0] == 0 and not q[4, :128].any()
    D = O.dequantize_row_groups(q, s, 128)
    for n in range(29):
        for j in range(3):
            x = X[n, j * 128:(j + 1) * 128]
            if s[n, j] == 0:
                continue
            assert np.float32(np.abs(x).max() / 448.0) == s[n, j]
            assert np.max(np.abs(O.e4m3_decode(q[n, j * 128:(j + 1) * 128]))) == 448.0
            tol = np.maximum(np.abs(x) * 2.0 ** -4, np.float64(s[n, j]) * 2.0 ** -10) * (1 + 1e-9)
            assert np.all(np.abs(D[n, j * 128:(j + 1) * 128] - x) <= tol)
    # exact multiples of the scale: codes times a power-of-two scale
    codes = rng.integers(0, 0x7F, (3, 128)).astype(np.uint8)
    codes[:, 0] = 0x7E                                     # 448 sets the scale
    vals = O.e4m3_decode(codes) * 2.0 ** -5
    q2, s2 = O.quantize_row_groups_f64(vals, 128)
    assert np.all(s2 == np.float32(2.0 ** -5)) and np.array_equal(q2, codes)
    # a value just off a midpoint between two codes is decided by its fp64
    # value, not by an fp32 rounding of it
    mid = (O.e4m3_decode(np.array([0x30]))[0] + O.e4m3_decode(np.array([0x31]))[0]) / 2
    row = np.zeros((1, 128))
    row[0, 0] = 448.0
    row[0, 1] = mid * (1 + 2.0 ** -40)
    q3, _ = O.quantize_row_groups_f64(row, 128)
    assert q3[0, 1] == 0x31


def test_weight_blocks_ragged():
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((300, 200)) * 0.02).astype(np.float32)
    q, s = O.quantize_weight_blocks(W, 128)
    assert s.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            blk = W[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == np.float32(np.abs(blk).max() / np.float32(448))
    D = O.dequantize_blocks(q, s, 128)
    assert D.shape == W.shape
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:300, :200]
    tol = np.maximum(np.abs(W.astype(np.float64)) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(D - W) <= tol)


# ---------------------------------------------------------------------------
# FP8 experts.  The only rounding between the dequantised operands and the
# output is the E4M3 quantisation of H in 1 x 128 groups, so an FP8 expert
# must equal the fp64 SwiGLU of the dequantised x and weights within the
# error that this rounding can carry through W_down:
#   |dH_j| <= max(|H_j| 2^-4, s_g 2^-10)
# (half an E4M3 step of a normal value, or half a subnormal step of the group
# scale s_g).  The planted mistakes below show the bound is tight enough to
# catch a transposed block-scale index and a missing quantisation of x.
# ---------------------------------------------------------------------------
def _blocky(rng, R, Cc, sd):
    """Gaussian matrix whose 128 x 128 blocks differ in size by up to 100x."""
    W = rng.standard_normal((R, Cc)) * sd
    for i in range(0, R, 128):
        for j in range(0, Cc, 128):
            W[i:i + 128, j:j + 128] *= 10.0 ** rng.uniform(-1, 1)
    return W.astype(np.float32)


def _outlier_rows(rng, n, d, big=300.0):
    """bf16-exact activations with one large value per 128-group (in a fixed
    column of each group, returned as well), so that quantising the row
    moves its small values a lot."""
    X = rng.standard_normal((n, d)).astype(np.float32)
    cols = np.arange(0, d, 128) + rng.integers(0, 128, d // 128)
    X[:, cols] = big
    return O.bf16_to_f32(O.f32_to_bf16_rne(X)), cols


def _expert_bound(Xd, Gd, Ud, Dd):
    H = O.silu(Xd @ Gd.T) * (Xd @ Ud.T)
    sg = np.repeat(np.abs(H).reshape(H.shape[0], -1, 128).max(axis=2) / 448.0, 128, axis=1)
    err = np.maximum(np.abs(H) * 2.0 ** -4, sg * 2.0 ** -10)
    return H, (err @ np.abs(Dd).T) * (1 + 1e-6) + 1e-12


def test_swiglu_fp8_within_h_rounding_bound():
    rng = np.random.default_rng(21)
    d = h = 256
    Wg, Wu, Wd = _blocky(rng, h, d, 0.05), _blocky(rng, h, d, 0.05), _blocky(rng, d, h, 0.05)
    # outliers of 1e5 push the other values of their group into the E4M3
    # subnormals; zero weight columns under them keep them out of G and U
    X, cols = _outlier_rows(rng, 16, d, 1e5)
    Wg[:, cols] = 0.0
    Wu[:, cols] = 0.0
    xq, xs = O.quantize_row_groups(X)
    gq, gs = O.quantize_weight_blocks(Wg)
    uq, us = O.quantize_weight_blocks(Wu)
    dq, ds = O.quantize_weight_blocks(Wd)
    y = O.swiglu_fp8(xq, xs, gq, gs, uq, us, dq, ds)
    Xd = O.dequantize_row_groups(xq, xs)
    Gd, Ud, Dd = O.dequantize_blocks(gq, gs), O.dequantize_blocks(uq, us), O.dequantize_blocks(dq, ds)
    H, bound = _expert_bound(Xd, Gd, Ud, Dd)
    assert np.all(np.abs(y - H @ Dd.T) <= bound)
    # planted: the gate scales read transposed
    y_t = O.swiglu_fp8(xq, xs, gq, gs.T.copy(), uq, us, dq, ds)
    assert np.any(np.abs(y_t - H @ Dd.T) > bound)
    # planted: x used without its quantisation
    H_raw = O.silu(X.astype(np.float64) @ Gd.T) * (X.astype(np.float64) @ Ud.T)
    assert np.any(np.abs(H_raw @ Dd.T - H @ Dd.T) > bound)


def test_moe_combine_fp8_within_bound_and_subset():
    rng = np.random.default_rng(22)
    N, d, E, K, h, hs = 24, 256, 4, 2, 128, 128
    x, _ = _outlier_rows(rng, N, d)
    w_gate = np.stack([_blocky(rng, h, d, 0.05) for _ in range(E)])
    w_up = np.stack([_blocky(rng, h, d, 0.05) for _ in range(E)])
    w_down = np.stack([_blocky(rng, d, h, 0.05) for _ in range(E)])
    ws = [np.stack([_blocky(rng, *shp, 0.05)]) for shp in ((hs, d), (hs, d), (d, hs))]
    Z = rng.standard_normal((N, E)).astype(np.float32)
    ids, _, _ = O.route(Z, None, K)
    S = O.mixture_weights(Z, ids)
    q = O.quantize_expert_weights(w_gate, w_up, w_down, *ws)
    y = O.moe_combine_fp8(x, q, ids, S)
    # reference: fp64 layer on the dequantised x rows and weights
    xq, xs = O.quantize_row_groups(x)
    Xd = O.dequantize_row_groups(xq, xs)
    deq = {k: np.stack([O.dequantize_blocks(c, s) for c, s in zip(q[k], q[sk])])
           for k, sk in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down"),
                         ("ws_gate", "ss_gate"), ("ws_up", "ss_up"), ("ws_down", "ss_down"))}
    y_ref = O.moe_combine(Xd, deq["w_gate"], deq["w_up"], deq["w_down"], deq["ws_gate"],
                          deq["ws_up"], deq["ws_down"], ids, S)
    bound = _expert_bound(Xd, deq["ws_gate"][0], deq["ws_up"][0], deq["ws_down"][0])[1]
    for e in range(E):
        rows, slots = np.nonzero(ids == e)
        b = _expert_bound(Xd[rows], deq["w_gate"][e], deq["w_up"][e], deq["w_down"][e])[1]
        bound[rows] += np.asarray(S, np.float64)[rows, slots][:, None] * b
    assert np.all(np.abs(y - y_ref) <= bound)
    # planted: the mixture weight dropped on the routed experts
    y_noS = O.moe_combine_fp8(x, q, ids, np.ones_like(S))
    assert np.any(np.abs(y_noS - y_ref) > bound)
    # rows are quantised independently, so a token subset is a row selection
    # (up to the summation order of the fp64 products)
    sub = [5, 0, 17]
    assert np.allclose(O.moe_combine_fp8(x, q, ids, S, token_subset=sub), y[sub],
                       rtol=1e-12, atol=1e-9)
