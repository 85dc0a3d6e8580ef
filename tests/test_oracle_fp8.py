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
