"""Pins of the linear (round-to-nearest) quantizer oracle (CPU only).

The oracle follows page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.1 (the
LinearQuantizer) with the readings listed in its header.  Every expected value
here comes from the pages' worked example, from a hand derivation written out
in the test, or from a library routine the reading reduces to (NumPy's
percentile); none is produced by the oracle itself.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_int8_example_through_linear_quantizer():
    # page "大模型量化：GPTQ/AWQ/GGUF 原理对比…", quantization basics: symmetric
    # INT8 of one float32 vector, no clipping
    g = _load("int8_worked_example.json")
    w = np.array(g["input_float32"], dtype=np.float32).astype(np.float64)
    out = oracle.linear_quantize(w[None, :], 8, True, -1, 1.0)
    assert out["scales"][0, 0] == pytest.approx(float(np.float32(3.7)) / 127, rel=1e-15)
    assert list(out["codes"][0] - 128) == g["codes_signed"]
    assert int(out["zeros"][0, 0]) == 128
    np.testing.assert_allclose(out["deq"][0], g["dequant_from_codes"], rtol=1e-6)
    assert out["mse"] == pytest.approx(g["mse_from_codes"], rel=1e-3)


@pytest.mark.parametrize("N", [1, 2, 7, 100, 1001])
@pytest.mark.parametrize("frac", [0.0, 0.005, 0.01, 0.3, 0.5, 0.99, 0.995, 1.0])
def test_percentile_is_numpy_linear_percentile(N, frac):
    # reading L2 is NumPy's default (linear) percentile; values compared to 1 ulp-ish
    rng = np.random.default_rng(N)
    a = rng.standard_normal(N) * 3.0
    ref = float(np.percentile(a, 100.0 * frac))
    assert oracle.percentile_linear(a, frac) == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_percentile_hand_positions():
    # 11 values 0, 10, ..., 100 (shuffled): position f·10
    a = np.array([30, 0, 100, 20, 90, 10, 80, 40, 70, 60, 50], dtype=np.float64)
    assert oracle.percentile_linear(a, 0.0) == 0.0
    assert oracle.percentile_linear(a, 1.0) == 100.0
    assert oracle.percentile_linear(a, 0.5) == 50.0
    assert oracle.percentile_linear(a, 0.25) == pytest.approx(25.0, abs=1e-12)   # p = 2.5
    assert oracle.percentile_linear(a, 0.99) == pytest.approx(99.0, abs=1e-12)   # p = 9.9


def test_asym_hand_case():
    # w = [-1, 0, 2, 3], 2-bit asym, no clipping: lo = -1, hi = 3, scale = 4/3,
    # zp = -rne(-3/4) = 1; codes rne(w·3/4 + 1) = rne(0.25, 1, 2.5, 3.25) = 0, 1, 2, 3
    # (2.5 -> 2, half to even); ŵ = (q - 1)·4/3 = -4/3, 0, 4/3, 8/3;
    # errors 1/3, 0, 2/3, 1/3 -> MSE = (1/9 + 4/9 + 1/9)/4 = 1/6;
    # Σwŵ = 4/3 + 8/3 + 8 = 12, ‖w‖² = 14, ‖ŵ‖² = 96/9.
    out = oracle.linear_quantize(np.array([[-1.0, 0.0, 2.0, 3.0]]), 2, False, -1, 1.0)
    assert out["scales"][0, 0] == pytest.approx(4.0 / 3.0, rel=1e-15)
    assert int(out["zeros"][0, 0]) == 1
    assert out["codes"][0].tolist() == [0, 1, 2, 3]
    np.testing.assert_allclose(out["deq"][0], [-4 / 3, 0, 4 / 3, 8 / 3], rtol=1e-15)
    assert out["mse"] == pytest.approx(1.0 / 6.0, rel=1e-14)
    assert out["cos"] == pytest.approx(12.0 / (np.sqrt(14.0) * np.sqrt(96.0 / 9.0) + 1e-8), rel=1e-14)


def test_sym_clip_hand_case():
    # row 0, 1, ..., 99 and one outlier 1000 (101 values), 8-bit sym, clip 0.98:
    # |w| sorted = 0..99, 1000; position 0.98·100 = 98 -> amax = 98, scale = 98/127.
    # codes rne(w·127/98): 1000 -> 1295.9 -> clamped to 127; 50 -> 64.79 -> 65;
    # 49 -> 63.5 -> 64 (half to even); stored +128.
    w = np.concatenate([np.arange(100, dtype=np.float64), [1000.0]])[None, :]
    out = oracle.linear_quantize(w, 8, True, -1, 0.98)
    assert out["scales"][0, 0] == pytest.approx(98.0 / 127.0, rel=1e-15)
    q = out["codes"][0] - 128
    assert q[100] == 127 and q[50] == 65 and q[49] == 64 and q[0] == 0
    assert q[98] == 127 and q[97] == 126


def test_asym_clip_hand_case():
    # same row, 8-bit asym, clip 0.98: positions 0.01·100 = 1 and 0.99·100 = 99
    # -> lo = 1, hi = 99; scale = 98/255; zp = -rne(255/98 = 2.602) = -3;
    # codes rne(w·255/98 - 3) clamped to [0, 255]: 0 -> -3 -> 0; 50 -> 127.1 -> 127;
    # 99 -> 254.6 -> 255; 1000 -> 255.
    w = np.concatenate([np.arange(100, dtype=np.float64), [1000.0]])[None, :]
    out = oracle.linear_quantize(w, 8, False, -1, 0.98)
    assert out["scales"][0, 0] == pytest.approx(98.0 / 255.0, rel=1e-15)
    assert int(out["zeros"][0, 0]) == -3
    q = out["codes"][0]
    assert q[0] == 0 and q[50] == 127 and q[99] == 255 and q[100] == 255 and q[2] == 2


@pytest.mark.parametrize("sym", [True, False])
def test_clip_one_is_min_max(sym):
    # no clipping: the grid comes from max|w| (sym) or min / max (asym)
    rng = np.random.default_rng(3)
    w = rng.standard_normal((3, 40))
    out = oracle.linear_quantize(w, 4, sym, -1, 1.0)
    for r in range(3):
        if sym:
            assert out["scales"][r, 0] == pytest.approx(np.max(np.abs(w[r])) / 7, rel=1e-15)
        else:
            s = (np.max(w[r]) - np.min(w[r])) / 15
            assert out["scales"][r, 0] == pytest.approx(s, rel=1e-15)
            assert out["zeros"][r, 0] == -int(np.rint(np.min(w[r]) / s))


@pytest.mark.parametrize("sym", [True, False])
def test_group_covering_row_equals_per_channel(sym):
    rng = np.random.default_rng(4)
    w = rng.standard_normal((5, 64))
    a = oracle.linear_quantize(w, 3, sym, -1, 0.97)
    b = oracle.linear_quantize(w, 3, sym, 64, 0.97)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("sym", [True, False])
def test_codes_on_grid_and_dequant_identity(bits, sym):
    rng = np.random.default_rng(bits)
    w = rng.standard_normal((6, 50)) * 0.02
    out = oracle.linear_quantize(w, bits, sym, 16, 0.99)
    assert out["codes"].min() >= 0 and out["codes"].max() <= 2 ** bits - 1
    G = out["scales"].shape[1]
    for r in range(6):
        for j in range(G):
            c0, c1 = 16 * j, min(16 * j + 16, 50)
            np.testing.assert_array_equal(
                out["deq"][r, c0:c1], (out["codes"][r, c0:c1] - out["zeros"][r, j]) * out["scales"][r, j])
    # every per-group error is at most half a step unless the value was clipped
    lo = np.repeat(out["zeros"], 16, axis=1)[:, :50]
    sc = np.repeat(out["scales"], 16, axis=1)[:, :50]
    inside = (out["codes"] > 0) & (out["codes"] < 2 ** bits - 1)
    assert np.all(np.abs(w - out["deq"])[inside] <= 0.5 * sc[inside] * (1 + 1e-12))


def test_all_zero_row_uses_the_floor():
    out = oracle.linear_quantize(np.zeros((1, 8)), 4, True, -1, 0.99)
    assert out["scales"][0, 0] == 1e-8 and np.all(out["codes"] == 8)
    out = oracle.linear_quantize(np.zeros((1, 8)), 4, False, -1, 0.99)
    assert out["scales"][0, 0] == 1e-8 and np.all(out["codes"] == 0)


def test_mse_and_cos_against_fractions():
    # exact rational check of L7 on a 2 x 3 case (sym 2-bit: qmax 1, range [-2, 1])
    w = [[Fraction(1, 2), Fraction(-3, 4), Fraction(1, 8)], [Fraction(2), Fraction(-1), Fraction(1, 2)]]
    out = oracle.linear_quantize(np.array(w, dtype=np.float64), 2, True, -1, 1.0)
    # row 0: scale 3/4, codes rne(2/3, -1, 1/6) = 1, -1, 0 -> ŵ 3/4, -3/4, 0
    # row 1: scale 2, codes rne(1, -1/2, 1/4) = 1, 0 (half to even), 0 -> ŵ 2, 0, 0
    deq = [[Fraction(3, 4), Fraction(-3, 4), Fraction(0)], [Fraction(2), Fraction(0), Fraction(0)]]
    se = sum((w[r][c] - deq[r][c]) ** 2 for r in range(2) for c in range(3))
    assert out["mse"] == pytest.approx(float(se / 6), rel=1e-14)
    dot = sum(w[r][c] * deq[r][c] for r in range(2) for c in range(3))
    nw = sum(x * x for row in w for x in row)
    nd = sum(x * x for row in deq for x in row)
    assert out["cos"] == pytest.approx(float(dot) / (np.sqrt(float(nw)) * np.sqrt(float(nd)) + 1e-8), rel=1e-13)
