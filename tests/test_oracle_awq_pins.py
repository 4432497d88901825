"""Pins of the AWQ channel-scaling oracle (oracle/awq.py), CPU only: a
hand-worked case, torch.median's lower-median convention, the reductions to
the plain LinearQuantizer, and exact round trips of the channel scale."""
import json
import os

import numpy as np
import pytest

from oracle import awq, linear_quantizer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_hand_case():
    g = _load("awq_hand_case.json")
    X = np.array(g["X"])
    abs_sum = awq.channel_abs_sum(X)
    assert abs_sum.tolist() == g["abs_sum"]
    out = awq.awq_quantize(g["W"], abs_sum, X.shape[0], g["s"], g["bits"], g["sym"], g["group_size"],
                           g["clip_ratio"])
    assert out["importance"].tolist() == g["importance"]
    assert out["median"] == g["median"]
    assert out["channel_scale"].tolist() == g["channel_scale"]
    assert out["codes"].tolist() == g["codes"]
    np.testing.assert_allclose(out["scales"], g["scales"], rtol=1e-15)
    assert out["zeros"].tolist() == g["zeros"]
    np.testing.assert_allclose(out["deq"], g["deq"], rtol=1e-15, atol=1e-16)
    assert out["mse"] == pytest.approx(g["mse"], rel=1e-12)


@pytest.mark.parametrize("n", [1, 2, 7, 8, 101, 1000])
def test_lower_median_is_torch_convention(n):
    v = np.random.default_rng(n).standard_normal(n)
    med = awq.lower_median(v)
    assert med == np.sort(v)[(n - 1) // 2]
    if n % 2 == 1:
        assert med == np.median(v)
    else:
        assert med < np.median(v) < np.sort(v)[n // 2] or np.sort(v)[n // 2 - 1] == np.sort(v)[n // 2]
    # about half the channels are strictly above it
    assert int(np.sum(v > med)) == n - 1 - (n - 1) // 2


def test_scale_one_is_the_plain_linear_quantizer():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((6, 256)) * 0.02
    abs_sum = rng.uniform(0, 10, 256)
    out = awq.awq_quantize(W, abs_sum, 100, s=1.0, bits=4, sym=False, group_size=128)
    ref = linear_quantizer.linear_quantize(W.astype(np.float32).astype(np.float64), 4, False, 128, 1.0)
    assert np.array_equal(out["codes"], ref["codes"])
    np.testing.assert_array_equal(out["scales"], ref["scales"])
    np.testing.assert_array_equal(out["deq"], ref["deq"])


def test_equal_importance_scales_nothing():
    W = np.random.default_rng(2).standard_normal((3, 64)) * 0.1
    out = awq.awq_quantize(W, np.full(64, 5.0), 10, s=2.0, bits=3, sym=True, group_size=32)
    assert np.all(out["channel_scale"] == 1.0)


@pytest.mark.parametrize("sym", [False, True])
def test_scaled_channels_and_round_trip(sym):
    """Exactly the channels above the median carry s; with s a power of two the
    scaled weight and the division back are exact, so the dequantized weight
    times the channel scale is the LinearQuantizer's output on W·scale."""
    rng = np.random.default_rng(3)
    n = 200
    W = (rng.standard_normal((5, n)) * 0.05).astype(np.float32).astype(np.float64)
    abs_sum = rng.uniform(0, 1, n)
    out = awq.awq_quantize(W, abs_sum, 7, s=2.0, bits=4, sym=sym, group_size=-1)
    imp = abs_sum / 7
    assert np.array_equal(out["channel_scale"] == 2.0, imp > np.sort(imp)[(n - 1) // 2])
    assert int(np.sum(out["channel_scale"] == 2.0)) == n // 2
    ref = linear_quantizer.linear_quantize(W * out["channel_scale"], 4, sym, -1, 1.0)
    np.testing.assert_array_equal(out["deq"] * out["channel_scale"], ref["deq"])
    assert np.array_equal(out["codes"], ref["codes"])
