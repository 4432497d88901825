"""The pins must fail when a plausible mistake is planted in the oracle (CPU only).

Each case swaps one oracle function for a subtly wrong version (a transposed
factor, a dropped zero-point widening, floor instead of round-half-even, a
sum instead of a mean, an ascending sort, a wrong sign) and checks that at
least one pin from test_oracle_pins.py then fails.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import exact_obs
from oracle import gptq_oracle as go

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_cases_pass():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        H = np.array(case["H"], dtype=np.float64)
        W = np.array(case["W"], dtype=np.float64)
        out = go.gptq_layer(W, H, None, case["bits"], case["group_size"], case["sym"],
                            desc_act=False, damp_percent=0.0)
        if out["codes"].tolist() != case["codes"]:
            return False
        if not np.allclose(out["loss0"], case["loss0"], rtol=1e-12):
            return False
    return True


def _exact_route_passes():
    for seed in range(12):
        rng = np.random.default_rng(seed)
        n, m = 4, 2
        A = rng.integers(-4, 5, size=(n, n + 2)).astype(np.float64)
        H = A @ A.T + np.eye(n)
        W = np.round(rng.standard_normal((m, n)) * 0.5, 3)
        key = np.diag(H).copy()
        out = go.gptq_layer(W, H, key, 3, 2, False, desc_act=True, damp_percent=0.01)
        lam = 0.01 * float(np.mean(key))
        order = sorted(range(n), key=lambda j: (-H[j, j], j))
        Hd = [[Fraction(float(H[i, j])) + (Fraction(lam) if i == j else 0) for j in order] for i in order]
        Wp = [[Fraction(float(W[r, j])) for j in order] for r in range(m)]
        codes, _, _, loss = exact_obs.gptq_exact(Wp, Hd, 3, 2, False)
        if out["codes_p"].tolist() != codes or not np.isclose(out["loss0"], float(loss), rtol=1e-9):
            return False
    return True


def _ties_pass():
    import test_oracle_pins as tp
    try:
        for bits in (3, 4, 8):
            tp.test_symmetric_range_zero_point_tie_goes_to_even(bits)
        tp.test_code_ties_match_exact_route()
    except AssertionError:
        return False
    return True


def _plain_rint_zero(v, bits, sym):
    s, z, lo, hi = _orig["group_params"](v, bits, sym)
    if not sym:
        z = np.rint(-lo / s)    # the rounded step decides the tie
    return s, z, lo, hi


def _plain_rint_codes(w, s, z, bits, sym, lo=None, hi=None):
    w = np.asarray(w, dtype=np.float64)
    if sym:
        q = 2 ** (bits - 1) - 1
        return np.clip(np.rint(w / s), -q, q) + z
    return np.clip(np.rint(w / s + z), 0, 2 ** bits - 1)


def _wrong_factor_lower(Hp):
    U = _orig["inverse_upper_factor"](Hp)
    return U.T.copy()            # lower factor handed out as if it were U


def _wrong_factor_transposed_solve(Hp):
    L = np.linalg.cholesky(np.asarray(Hp, dtype=np.float64))
    return L.T.copy()            # chol(H) instead of chol(H^-1)


def _no_widening(v, bits, sym):
    if sym:
        return _orig["group_params"](v, bits, sym)
    lo, hi = np.min(v, axis=1), np.max(v, axis=1)
    s = np.maximum((hi - lo) / (2 ** bits - 1), go.SCALE_FLOOR)
    return s, np.round(-lo / s), lo, hi


def _floor_codes(w, s, z, bits, sym, lo=None, hi=None):
    if sym:
        q = 2 ** (bits - 1) - 1
        return np.clip(np.floor(w / s), -q, q) + z
    return np.clip(np.floor(w / s + z), 0, 2 ** bits - 1)


def _damping_sum(key, p):
    return float(p) * float(np.sum(key))


def _ascending(key, desc_act):
    if not desc_act:
        return np.arange(len(key))
    return np.argsort(np.asarray(key), kind="stable")


def _wrong_sign_dequant(q, s, z):
    return (z - np.asarray(q, dtype=np.float64)) * s


_orig = {name: getattr(go, name) for name in
         ("inverse_upper_factor", "group_params", "quantize_values", "damping", "act_order",
          "dequantize_values")}

PLANTS = [
    ("inverse_upper_factor", _wrong_factor_lower),
    ("inverse_upper_factor", _wrong_factor_transposed_solve),
    ("group_params", _no_widening),
    ("quantize_values", _floor_codes),
    ("damping", _damping_sum),
    ("act_order", _ascending),
    ("dequantize_values", _wrong_sign_dequant),
    ("group_params", _plain_rint_zero),
    ("quantize_values", _plain_rint_codes),
]


def test_unplanted_oracle_passes_the_checks():
    assert _hand_cases_pass() and _exact_route_passes() and _ties_pass()


@pytest.mark.parametrize("name,fn", PLANTS, ids=[f"{n}:{f.__name__}" for n, f in PLANTS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(go, name, fn)
    assert not (_hand_cases_pass() and _exact_route_passes() and _ties_pass())


# ---------------------------------------------------------------------------
# The linear (round-to-nearest) quantizer's pins bite too
# ---------------------------------------------------------------------------
from oracle import linear_quantizer as lq  # noqa: E402
import test_oracle_linear_pins as lp  # noqa: E402


def _linear_pins_pass():
    checks = [
        lp.test_worked_int8_example_through_linear_quantizer,
        lambda: lp.test_percentile_is_numpy_linear_percentile(100, 0.99),
        lambda: lp.test_percentile_is_numpy_linear_percentile(7, 0.3),
        lp.test_percentile_hand_positions,
        lp.test_asym_hand_case,
        lp.test_sym_clip_hand_case,
        lp.test_asym_clip_hand_case,
        lambda: lp.test_clip_one_is_min_max(True),
        lambda: lp.test_clip_one_is_min_max(False),
        lambda: lp.test_codes_on_grid_and_dequant_identity(4, False),
        lp.test_all_zero_row_uses_the_floor,
        lp.test_mse_and_cos_against_fractions,
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def _pct_rank_n(values, frac):   # position f·N instead of f·(N-1)
    a = np.sort(np.asarray(values, dtype=np.float64).ravel())
    p = float(frac) * a.size
    i = min(int(np.floor(p)), a.size - 1)
    if i >= a.size - 1:
        return float(a[-1])
    return float(a[i] + (a[i + 1] - a[i]) * (p - i))


def _codes_floor(v, scale, zp, qmin, qmax, sym):
    v = np.asarray(v, dtype=np.float64)
    q = np.floor(v / scale) if sym else np.floor(v / scale + zp)
    return np.clip(q, qmin, qmax)


def _grid_wrong_qmax(v, bits, sym, clip_ratio):
    s, zp, qmin, qmax = _orig_grid(v, bits, sym, clip_ratio)
    if sym:
        s = s * (2 ** (bits - 1) - 1) / 2 ** (bits - 1)   # divides by 2^(b-1)
    return s, zp, qmin, qmax


def _grid_zp_sign(v, bits, sym, clip_ratio):
    s, zp, qmin, qmax = _orig_grid(v, bits, sym, clip_ratio)
    return s, -zp, qmin, qmax


def _grid_widened(v, bits, sym, clip_ratio):   # the GPTQ path's range, not the page's
    v = np.asarray(v, dtype=np.float64)
    if sym:
        return _orig_grid(v, bits, sym, clip_ratio)
    lo, hi = min(float(np.min(v)), 0.0), max(float(np.max(v)), 0.0)
    s = max((hi - lo) / (2 ** bits - 1), 1e-8)
    return s, -float(np.rint(lo / s)), 0, 2 ** bits - 1


_orig_grid = lq.linear_grid


def _lq_mse_sum(W, bits, sym, group_size, clip_ratio):
    out = _orig_lq(W, bits, sym, group_size, clip_ratio)
    out["mse"] = out["mse"] * np.asarray(W).size
    return out


_orig_lq = lq.linear_quantize


def test_linear_pins_pass_unpatched():
    assert _linear_pins_pass()


@pytest.mark.parametrize("target,wrong", [
    ("percentile_linear", _pct_rank_n),
    ("linear_codes", _codes_floor),
    ("linear_grid", _grid_wrong_qmax),
    ("linear_grid", _grid_zp_sign),
    ("linear_grid", _grid_widened),
    ("linear_quantize", _lq_mse_sum),
], ids=["percentile_rank_N", "floor_rounding", "sym_qmax_2^(b-1)", "zero_point_sign", "asym_widened_to_0",
        "mse_sum_not_mean"])
def test_linear_pins_catch(monkeypatch, target, wrong):
    monkeypatch.setattr(lq, target, wrong)
    monkeypatch.setattr(oracle_pkg, target, wrong)
    assert not _linear_pins_pass()


import oracle as oracle_pkg  # noqa: E402


# ---------------------------------------------------------------------------
# The quantized-weight product's pins bite too
# ---------------------------------------------------------------------------
from oracle import quantized_matmul as dm  # noqa: E402
import test_oracle_dequant_pins as dp  # noqa: E402


def _dequant_pins_pass():
    checks = [dp.test_hand_case, dp.test_codes_at_the_zero_point_give_zero]
    checks += [lambda b=b: dp.test_brute_force_from_packed_words(b) for b in (2, 3, 4, 8)]
    checks += [lambda a=a: dp.test_product_error_is_the_quantizers_loss(*a)
               for a in ((4, 4, False), (3, 8, False), (2, 4, True), (8, -1, False))]
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


_dm_orig = {"dequantized_weight": dm.dequantized_weight, "unpack_codes": dm.unpack_codes}


def _contiguous_groups(qweight, scales, zeros, g_idx, n, bits):
    g = max(1, -(-n // np.asarray(scales).shape[1]))
    return _dm_orig["dequantized_weight"](qweight, scales, zeros, np.arange(n) // g, n, bits)


def _zero_sign(qweight, scales, zeros, g_idx, n, bits):
    Q = dm.unpack_codes(np.asarray(qweight).view(np.uint32), n, bits).astype(np.float64)
    gi = np.asarray(g_idx, dtype=np.int64)
    return (np.asarray(zeros, dtype=np.float64)[:, gi] - Q) * np.asarray(scales, dtype=np.float64)[:, gi]


def _reversed_nibbles(qweight, n, bits):
    Q = _dm_orig["unpack_codes"](qweight, n, bits)
    per = 8 if bits <= 4 else 4
    out = Q.copy()
    for w0 in range(0, n - n % per, per):
        out[:, w0:w0 + per] = Q[:, w0:w0 + per][:, ::-1]
    return out


def _scale_by_row_group(qweight, scales, zeros, g_idx, n, bits):
    Q = dm.unpack_codes(np.asarray(qweight).view(np.uint32), n, bits).astype(np.float64)
    gi = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float64)
    return (Q - np.asarray(zeros, dtype=np.float64)[:, gi]) * s[:, :1]   # first group's scale


DM_PLANTS = [
    ("dequantized_weight", _contiguous_groups),
    ("dequantized_weight", _zero_sign),
    ("unpack_codes", _reversed_nibbles),
    ("dequantized_weight", _scale_by_row_group),
]


def test_unplanted_dequant_oracle_passes():
    assert _dequant_pins_pass()


@pytest.mark.parametrize("name,fn", DM_PLANTS, ids=[f"{n}:{f.__name__}" for n, f in DM_PLANTS])
def test_planted_dequant_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(dm, name, fn)
    assert not _dequant_pins_pass()


# ---------------------------------------------------------------------------
# The AWQ channel-scaling pins bite too
# ---------------------------------------------------------------------------
from oracle import awq  # noqa: E402
import test_oracle_awq_pins as ap  # noqa: E402


def _awq_pins_pass():
    checks = [ap.test_hand_case, ap.test_scale_one_is_the_plain_linear_quantizer,
              ap.test_equal_importance_scales_nothing]
    checks += [lambda n=n: ap.test_lower_median_is_torch_convention(n) for n in (2, 8, 101)]
    checks += [lambda s=s: ap.test_scaled_channels_and_round_trip(s) for s in (False, True)]
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


_awq_orig = {k: getattr(awq, k) for k in ("lower_median", "channel_scale", "channel_abs_sum", "awq_quantize")}


def _mean_median(v):
    return float(np.median(np.asarray(v, dtype=np.float64)))


def _scale_at_or_above(abs_sum, tokens, s=2.0):
    imp = np.asarray(abs_sum, dtype=np.float64) / float(tokens)
    med = awq.lower_median(imp)
    sc = np.ones(imp.shape, dtype=np.float32)
    sc[imp >= med] = np.float32(s)
    return sc, imp, med


def _signed_sum(X):
    return np.sum(np.asarray(X, dtype=np.float64), axis=0)


def _dequant_times_scale(W, abs_sum, tokens, s=2.0, bits=4, sym=False, group_size=128, clip_ratio=1.0):
    out = _awq_orig["awq_quantize"](W, abs_sum, tokens, s, bits, sym, group_size, clip_ratio)
    out["deq"] = out["deq"] * out["channel_scale"].astype(np.float64) ** 2
    return out


AWQ_PLANTS = [
    ("lower_median", _mean_median),
    ("channel_scale", _scale_at_or_above),
    ("channel_abs_sum", _signed_sum),
    ("awq_quantize", _dequant_times_scale),
]


def test_unplanted_awq_oracle_passes():
    assert _awq_pins_pass()


@pytest.mark.parametrize("name,fn", AWQ_PLANTS, ids=[f"{n}:{f.__name__}" for n, f in AWQ_PLANTS])
def test_planted_awq_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(awq, name, fn)
    assert not _awq_pins_pass()
