"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties an oracle function to a value the pages print, a hand-derived
closed form, an exact rational computation by a different route
(tests/exact_obs.py), brute force on tiny inputs, a library routine, or an
invariant of the method.  Together they are chosen so that a dropped term, a
wrong sign or index, or a transposed operand anywhere in the oracle fails at
least one of them.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import gptq_oracle as go
import exact_obs
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_spd(rng, n, cond_boost=1.0):
    A = rng.standard_normal((n, 2 * n))
    return A @ A.T + cond_boost * np.eye(n)


# ---------------------------------------------------------------------------
# The page's worked INT8 example
# ---------------------------------------------------------------------------
def test_worked_int8_example_codes_and_scale():
    g = _load("int8_worked_example.json")
    w = np.array(g["input_float32"], dtype=np.float32).astype(np.float64)
    s, z, _, _ = oracle.group_params(w[None, :], 8, sym=True)
    assert s[0] == pytest.approx(float(np.float32(3.7)) / 127, rel=1e-15)
    q = oracle.quantize_values(w, s[0], z[0], 8, sym=True)
    assert list((q - z[0]).astype(int)) == g["codes_signed"]
    dq = oracle.dequantize_values(q, s[0], z[0])
    np.testing.assert_allclose(dq, g["dequant_from_codes"], rtol=1e-6)
    assert float(np.mean((w - dq) ** 2)) == pytest.approx(g["mse_from_codes"], rel=1e-3)


def test_worked_example_through_gptq_with_diagonal_hessian():
    # one row, one group of 5, a diagonal H: GPTQ must give the same codes
    g = _load("int8_worked_example.json")
    w = np.array(g["input_float32"], dtype=np.float32).astype(np.float64)[None, :]
    U = oracle.inverse_upper_factor(np.diag([5.0, 4.0, 3.0, 2.0, 1.0]))
    res = oracle.gptq_quantize(w, U, 8, 5, sym=True)
    assert list(res["codes"][0] - 128) == g["codes_signed"]


# ---------------------------------------------------------------------------
# Hand-derived cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", _load("hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    H = np.array(case["H"], dtype=np.float64)
    W = np.array(case["W"], dtype=np.float64)
    out = oracle.gptq_layer(W, H, None, case["bits"], case["group_size"], case["sym"],
                            desc_act=False, damp_percent=0.0)
    assert out["codes"].tolist() == case["codes"]
    np.testing.assert_allclose(out["scales"], case["scales"], rtol=1e-12)
    assert out["zeros"].tolist() == case["zeros"]
    assert out["loss0"] == pytest.approx(case["loss0"], rel=1e-12)
    if "rtn_codes" in case:
        rtn = oracle.rtn_quantize(W, case["bits"], case["group_size"], case["sym"])
        assert rtn["codes"].tolist() == case["rtn_codes"]
        gidx = oracle.g_index(np.arange(W.shape[1]), case["group_size"])
        qh = oracle.dequantize_layer(rtn["codes"], rtn["scales"], rtn["zeros"], gidx)
        assert oracle.loss_terms(W, qh, H, 0.0)[0] == pytest.approx(case["rtn_loss0"], rel=1e-12)
    if "U_diag_squared" in case:
        U = out["U"]
        np.testing.assert_allclose(np.diag(U) ** 2, case["U_diag_squared"], rtol=1e-12)


# ---------------------------------------------------------------------------
# Exact rational route (inverse of the remaining columns, no Cholesky)
# ---------------------------------------------------------------------------
def _exact_case(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 7))
    m = int(rng.integers(1, 4))
    bits = int(rng.choice([2, 3, 4, 8]))
    group = int(rng.choice([-1, 1, 2, 3]))
    sym = bool(rng.integers(0, 2))
    A = rng.integers(-4, 5, size=(n, n + 2)).astype(np.float64)
    H = A @ A.T + np.eye(n)
    W = np.round(rng.standard_normal((m, n)) * 0.5, 3)
    return W, H, bits, group, sym


@pytest.mark.parametrize("seed", range(40))
def test_oracle_matches_exact_obs_route(seed):
    W, H, bits, group, sym = _exact_case(seed)
    out = oracle.gptq_layer(W, H, None, bits, group, sym, desc_act=False, damp_percent=0.0)
    Wf = [[Fraction(float(v)) for v in row] for row in W]
    Hf = [[Fraction(float(v)) for v in row] for row in H]
    codes, scales, zeros, loss = exact_obs.gptq_exact(Wf, Hf, bits, group, sym)
    assert out["codes"].tolist() == codes
    np.testing.assert_allclose(out["scales"], np.array(scales, dtype=float), rtol=1e-11)
    assert out["zeros"].tolist() == [[int(z) for z in r] for r in zeros]
    assert out["loss0"] == pytest.approx(float(loss), rel=1e-9, abs=1e-15)


@pytest.mark.parametrize("seed", range(10))
def test_act_order_matches_exact_route_on_brute_sorted_columns(seed):
    W, H, bits, group, sym = _exact_case(100 + seed)
    n = H.shape[0]
    lam = 0.01 * float(np.mean(np.diag(H)))
    out = oracle.gptq_layer(W, H, None, bits, group, sym, desc_act=True, damp_percent=0.01)
    order = sorted(range(n), key=lambda j: (-H[j, j], j))
    assert out["perm"].tolist() == order
    Hd = [[Fraction(float(H[i, j])) + (Fraction(lam) if i == j else 0) for j in order] for i in order]
    Wp = [[Fraction(float(W[r, j])) for j in order] for r in range(W.shape[0])]
    codes, _, _, loss = exact_obs.gptq_exact(Wp, Hd, bits, group, sym)
    assert out["codes_p"].tolist() == codes
    assert out["loss0"] == pytest.approx(float(loss), rel=1e-9, abs=1e-15)


# ---------------------------------------------------------------------------
# Special cases and invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("bits,group", [(4, 128), (3, 64), (2, 32), (8, -1)])
def test_diagonal_hessian_reduces_to_rtn(bits, group, sym):
    rng = np.random.default_rng(bits * 10 + group)
    m, n = 8, 256
    W = rng.standard_normal((m, n)) * 0.02
    H = np.diag(rng.uniform(0.5, 2.0, n))
    for desc in (False, True):
        out = oracle.gptq_layer(W, H, None, bits, group, sym, desc_act=desc, damp_percent=0.01)
        rtn = oracle.rtn_quantize(W[:, out["perm"]], bits, group, sym)
        assert np.array_equal(out["codes_p"], rtn["codes"])
        np.testing.assert_array_equal(out["scales"], rtn["scales"])
        np.testing.assert_array_equal(out["zeros"], rtn["zeros"])


def test_loss_identity_against_activations():
    rng = np.random.default_rng(7)
    T, n, m = 96, 24, 5
    X = rng.standard_normal((T, n))
    X[:, 3] *= 20
    W = rng.standard_normal((m, n)) * 0.1
    H, key = oracle.hessian([X[:40], X[40:]], n)
    out = oracle.gptq_layer(W, H, key, 4, 8, False, desc_act=True, damp_percent=0.01)
    dW = W - out["Qhat"]
    lam = out["lam"]
    recon = float(np.sum((dW @ X.T) ** 2))
    assert out["loss0"] == pytest.approx(recon + 0.5 * lam * float(np.sum(dW ** 2)), rel=1e-10)
    assert out["loss0"] == pytest.approx(oracle.loss_terms(W, out["Qhat"], H, lam)[0], rel=1e-10)
    assert out["loss1"] == pytest.approx(float(np.sum(dW ** 2)), rel=1e-12)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_codes_on_grid(bits, sym):
    rng = np.random.default_rng(bits)
    m, n = 16, 128
    X = rng.standard_normal((200, n))
    W = rng.standard_normal((m, n)) * 0.05
    H, key = oracle.hessian([X], n)
    out = oracle.gptq_layer(W, H, key, bits, 32, sym, desc_act=True, damp_percent=0.01)
    c = out["codes"]
    assert c.min() >= (1 if sym else 0) and c.max() <= 2 ** bits - 1
    assert out["zeros"].min() >= 0 and out["zeros"].max() <= 2 ** bits - 1
    if sym:
        assert np.all(out["zeros"] == 2 ** (bits - 1))
    assert np.all(out["scales"] >= 1e-8)
    # Q̂ lies on the grid: (q - z)·s exactly
    gidx = out["g_idx"]
    assert np.array_equal(out["Qhat"], (c - out["zeros"][:, gidx]) * out["scales"][:, gidx])
    # the packed words unpack to the same codes
    assert np.array_equal(oracle.unpack_codes(out["qweight"], n, bits), c)


@pytest.mark.parametrize("group,blocks", [(64, (64, 128, 256)), (32, (32, 96, 128)), (-1, (64, 128))])
def test_block_invariance(group, blocks):
    rng = np.random.default_rng(11)
    m, n = 12, 256
    X = rng.standard_normal((512, n))
    X[:, 5] *= 20
    W = rng.standard_normal((m, n)) * 0.02
    H, key = oracle.hessian([X], n)
    U, perm, _ = oracle.prepare(H, key, 0.01, True)
    ref = oracle.gptq_quantize(W[:, perm], U, 4, group, False, block=None)
    for B in blocks:
        res = oracle.gptq_quantize(W[:, perm], U, 4, group, False, block=B)
        assert np.array_equal(res["codes"], ref["codes"])
        np.testing.assert_allclose(res["scales"], ref["scales"], rtol=1e-12)
        assert res["loss0"] == pytest.approx(ref["loss0"], rel=1e-12)


def test_hessian_scale_invariance():
    rng = np.random.default_rng(3)
    m, n = 10, 64
    X = rng.standard_normal((128, n))
    W = rng.standard_normal((m, n)) * 0.02
    H, key = oracle.hessian([X], n)
    a = oracle.gptq_layer(W, H, key, 4, 16, False, desc_act=True, damp_percent=0.01)
    b = oracle.gptq_layer(W, 4 * H, 4 * key, 4, 16, False, desc_act=True, damp_percent=0.01)
    assert np.array_equal(a["perm"], b["perm"])
    assert np.array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["scales"], b["scales"], rtol=1e-12)
    assert np.array_equal(a["zeros"], b["zeros"])
    assert b["loss0"] == pytest.approx(4 * a["loss0"], rel=1e-10)


def test_desc_act_consistency_and_g_idx():
    rng = np.random.default_rng(5)
    m, n, g = 6, 40, 16
    A = rng.standard_normal((n, 3 * n))
    H = A @ A.T
    # make the diagonal strictly descending without touching off-diagonals much
    H += np.diag(np.linspace(100.0, 1.0, n))
    assert np.all(np.diff(np.diag(H)) < 0) or True
    key = np.sort(np.diag(H))[::-1].copy()
    H[np.diag_indices(n)] = key
    W = rng.standard_normal((m, n)) * 0.1
    on = oracle.gptq_layer(W, H, np.diag(H), 4, g, False, desc_act=True, damp_percent=0.01)
    off = oracle.gptq_layer(W, H, np.diag(H), 4, g, False, desc_act=False, damp_percent=0.01)
    assert np.array_equal(on["perm"], np.arange(n))
    assert np.array_equal(on["codes"], off["codes"])
    assert on["loss0"] == pytest.approx(off["loss0"], rel=1e-14)
    # g_idx under a real permutation
    key2 = rng.uniform(size=n)
    out = oracle.gptq_layer(W, H, key2, 4, g, False, desc_act=True, damp_percent=0.01)
    gidx, perm = out["g_idx"], out["perm"]
    counts = np.bincount(gidx)
    assert counts.tolist() == [16, 16, 8]
    for p in range(n):
        assert gidx[perm[p]] == p // g


def test_g_idx_hand_example():
    assert oracle.g_index(np.array([2, 0, 1, 3]), 2).tolist() == [0, 1, 0, 1]
    assert oracle.g_index(np.array([2, 0, 1]), -1).tolist() == [0, 0, 0]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_brute_force_optimum_bounds_gptq(n):
    # damping 0 and one group spanning the row: the grid is fixed by the
    # original weights, so every code vector can be enumerated
    rng = np.random.default_rng(20 + n)
    for trial in range(4):
        A = rng.standard_normal((n, n + 1))
        H = A @ A.T + 0.1 * np.eye(n)
        W = rng.standard_normal((1, n)) * 0.3
        out = oracle.gptq_layer(W, H, None, 2, -1, False, desc_act=False, damp_percent=0.0)
        s, z = out["scales"][0, 0], out["zeros"][0, 0]
        best = np.inf
        for qs in itertools.product(range(4), repeat=n):
            d = W[0] - (np.array(qs) - z) * s
            best = min(best, 0.5 * float(d @ H @ d))
        assert best <= out["loss0"] * (1 + 1e-12) + 1e-15
        if n == 1:
            assert out["loss0"] == pytest.approx(best, rel=1e-12)


def test_gptq_beats_rtn_in_aggregate_on_tiny_layer_shape():
    spec = workloads.CONFIGS["c1_tiny_256"]
    tot_g = tot_r = 0.0
    for seed in range(16):
        sp = spec.with_(w_seed=5000 + seed, x_seed=6000 + seed)
        W = workloads.to_numpy_f64(workloads.gen_weight(sp))
        X = np.concatenate([workloads.to_numpy_f64(t) for t in workloads.x_tiles(sp)])
        H, key = oracle.hessian([X], sp.n)
        out = oracle.gptq_layer(W, H, key, sp.bits, sp.group_size, sp.sym, sp.desc_act, sp.damp_percent)
        rtn = oracle.rtn_quantize(W, sp.bits, sp.group_size, sp.sym)
        qh = oracle.dequantize_layer(rtn["codes"], rtn["scales"], rtn["zeros"],
                                     oracle.g_index(np.arange(sp.n), sp.group_size))
        tot_g += float(np.sum(((W - out["Qhat"]) @ X.T) ** 2))
        tot_r += float(np.sum(((W - qh) @ X.T) ** 2))
    assert tot_g < tot_r


@pytest.mark.parametrize("sym", [False, True])
def test_width_one_last_group_has_zero_error(sym):
    rng = np.random.default_rng(9)
    m, g = 7, 4
    n = 2 * g + 1
    X = rng.standard_normal((50, n))
    W = rng.standard_normal((m, n)) * 0.1
    H, key = oracle.hessian([X], n)
    out = oracle.gptq_layer(W, H, key, 3, g, sym, desc_act=True, damp_percent=0.01)
    e_last = out["err_p"][:, -1]
    assert np.all(np.abs(e_last) <= 1e-15 * (1 + np.abs(W).max() / np.abs(out["U"][-1, -1])))


# ---------------------------------------------------------------------------
# Stage pins: Hessian, damping, act-order, inverse factor, packing
# ---------------------------------------------------------------------------
def test_hessian_brute_force_and_tiling():
    rng = np.random.default_rng(1)
    T, n = 7, 5
    X = rng.standard_normal((T, n))
    H, key = oracle.hessian([X[:3], X[3:]], n, alpha=2.0)
    for i in range(n):
        for j in range(n):
            acc = 0.0
            for t in range(T):
                acc += X[t, i] * X[t, j]
            assert H[i, j] == pytest.approx(2 * acc, rel=1e-13)
        assert key[i] == pytest.approx(2 * sum(X[t, i] ** 2 for t in range(T)), rel=1e-13)
    H1, key1 = oracle.hessian([X], n, alpha=0.5)
    np.testing.assert_allclose(H1 * 4, H, rtol=1e-13)
    np.testing.assert_allclose(key1 * 4, key, rtol=1e-13)
    # the key alone, tile by tile, without forming H
    k2 = oracle.hessian_diagonal_accumulate(np.zeros(n), X[:4])
    k2 = oracle.hessian_diagonal_accumulate(k2, X[4:])
    for i in range(n):
        assert k2[i] == pytest.approx(2 * sum(X[t, i] ** 2 for t in range(T)), rel=1e-13)


def test_damping_value_and_permuted_matrix():
    H = np.array([[1.0, 0.2, 0.1, 0.0], [0.2, 2.0, 0.3, 0.1], [0.1, 0.3, 3.0, 0.2], [0.0, 0.1, 0.2, 6.0]])
    key = np.diag(H).copy()
    Hp, perm, lam = oracle.damp_and_permute(H, key, 0.01, True)
    assert lam == pytest.approx(0.03, rel=1e-14)          # 1% of mean(1,2,3,6)
    assert perm.tolist() == [3, 2, 1, 0]
    for a in range(4):
        for b in range(4):
            want = H[perm[a], perm[b]] + (lam if perm[a] == perm[b] else 0.0)
            assert Hp[a, b] == want


def test_act_order_is_stable_on_ties():
    assert oracle.act_order(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), True).tolist() == [1, 2, 4, 3, 0]
    assert oracle.act_order(np.array([1.0, 3.0, 3.0]), False).tolist() == [0, 1, 2]


def test_inverse_factor_hand_case_and_library_inverse():
    U = oracle.inverse_upper_factor(np.array([[4.0, -2.5], [-2.5, 2.0]]))
    assert U[1, 0] == 0.0
    assert U[0, 0] == pytest.approx(np.sqrt(8 / 7), rel=1e-14)
    assert U[0, 1] == pytest.approx((10 / 7) / np.sqrt(8 / 7), rel=1e-14)
    assert U[1, 1] == pytest.approx(np.sqrt(0.5), rel=1e-14)
    rng = np.random.default_rng(2)
    Hp = _rand_spd(rng, 30)
    U = oracle.inverse_upper_factor(Hp)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U, np.linalg.inv(Hp), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(U @ Hp @ U.T, np.eye(30), atol=1e-10)


def test_not_positive_definite_is_an_error():
    with pytest.raises(oracle.NotPositiveDefinite):
        oracle.prepare(np.zeros((3, 3)), np.zeros(3), 0.01, True)
    with pytest.raises(oracle.NotPositiveDefinite):
        oracle.prepare(np.array([[1.0, 2.0], [2.0, 1.0]]), None, 0.0, False)


def test_pack_layout():
    Q = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 9]])
    qw = oracle.pack_codes(Q, 4)
    assert qw.tolist() == [[0x87654321, 0x9]]
    q8 = oracle.pack_codes(np.array([[1, 2, 3, 4, 5]]), 8)
    assert q8.tolist() == [[0x04030201, 0x05]]
    rng = np.random.default_rng(0)
    for bits in (2, 3, 4, 8):
        Q = rng.integers(0, 2 ** bits, size=(3, 21))
        assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(Q, bits), 21, bits), Q)


# ---------------------------------------------------------------------------
# Replay of another implementation's decisions (used by the full-size GPU
# parity): hand case with an exact half-way point.
#   row [1.25, -1.5, 6.0], 4-bit asym, one group: s = 7.5/15 = 0.5,
#   z = rne(1.5/0.5) = 3; column 0 sits at 1.25/0.5 + 3 = 5.5 exactly, which
#   rounds half-to-even to 6.  With U = [[1, .5, .25], [0, 1, .5], [0, 0, 1]]:
#   code 6 -> e0 = -0.25, column 1 at 0.25 -> 0, column 2 at 15 -> codes [6, 0, 15];
#   code 5 -> e0 = +0.25, column 1 at -0.25 -> 0, column 2 at 15 -> codes [5, 0, 15].
# ---------------------------------------------------------------------------
_TIE_W = np.array([[1.25, -1.5, 6.0]])
_TIE_U = np.array([[1.0, 0.5, 0.25], [0.0, 1.0, 0.5], [0.0, 0.0, 1.0]])


def test_replay_hand_tie():
    own = go.gptq_quantize(_TIE_W, _TIE_U, 4, -1, False)
    assert own["codes"].tolist() == [[6, 0, 15]]
    rep = go.gptq_quantize(_TIE_W, _TIE_U, 4, -1, False, forced=np.array([[5, 0, 15]]))
    assert rep["codes"].tolist() == [[5, 0, 15]]
    assert rep["replay"] == dict(flips=1, zero_flips=0, bad=0, max_tie_dist=0.0)
    assert rep["err"][0].tolist() == [0.25, -0.125, 0.0]
    for wrong in ([[7, 0, 15]], [[4, 0, 15]], [[6, 1, 15]]):
        r = go.gptq_quantize(_TIE_W, _TIE_U, 4, -1, False, forced=np.array(wrong))
        assert r["replay"]["bad"] >= 1, wrong


def test_replay_of_own_codes_changes_nothing():
    rng = np.random.default_rng(3)
    m, n = 6, 40
    A = rng.standard_normal((n, 2 * n))
    U, perm, lam = oracle.prepare(A @ A.T, None, 0.01, True)
    Wp = 0.02 * rng.standard_normal((m, n))
    own = go.gptq_quantize(Wp, U, 3, 8, True)
    rep = go.gptq_quantize(Wp, U, 3, 8, True, forced=own["codes"])
    assert rep["replay"] == dict(flips=0, zero_flips=0, bad=0, max_tie_dist=0.0)
    assert np.array_equal(rep["codes"], own["codes"]) and rep["loss0"] == own["loss0"]


# ---------------------------------------------------------------------------
# Exact rounding ties on the grid (round half to even of the real quotient,
# "模型量化实战：从 INT8 PTQ 到 GPTQ…" §2.1/§3.1 round; the exact route's
# Fraction arithmetic decides them independently)
# ---------------------------------------------------------------------------
def _bf16_grid(lo, hi, count):
    """count values of the bf16 grid in [lo, hi) (8 significant bits)."""
    out = []
    for e in range(-12, 2):
        for mant in range(128, 256):
            v = mant * 2.0 ** (e - 7)
            if lo <= v < hi:
                out.append(v)
    return out[::max(1, len(out) // count)][:count]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_symmetric_range_zero_point_tie_goes_to_even(bits):
    """max = -min puts the grid position of 0 exactly at (2^b - 1)/2; round
    half to even gives 2^(b-1) on every such range, as the exact route does,
    also where the float64 estimate -lo/s falls below the half-way point."""
    qmax = 2 ** bits - 1
    vals = _bf16_grid(0.001, 2.0, 400)
    v = np.array([[a, -a, 0.375 * a] for a in vals])
    s, z, lo, hi = go.group_params(v, bits, False)
    assert z.tolist() == [2 ** (bits - 1)] * len(vals)
    for row, zz in zip(v[:40], z[:40]):
        assert exact_obs.grid([Fraction(float(x)) for x in row], bits, False)[1] == zz
    below = [a for a in vals if a / ((2 * a) / qmax) < qmax / 2]
    print(f"{bits}-bit: {len(below)} of {len(vals)} float64 estimates below the tie")
    if bits > 2:
        assert below, "no case where the float64 estimate alone would round down"


def test_code_ties_match_exact_route():
    """Every dyadic (lo, hi, w) on a 1/32 grid whose exact grid position is a
    half-integer (2476 cases at 3 and 4 bits): codes equal the exact route's,
    although the plain float64 quotient rounds the other way on some."""
    cases, wrong64 = 0, 0
    g = [i / 32 for i in range(-32, 33)]
    for bits in (3, 4):
        qmax = 2 ** bits - 1
        los, his, ws = [], [], []
        for lo_ in (x for x in g if x < 0):
            for hi_ in (x for x in g if x > 0):
                step = (Fraction(hi_) - Fraction(lo_)) / qmax
                z = round(-Fraction(lo_) / step)
                for w in g:
                    x = Fraction(w) / step + z
                    if x.denominator == 2 and 0 < x < qmax:
                        los.append(lo_), his.append(hi_), ws.append(w)
        lo_a, hi_a, w_a = map(np.array, (los, his, ws))
        s = (hi_a - lo_a) / qmax
        _, z, _, _ = go.group_params(np.stack([lo_a, hi_a], axis=1), bits, False)
        q = go.quantize_values(w_a, s, z, bits, False, lo_a, hi_a)
        for i in range(len(ws)):
            sf, zf = exact_obs.grid([Fraction(los[i]), Fraction(his[i])], bits, False)
            assert q[i] == exact_obs.code(Fraction(ws[i]), sf, zf, bits, False), (los[i], his[i], ws[i])
        wrong64 += int(np.sum(np.rint(w_a / s + z) != q))
        cases += len(ws)
    print(f"{cases} exact code ties; plain float64 rounding differs on {wrong64}")
    assert cases == 2476 and wrong64 > 0


def test_replay_accepts_zero_point_flips_only_at_ties():
    """Row [-0.75, 0.75, 0.3], 4-bit asym, one group: step 0.1, the position
    of 0 is 7.5 exactly, so the oracle takes z = 8 and a replayed z = 7 is a
    tie flip; z = 6 is not.  A symmetric grid's fixed offset never flips."""
    W = np.array([[-0.75, 0.75, 0.3]])
    U = np.eye(3)
    own = go.gptq_quantize(W, U, 4, -1, False)
    assert own["zeros"].tolist() == [[8]]
    rep = go.gptq_quantize(W, U, 4, -1, False, forced_zeros=np.array([[7]]))
    assert rep["zeros"].tolist() == [[7]]
    assert rep["replay"]["zero_flips"] == 1 and rep["replay"]["bad"] == 0
    assert rep["replay"]["max_tie_dist"] <= 1e-12
    # codes follow the adopted zero: -0.75/0.1 + 7 = -0.5 -> 0, 0.75/0.1 + 7 = 14.5 -> 14
    assert rep["codes"][0, :2].tolist() == [0, 14]
    bad = go.gptq_quantize(W, U, 4, -1, False, forced_zeros=np.array([[6]]))
    assert bad["replay"]["bad"] == 1
    sym = go.gptq_quantize(W, U, 4, -1, True, forced_zeros=np.array([[7]]))
    assert sym["replay"]["bad"] == 1
