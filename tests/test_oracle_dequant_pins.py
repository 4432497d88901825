"""Pins of the quantized-weight matrix product oracle (oracle/quantized_matmul.py),
CPU only: a hand-worked case, the exact link to the quantizer's own loss, a
brute-force product that reads the packed words bit by bit, and zero codes."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import quantized_matmul as dm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_hand_case():
    g = _load("w4a16_hand_case.json")
    qw = np.array([[int(h, 16)] for h in g["qweight_hex"]], dtype=np.uint32)
    assert oracle.g_index(np.array(g["perm_processing_order"]), g["group_size"]).tolist() == g["g_idx"]
    What = dm.dequantized_weight(qw, g["scales"], g["zeros"], g["g_idx"], 8, g["bits"])
    assert What.tolist() == g["dequantized"]
    Y = dm.dequant_matmul(g["X"], qw, g["scales"], g["zeros"], g["g_idx"], 8, g["bits"])
    assert Y.tolist() == g["Y"]


@pytest.mark.parametrize("bits,group,sym", [(4, 4, False), (3, 8, False), (2, 4, True), (8, -1, False)])
def test_product_error_is_the_quantizers_loss(bits, group, sym):
    """With H = 2·XᵀX the quantizer's loss satisfies ½·tr(ΔW (H + λI) ΔWᵀ) =
    ‖X ΔWᵀ‖² + (λ/2)‖ΔW‖², so ‖X Wᵀ - Y‖² = loss0 - (λ/2)·loss1 for the
    product Y of X with the packed output (the quantizer's loss0 is its own
    ½Σe², computed in processing order without this module)."""
    rng = np.random.default_rng(bits * 10 + (group if group > 0 else 99))
    T, n, m = 60, 24, 5
    X = rng.standard_normal((T, n)) * rng.uniform(0.2, 3.0, n)
    W = rng.standard_normal((m, n)) * 0.1
    H, key = oracle.hessian([X], n)
    out = oracle.gptq_layer(W, H, key, bits, group, sym, desc_act=True, damp_percent=0.01)
    qw = oracle.pack_codes(out["codes"], bits)
    Y = dm.dequant_matmul(X, qw, out["scales"], out["zeros"], out["g_idx"], n, bits)
    lhs = float(np.sum((X @ W.T - Y) ** 2))
    assert lhs == pytest.approx(out["loss0"] - 0.5 * out["lam"] * out["loss1"], rel=1e-9)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_brute_force_from_packed_words(bits):
    rng = np.random.default_rng(bits)
    T, n, m, g = 3, 13, 4, 4
    G = (n + g - 1) // g
    Q = rng.integers(0, 2 ** bits, size=(m, n))
    qw = oracle.pack_codes(Q, bits)
    scales = rng.uniform(0.01, 0.5, size=(m, G))
    zeros = rng.integers(0, 2 ** bits, size=(m, G))
    gidx = rng.permutation(np.arange(n) // g)
    X = rng.standard_normal((T, n))
    per, width = (8, 4) if bits <= 4 else (4, 8)
    Y_bf = np.zeros((T, m))
    for t in range(T):
        for r in range(m):
            acc = 0.0
            for k in range(n):
                word = int(qw[r, k // per])
                q = (word >> (width * (k % per))) & ((1 << width) - 1)
                acc += float(X[t, k]) * (q - int(zeros[r, gidx[k]])) * float(scales[r, gidx[k]])
            Y_bf[t, r] = acc
    Y = dm.dequant_matmul(X, qw, scales, zeros, gidx, n, bits)
    np.testing.assert_allclose(Y, Y_bf, rtol=1e-12, atol=1e-12)


def test_codes_at_the_zero_point_give_zero():
    rng = np.random.default_rng(5)
    m, n, g = 3, 16, 8
    zeros = rng.integers(0, 16, size=(m, 2))
    gidx = rng.permutation(np.arange(n) // g)
    Q = zeros[:, gidx]
    Y = dm.dequant_matmul(rng.standard_normal((4, n)), oracle.pack_codes(Q, 4), rng.uniform(0.1, 1, (m, 2)),
                          zeros, gidx, n, 4)
    assert np.all(Y == 0.0)
