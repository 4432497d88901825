"""Exact rational GPTQ by a second route, used only to pin the oracle.

The oracle spreads each column's error with a row of U, the upper Cholesky
factor of H⁻¹.  This module does not use U at all: for every column c it
inverts the Hessian restricted to the columns still to be quantized (the
optimal-brain-surgeon form the GPTQ section of "大模型量化：GPTQ/AWQ/GGUF
原理对比" describes: the error of a quantized column is pushed onto the
remaining columns in proportion to the inverse Hessian).  All arithmetic is
in ``fractions.Fraction``, so no rounding error enters the weights, scales
and errors, and the loss is the exact ½·d²/[H_F⁻¹]_cc sum.

Python's ``round`` of a Fraction rounds half to even, like numpy's, so the
zero point and each code are the exact round-half-to-even of their
definition on the exact grid step.
"""
from __future__ import annotations

from fractions import Fraction

SCALE_FLOOR = Fraction(1e-8)


def as_frac(x):
    return x if isinstance(x, Fraction) else Fraction(x)


def inverse(M):
    """Gauss-Jordan inverse of a square matrix of Fractions."""
    n = len(M)
    A = [[as_frac(v) for v in row] + [Fraction(int(i == j)) for j in range(n)]
         for i, row in enumerate(M)]
    for col in range(n):
        piv = next(r for r in range(col, n) if A[r][col] != 0)
        A[col], A[piv] = A[piv], A[col]
        p = A[col][col]
        A[col] = [v / p for v in A[col]]
        for r in range(n):
            if r != col and A[r][col] != 0:
                f = A[r][col]
                A[r] = [a - f * b for a, b in zip(A[r], A[col])]
    return [row[n:] for row in A]


def grid(vals, bits, sym):
    """(scale, zero) of one group, exactly."""
    if sym:
        qmax = 2 ** (bits - 1) - 1
        s = max(max(abs(v) for v in vals) / qmax, SCALE_FLOOR)
        return s, Fraction(2 ** (bits - 1))
    lo = min(min(vals), Fraction(0))
    hi = max(max(vals), Fraction(0))
    s = max((hi - lo) / (2 ** bits - 1), SCALE_FLOOR)
    return s, Fraction(round(-lo / s))


def code(w, s, z, bits, sym):
    if sym:
        qmax = 2 ** (bits - 1) - 1
        return min(max(round(w / s), -qmax), qmax) + int(z)
    return min(max(round(w / s + z), 0), 2 ** bits - 1)


def gptq_exact(W, H, bits, group, sym):
    """GPTQ in processing order 0..n-1 (no act-order), exact.

    Returns (codes, scales, zeros, loss0) with codes[r][c] the stored code.
    """
    W = [[as_frac(v) for v in row] for row in W]
    H = [[as_frac(v) for v in row] for row in H]
    m, n = len(W), len(H)
    gw = n if group == -1 else group
    codes = [[0] * n for _ in range(m)]
    scales = [[None] * ((n + gw - 1) // gw) for _ in range(m)]
    zeros = [[None] * ((n + gw - 1) // gw) for _ in range(m)]
    loss = Fraction(0)
    # inverse of H restricted to the columns not yet quantized, per step
    inv_rest = [inverse([row[c:] for row in H[c:]]) for c in range(n)]
    for r in range(m):
        w = list(W[r])
        s = z = None
        for c in range(n):
            if c % gw == 0:
                s, z = grid(w[c:min(c + gw, n)], bits, sym)
                scales[r][c // gw] = s
                zeros[r][c // gw] = z
            q = code(w[c], s, z, bits, sym)
            codes[r][c] = q
            d = w[c] - (q - z) * s
            Hi = inv_rest[c]
            loss += d * d / (2 * Hi[0][0])
            for k in range(c + 1, n):
                w[k] -= d * Hi[k - c][0] / Hi[0][0]
    return codes, scales, zeros, loss


def rtn_exact(W, bits, group, sym):
    W = [[as_frac(v) for v in row] for row in W]
    m, n = len(W), len(W[0])
    gw = n if group == -1 else group
    codes = [[0] * n for _ in range(m)]
    for r in range(m):
        for c0 in range(0, n, gw):
            s, z = grid(W[r][c0:c0 + gw], bits, sym)
            for c in range(c0, min(c0 + gw, n)):
                codes[r][c] = code(W[r][c], s, z, bits, sym)
    return codes


def quad_loss(W, Qhat, H):
    """½·Σ_r (w_r - q̂_r) H (w_r - q̂_r)ᵀ, exactly."""
    tot = Fraction(0)
    n = len(H)
    for wr, qr in zip(W, Qhat):
        d = [as_frac(a) - as_frac(b) for a, b in zip(wr, qr)]
        tot += sum(d[i] * as_frac(H[i][j]) * d[j] for i in range(n) for j in range(n))
    return tot / 2
