"""Plain float64 CPU oracle of the page's linear (round-to-nearest) quantizer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or constant generator with the HIP library.

Written from page "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析"
(qwbw.cn/news/15203): §2.1 (the affine formula x_q = round(x/scale + zp),
x = (x_q - zp)·scale) and §3.1 (the LinearQuantizer: symmetric or asymmetric
grid, per-channel granularity, clip_ratio percentile clipping, the 1e-8 scale
floor, quantize / dequantize, and quantization_error = (MSE, cosine
similarity)).  The worked INT8 example of page "大模型量化：GPTQ/AWQ/GGUF 原理
对比…" (section on quantization basics) pins the symmetric grid.

Readings taken where the page is silent, garbled or loose (also listed in the
design notes of the repository):
  * L1 "per channel" means per output row of the [m, n] weight (the page's
    comment says output channel; its code reduces along axis 0).  Per-group
    granularity (g consecutive columns of a row) is added; g = -1 is one
    group per row.
  * L2 percentile(v, f) is linear interpolation between order statistics:
    sorted a[0..N-1], position p = f·(N-1), i = floor(p), t = p - i,
    value a[i] + (a[i+1] - a[i])·t (a[N-1] when i = N-1).  This is the
    interpolation the page's NumPy call uses by default.
  * L3 symmetric: amax = percentile(|w|, c) for clip ratio c < 1, else
    max|w| (the same value); scale = amax / (2^(b-1) - 1); codes
    rne(w/scale) clamped to [-2^(b-1), 2^(b-1) - 1] (the page's qmin/qmax).
  * L4 asymmetric: lo = percentile(w, (1-c)/2), hi = percentile(w, 1-(1-c)/2)
    for c < 1, else min and max (the same values); scale = (hi - lo) /
    (2^b - 1); zp = -rne(lo / scale); codes rne(w/scale + zp) clamped to
    [0, 2^b - 1].  The range is not widened to include 0 (the page's
    LinearQuantizer does not), so zp may lie outside [0, 2^b - 1].
  * L5 scale floor 1e-8 in both modes (the page applies it after the
    asymmetric branch; an all-zero symmetric group would otherwise divide by
    zero).
  * L6 all grid and code arithmetic in float64 (the page's NumPy computes
    percentiles in float64); rne = round half to even.
  * L7 MSE = mean over all m·n elements of (w - ŵ)²; cosine =
    Σ w·ŵ / (‖w‖·‖ŵ‖ + 1e-8), ŵ = (q - zp)·scale with the float64 scale.
  * L8 storage as in the GPTQ path: symmetric codes offset by 2^(b-1) (the
    stored zero is then 2^(b-1)), asymmetric codes as they are with zp as
    the stored zero, so ŵ = (stored code - stored zero)·scale in both modes.
"""
from __future__ import annotations

import numpy as np

SCALE_FLOOR = 1e-8


def percentile_linear(values, frac):
    """Reading L2: linear interpolation between the order statistics of
    `values` at fractional position frac·(N-1)."""
    a = np.sort(np.asarray(values, dtype=np.float64).ravel())
    N = a.size
    if N == 0:
        raise ValueError("percentile of an empty set")
    p = float(frac) * (N - 1)
    i = int(np.floor(p))
    if i >= N - 1:
        return float(a[N - 1])
    t = p - i
    return float(a[i] + (a[i + 1] - a[i]) * t)


def linear_grid(v, bits, sym, clip_ratio):
    """Scale and zero point of one group of values (§3.1 _compute_scale_zp,
    readings L3-L5).  Returns (scale, zp, qmin, qmax); zp = 0 when sym."""
    v = np.asarray(v, dtype=np.float64).ravel()
    c = float(clip_ratio)
    if sym:
        qmax = 2 ** (bits - 1) - 1
        qmin = -(2 ** (bits - 1))
        amax = percentile_linear(np.abs(v), c) if c < 1.0 else float(np.max(np.abs(v)))
        scale = max(amax / qmax, SCALE_FLOOR)
        return scale, 0.0, qmin, qmax
    qmin, qmax = 0, 2 ** bits - 1
    if c < 1.0:
        f = (1.0 - c) / 2.0
        lo = percentile_linear(v, f)
        hi = percentile_linear(v, 1.0 - f)
    else:
        lo, hi = float(np.min(v)), float(np.max(v))
    scale = max((hi - lo) / (qmax - qmin), SCALE_FLOOR)
    zp = qmin - float(np.rint(lo / scale))
    return scale, zp, qmin, qmax


def linear_codes(v, scale, zp, qmin, qmax, sym):
    """Signed (sym) or unsigned (asym) codes of one group (§2.1, §3.1)."""
    v = np.asarray(v, dtype=np.float64)
    if sym:
        q = np.rint(v / scale)
    else:
        q = np.rint(v / scale + zp)
    return np.clip(q, qmin, qmax)


def linear_quantize(W, bits, sym, group_size, clip_ratio):
    """The page's LinearQuantizer applied per output row (group_size = -1) or
    per group of `group_size` consecutive columns of a row.

    W: [m, n] float (converted exactly to float64).  Returns a dict with the
    stored codes [m, n] int64 (reading L8), scales [m, G] float64, stored
    zeros [m, G] int64, the dequantized weights, mse and cos (reading L7).
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    g = n if group_size == -1 else int(group_size)
    G = (n + g - 1) // g
    off = 2 ** (bits - 1) if sym else 0
    codes = np.zeros((m, n), dtype=np.int64)
    scales = np.zeros((m, G), dtype=np.float64)
    zeros = np.zeros((m, G), dtype=np.int64)
    deq = np.zeros((m, n), dtype=np.float64)
    for r in range(m):
        for j in range(G):
            c0, c1 = j * g, min((j + 1) * g, n)
            v = W[r, c0:c1]
            s, zp, qmin, qmax = linear_grid(v, bits, sym, clip_ratio)
            q = linear_codes(v, s, zp, qmin, qmax, sym)
            codes[r, c0:c1] = q.astype(np.int64) + off
            scales[r, j] = s
            zeros[r, j] = int(zp) + off
            deq[r, c0:c1] = (q - zp) * s
    err = W - deq
    mse = float(np.mean(err * err)) if W.size else 0.0
    dot = float(np.sum(W * deq))
    cos = dot / (np.sqrt(float(np.sum(W * W))) * np.sqrt(float(np.sum(deq * deq))) + 1e-8)
    return {"codes": codes, "scales": scales, "zeros": zeros, "deq": deq, "mse": mse, "cos": cos}
