"""Plain float64 CPU oracle of the quantized-weight matrix product (W4A16).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or constant generator with the HIP library.

Written from page "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析"
(qwbw.cn/news/15203): §2.1 (dequantization x = (x_q - zero_point)·scale) and
§4.3 (INT4 weights have no native matrix product: they are dequantized to a
16-bit type and then multiplied; the gain is the 4x smaller weight traffic).

The product of activations X [T, n] with the quantizer's output (codes in
original column order, per-row per-group scale and zero, g_idx giving each
input column's group) is, by that definition,
    Y[t, r] = Σ_k X[t, k] · (q[r, k] - z[r, g_idx[k]]) · s[r, g_idx[k]],
computed here exactly as written (dequantize, then one matrix product) in
float64 from the exact bytes the GPU reads.
"""
from __future__ import annotations

import numpy as np

from .gptq_oracle import dequantize_layer, unpack_codes


def dequantized_weight(qweight, scales, zeros, g_idx, n, bits):
    """Ŵ [m, n] float64 from packed codes (uint32 words, the quantizer's
    nibble / byte layout), scales [m, G], zeros [m, G] and g_idx [n]."""
    Q = unpack_codes(np.asarray(qweight).view(np.uint32), n, bits).astype(np.float64)
    return dequantize_layer(Q, np.asarray(scales, dtype=np.float64),
                            np.asarray(zeros, dtype=np.float64), np.asarray(g_idx, dtype=np.int64))


def dequant_matmul(X, qweight, scales, zeros, g_idx, n, bits):
    """Y [T, m] = X [T, n] · Ŵᵀ in float64 (§4.3: dequantize, then multiply)."""
    X = np.asarray(X, dtype=np.float64)
    return X @ dequantized_weight(qweight, scales, zeros, g_idx, n, bits).T
