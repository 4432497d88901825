"""Plain float64 CPU oracle of the pages' activation-aware channel scaling (AWQ).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or constant generator with the HIP library.

Written from page "大模型量化：GPTQ/AWQ/GGUF 原理对比，4-bit 量化对推理精度的影响"
(lwxnote.com), section on AWQ (the awq_quantize sketch and the explanation
after it): each input channel's importance is the mean absolute activation
over the calibration tokens; channels whose importance exceeds the median
are multiplied by a protection factor s (2.0 by default), the others by 1;
the scaled weight is quantized; dequantizing divides by the channel scale
again, and at inference the activations are divided by it.

Readings taken where the page is silent (also listed in the design notes):
  * A1 the quantizer the sketch calls is the pages' LinearQuantizer
    (page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.1, oracle.linear_quantizer),
    per output row or per group, with its own sym / clip settings.
  * A2 median is torch.median's: for an even count the lower of the two
    middle values, sorted[(n-1)//2]; a channel is important when its
    importance is strictly greater.
  * A3 importance = Σ_t |x_t| / T in float64 (the sum over tokens is
    accumulated in float64 from the exact activation values).
  * A4 the scaled weight is the float32 product fl(w·scale) (the sketch
    multiplies two float tensors); with s a power of two it is exact.
  * A5 the returned error is the LinearQuantizer's quantization_error (MSE
    and cosine) between W and the dequantized weight divided by the channel
    scale, ŵ = (q - zp)·scale_row / scale_channel, in float64.
"""
from __future__ import annotations

import numpy as np

from .linear_quantizer import linear_quantize


def channel_abs_sum(X):
    """Σ_t |x_t| per input channel (float64) of activations X [T, n]."""
    return np.sum(np.abs(np.asarray(X, dtype=np.float64)), axis=0)


def lower_median(v):
    """torch.median of a 1-D array: the lower middle value (reading A2)."""
    a = np.sort(np.asarray(v, dtype=np.float64).ravel())
    if a.size == 0:
        raise ValueError("median of an empty set")
    return float(a[(a.size - 1) // 2])


def channel_scale(abs_sum, tokens, s=2.0):
    """Per-channel scale: s where mean|x| exceeds its median, else 1 (float32)."""
    importance = np.asarray(abs_sum, dtype=np.float64) / float(tokens)
    med = lower_median(importance)
    scale = np.ones(importance.shape, dtype=np.float32)
    scale[importance > med] = np.float32(s)
    return scale, importance, med


def awq_quantize(W, abs_sum, tokens, s=2.0, bits=4, sym=False, group_size=128, clip_ratio=1.0):
    """The sketch's steps: importance, median mask, scale, quantize W·scale,
    dequantize / scale.  W [m, n]; abs_sum [n] = Σ_t |x_t| over `tokens`
    calibration tokens.  Returns the LinearQuantizer's codes / scales / zeros
    of the scaled weight, the channel scale, the dequantized weight in the
    original domain, and (mse, cos) against W."""
    W = np.asarray(W, dtype=np.float64)
    scale, importance, med = channel_scale(abs_sum, tokens, s)
    W_scaled = (W.astype(np.float32) * scale[None, :]).astype(np.float64)
    q = linear_quantize(W_scaled, bits, sym, group_size, clip_ratio)
    What = q["deq"] / scale.astype(np.float64)[None, :]
    err = W - What
    mse = float(np.mean(err * err)) if W.size else 0.0
    cos = float(np.sum(W * What)) / (np.sqrt(float(np.sum(W * W))) * np.sqrt(float(np.sum(What * What))) + 1e-8)
    return {"codes": q["codes"], "scales": q["scales"], "zeros": q["zeros"], "channel_scale": scale,
            "importance": importance, "median": med, "deq": What, "mse": mse, "cos": cos}
