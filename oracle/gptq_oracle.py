"""Plain float64 CPU oracle of the GPTQ layer-quantization path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or constant generator with the HIP library.

It is written step by step from these web pages (cited by title and section):

  [P3] "Llama-2 GPTQ quantization in practice" (mjmagnets.cn/news/197986):
       §2.1 layer objective, §2.2.1 Hessian from calibration activations,
       §3.3 quantize_config {bits, group_size, damp_percent, desc_act}.
  [P4] "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析"
       (qwbw.cn/news/15203): §2.1 affine quantization formula, §3.1 the
       LinearQuantizer (sym / asym, scale floor), §3.2 the GPTQQuantizer
       sketch (accumulate_hessian, prepare, quantize_block).
  [P5] "大模型量化：GPTQ/AWQ/GGUF 原理对比，4-bit 量化对推理精度的影响"
       (lwxnote.com): section "quantization basics" (symmetric INT8 worked
       example), section "GPTQ: Hessian + error compensation" (column-by-column
       quantization and the compensation flow).
  [P2] "GPTQ量化损失深度解析" (bmjup.com/post/14319): desc_act sorts columns by
       sensitivity, group_size 128, sym=False.
  [P1] "Qwen2.5模型GPTQ量化精度损失实测" (m.cn486.com): act-order reorders
       weights.

Everything is float64.  Inputs arrive as the exact bytes the GPU consumed
(bf16 / fp32, converted exactly to float64).

Readings taken where the pages are silent, garbled or contradict each other
(each one is also listed in the design notes of the repository):
  * H is the plain sum 2·XᵀX, no 1/T ([P4] §3.2; [P3] §2.2.1 writes an
    expectation, which only rescales H and the loss).
  * damping λ = p·mean(diag H), added before any factorisation ([P4] §3.2).
  * The inverse factor is the upper Cholesky factor of H⁻¹, taken once
    ([P4] §3.2 applies the factorisation twice, which is a slip).
  * Column c's error is spread with row c of that factor (the sketches in
    [P4] §3.2 and [P5] use a row index of the output or a static inverse).
  * Scale and zero are per output row and per group of g consecutive
    processed columns, fixed at the group's first column from the current
    (already compensated) weights; g = -1 is one group per row.
  * asym range is widened to include 0: [min(w,0), max(w,0)], so the zero
    point is an integer in [0, 2^b-1] and 0 is exact.
  * sym clamp is ±(2^(b-1)-1) ([P5]); codes are stored offset by 2^(b-1).
  * rounding is round-half-to-even (numpy / torch round).  asym codes are
    rne(w/s + z) as [P4] §2.1 and §3.1 write it; sym codes are rne(w/s).
  * scale floor 1e-8 ([P4] §3.1).
  * the two integers the grid decides, each zero point and each code, are
    the exact round-half-to-even of their real-valued definition on the
    exact grid step (hi - lo)/(2^b - 1) (sym: max|w|/(2^(b-1) - 1)), not of
    a rounded copy of it: a float64 estimate decides, and wherever it lies
    too close to a half-integer for its rounding error to be ruled out, the
    quotient is evaluated in exact rational arithmetic.  The stored scale is
    that step rounded to float64.  So a range with max = -min puts the zero
    point exactly at (2^b - 1)/2 and it goes to the even neighbour.
  * desc_act: stable sort of the diagonal of H, descending, ties to the lower
    original column index.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import scipy.linalg

SCALE_FLOOR = 1e-8


class NotPositiveDefinite(ValueError):
    """The damped, permuted Hessian has no Cholesky factorisation."""


# ---------------------------------------------------------------------------
# Stage 1: Hessian accumulation  ([P4] §3.2 accumulate_hessian; [P3] §2.2.1)
# ---------------------------------------------------------------------------
def hessian_accumulate(H, key, X, alpha=2.0):
    """Return (H + alpha·XᵀX, key + alpha·Σ_t x_t²) in float64.

    X is one token tile [tokens, n] (rows are calibration tokens, the layer's
    input activations).  H is the running Hessian [n, n]; key is the running
    diagonal, kept separately so that the act-order sort sees it in float64.
    Calling this once per tile over all tiles equals one call on the whole X.
    """
    X = np.asarray(X, dtype=np.float64)
    S = X.T @ X                       # Σ_t x_t x_tᵀ
    H = np.asarray(H, dtype=np.float64) + alpha * S
    key = np.asarray(key, dtype=np.float64) + alpha * np.einsum("ti,ti->i", X, X)
    return H, key


def hessian_diagonal_accumulate(key, X, alpha=2.0):
    """key + alpha·Σ_t x_t² (the diagonal of alpha·XᵀX) in float64, without
    forming H: the act-order key of a layer too wide for the full product."""
    X = np.asarray(X, dtype=np.float64)
    return np.asarray(key, dtype=np.float64) + alpha * np.einsum("ti,ti->i", X, X)


def hessian(x_tiles, n, alpha=2.0):
    """H = alpha·XᵀX and its diagonal key, accumulated over an iterable of tiles."""
    H = np.zeros((n, n))
    key = np.zeros(n)
    for X in x_tiles:
        H, key = hessian_accumulate(H, key, X, alpha)
    return H, key


# ---------------------------------------------------------------------------
# Stage 2: damping and act-order  ([P4] §3.2 prepare; [P2]; [P1])
# ---------------------------------------------------------------------------
def damping(key, damp_percent):
    """λ = damp_percent · mean(diag H)."""
    return float(damp_percent) * float(np.mean(np.asarray(key, dtype=np.float64)))


def act_order(key, desc_act):
    """perm[p] = original column processed at position p.

    desc_act: columns by descending diag(H), stable (equal keys keep their
    original order).  Otherwise the identity.
    """
    key = np.asarray(key, dtype=np.float64)
    if not desc_act:
        return np.arange(key.shape[0], dtype=np.int64)
    return np.argsort(-key, kind="stable").astype(np.int64)


def damp_and_permute(H, key, damp_percent, desc_act):
    """Return (H_p, perm, lam): H_p = P (H + λI) Pᵀ in processing order."""
    H = np.asarray(H, dtype=np.float64)
    if key is None:
        key = np.diag(H).copy()
    lam = damping(key, damp_percent)
    Hd = H + lam * np.eye(H.shape[0])
    perm = act_order(key, desc_act)
    Hp = Hd[np.ix_(perm, perm)]
    return Hp, perm, lam


# ---------------------------------------------------------------------------
# Stage 3: inverse factor  ([P4] §3.2 prepare, with the factorisation once)
# ---------------------------------------------------------------------------
def inverse_upper_factor(Hp):
    """U upper triangular with positive diagonal and UᵀU = Hp⁻¹.

    The route the page names: L = chol(Hp); Hp⁻¹ = L⁻ᵀL⁻¹ (the Cholesky
    inverse); U = upper Cholesky factor of Hp⁻¹.
    """
    Hp = np.asarray(Hp, dtype=np.float64)
    n = Hp.shape[0]
    if n == 0:
        return np.zeros((0, 0))
    try:
        L = np.linalg.cholesky(Hp)
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    Linv = scipy.linalg.solve_triangular(L, np.eye(n), lower=True)
    Hinv = Linv.T @ Linv
    Hinv = 0.5 * (Hinv + Hinv.T)
    try:
        U = np.linalg.cholesky(Hinv).T
    except np.linalg.LinAlgError as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    return U


def prepare(H, key, damp_percent, desc_act):
    """Stages 2 and 3 together: (U, perm, lam)."""
    Hp, perm, lam = damp_and_permute(H, key, damp_percent, desc_act)
    if not np.all(np.isfinite(Hp)):
        raise ValueError("non-finite Hessian")
    return inverse_upper_factor(Hp), perm, lam


# ---------------------------------------------------------------------------
# The quantization grid  ([P4] §2.1, §3.1; [P5] quantization basics)
# ---------------------------------------------------------------------------
# A float64 estimate x of a grid position carries four roundings (the range
# width, the step, the quotient, adding the zero point), so it is within
# 4·2^-53·(|w/step| + |x|) of the exact value: below 2.3e-13 wherever the
# rounding is not clamped away on a grid of at most 255 steps.  Positions
# estimated closer than the filter bound 1e-12·(1 + |x|) to a half-integer
# are re-evaluated exactly, so every rounding below is the exact
# round-half-to-even of the real number the definition names.
_TIE_FILTER = 1e-12


def _exact_step(lo, hi, qmax):
    """The exact grid step (hi - lo)/qmax of float64 range ends, floored at
    1e-8 (the floor as the float64 constant), as a Fraction."""
    step = (Fraction(float(hi)) - Fraction(float(lo))) / qmax
    return max(step, Fraction(SCALE_FLOOR))


def _rne(x, exact_at):
    """Round half to even of real numbers whose float64 estimates are x.

    Where an estimate lies within the filter bound of a half-integer, the
    value exact_at(index) (a Fraction) is rounded instead; Python's round of
    a Fraction is round-half-to-even."""
    x = np.asarray(x, dtype=np.float64)
    q = np.rint(x)
    near = np.abs((x - np.floor(x)) - 0.5) <= _TIE_FILTER * (1.0 + np.abs(x))
    for idx in zip(*np.nonzero(near)):
        q[idx] = float(round(exact_at(idx)))
    return q


def _qmax(bits, sym):
    return 2 ** (bits - 1) - 1 if sym else 2 ** bits - 1


def group_params(v, bits, sym):
    """Per-row grid of one group of current weights v [m, w]: (s, z, lo, hi).

    asym: range [lo, hi] = [min(v,0), max(v,0)] split into 2^b-1 steps; the
          zero point is the rounded position of 0 on that grid, rne(-lo/step).
    sym:  step = max|v| / (2^(b-1)-1) (lo = 0, hi = max|v|); the zero is the
          storage offset 2^(b-1).
    The step is floored at 1e-8.  s is the step rounded to float64 (the
    stored scale); lo and hi define the exact step for the decisions.
    """
    v = np.asarray(v, dtype=np.float64)
    qmax = _qmax(bits, sym)
    if sym:
        lo = np.zeros(v.shape[0])
        hi = np.max(np.abs(v), axis=1)
    else:
        lo = np.minimum(np.min(v, axis=1), 0.0)
        hi = np.maximum(np.max(v, axis=1), 0.0)
    s = np.maximum((hi - lo) / qmax, SCALE_FLOOR)
    if sym:
        z = np.full(v.shape[0], float(2 ** (bits - 1)))
    else:
        z = _rne(-lo / s, lambda i: -Fraction(float(lo[i])) / _exact_step(lo[i], hi[i], qmax))
    return s, z, lo, hi


def quantize_values(w, s, z, bits, sym, lo=None, hi=None):
    """Stored integer code of w on the grid (s, z); all arrays broadcast.

    asym: rne(w/step + z) clamped to [0, 2^b-1]; sym: rne(w/step) clamped to
    ±(2^(b-1)-1), plus the offset z.  step is the exact (hi - lo)/qmax when
    the range ends are given, else s itself."""
    w, s, z = np.broadcast_arrays(*(np.asarray(a, dtype=np.float64) for a in (w, s, z)))
    qmax = _qmax(bits, sym)
    if lo is None:
        def step(i):
            return Fraction(float(s[i]))
    else:
        lo_b, hi_b = np.broadcast_arrays(np.asarray(lo, dtype=np.float64), np.asarray(hi, dtype=np.float64))
        lo_b, hi_b = np.broadcast_to(lo_b, w.shape), np.broadcast_to(hi_b, w.shape)

        def step(i):
            return _exact_step(lo_b[i], hi_b[i], qmax)
    if sym:
        q = _rne(w / s, lambda i: Fraction(float(w[i])) / step(i))
        return np.clip(q, -qmax, qmax) + z
    q = _rne(w / s + z, lambda i: Fraction(float(w[i])) / step(i) + Fraction(float(z[i])))
    return np.clip(q, 0, qmax)


def dequantize_values(q, s, z):
    """x̂ = (q - z)·s  ([P4] §2.1)."""
    return (np.asarray(q, dtype=np.float64) - z) * s


# ---------------------------------------------------------------------------
# Stage 4: column-by-column quantization with error compensation
# ([P5] GPTQ section; [P4] §3.2 quantize_block)
# ---------------------------------------------------------------------------
def _group_width(g, n):
    return n if g == -1 else g


def gptq_quantize(Wp, U, bits, group_size, sym, block=None, forced=None, forced_zeros=None,
                  tie_tol=1e-4):
    """GPTQ on permuted weights Wp [m, n] with the inverse factor U [n, n].

    For each processed column c in order:
      * at the first column of a group, fix each row's (s, z) from the
        current weights of that group;
      * q = code of w_c; e = (w_c - x̂_c) / U[c,c]; the loss gains ½Σe²;
      * every later column k gets w_k -= e·U[c,k].
    block=None applies each column's update to all later columns at once.
    block=B defers updates beyond the current B-column block and applies them
    with one matrix product when the block ends; it computes the same thing
    (only the order of the additions to each w_k changes).

    Replay of another implementation's decisions (a diagnostic for results
    that part ways only at rounding ties): forced (codes [m, n], processed
    order) and forced_zeros (zero points [m, G], group order) are adopted
    wherever they differ from this oracle's own decision, so both sides stay
    on one trajectory.  Each such difference must be one step across a
    rounding boundary: the unrounded grid position (w/step + z for a code,
    -lo/step for a zero point) within tie_tol steps of the half-integer
    between the two choices; any other difference counts as bad.  The result
    then also holds replay = dict(flips, zero_flips, bad, max_tie_dist).

    Returns dict(codes [m,n] processed order, scales [m,G], zeros [m,G],
    err [m,n], loss0 = ½Σe²).
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    m, n = W.shape
    gw = _group_width(group_size, n)
    G = (n + gw - 1) // gw if n else 0
    codes = np.zeros((m, n))
    scales = np.zeros((m, G))
    zeros = np.zeros((m, G))
    err = np.zeros((m, n))
    loss0 = 0.0
    B = n if block is None else block
    if block is not None and group_size != -1 and block % group_size != 0:
        raise ValueError("block must be a multiple of group_size")
    s = z = lo = hi = None
    replay = dict(flips=0, zero_flips=0, bad=0, max_tie_dist=0.0)

    def judge(own, other, x, key):
        # other differs from own on the masked rows; x = unrounded position
        d = np.abs(other - own)
        dist = np.abs(x - (np.minimum(own, other) + 0.5))
        ok = (d == 1) & (dist <= tie_tol)
        replay[key] += int(own.size)
        replay["bad"] += int((~ok).sum())
        if own.size:
            replay["max_tie_dist"] = max(replay["max_tie_dist"], float(dist.max()))

    for i1 in range(0, n, max(B, 1)):
        i2 = min(i1 + B, n)
        for c in range(i1, i2):
            if c % gw == 0:
                s, z, lo, hi = group_params(W[:, c:min(c + gw, n)], bits, sym)
                if forced_zeros is not None:
                    zf = np.asarray(forced_zeros[:, c // gw], dtype=np.float64)
                    d = zf != z
                    if d.any():
                        if sym:   # the offset is fixed: any difference is wrong
                            replay["zero_flips"] += int(d.sum())
                            replay["bad"] += int(d.sum())
                        else:
                            judge(z[d], zf[d], -lo[d] / s[d], "zero_flips")
                        z = zf
                scales[:, c // gw] = s
                zeros[:, c // gw] = z
            q = quantize_values(W[:, c], s, z, bits, sym, lo, hi)
            if forced is not None:
                qf = np.asarray(forced[:, c], dtype=np.float64)
                d = qf != q
                if d.any():
                    # position on the grid before rounding, in code units
                    x = W[d, c] / s[d] + (z[d] if not sym else 0.0)
                    own = q[d] - (z[d] if sym else 0.0)
                    other = qf[d] - (z[d] if sym else 0.0)
                    judge(own, other, x, "flips")
                q = qf
            e = (W[:, c] - dequantize_values(q, s, z)) / U[c, c]
            codes[:, c] = q
            err[:, c] = e
            loss0 += 0.5 * float(np.dot(e, e))
            W[:, c + 1:i2] -= np.outer(e, U[c, c + 1:i2])
        if i2 < n:
            W[:, i2:] -= err[:, i1:i2] @ U[i1:i2, i2:]
    out = dict(codes=codes.astype(np.int64), scales=scales,
               zeros=zeros.astype(np.int64), err=err, loss0=loss0)
    if forced is not None or forced_zeros is not None:
        out["replay"] = replay
    return out


def rtn_quantize(Wp, bits, group_size, sym):
    """Round-to-nearest on the same per-row, per-group grid, no compensation."""
    Wp = np.asarray(Wp, dtype=np.float64)
    m, n = Wp.shape
    gw = _group_width(group_size, n)
    G = (n + gw - 1) // gw if n else 0
    codes = np.zeros((m, n))
    scales = np.zeros((m, G))
    zeros = np.zeros((m, G))
    for gi in range(G):
        c0, c1 = gi * gw, min((gi + 1) * gw, n)
        s, z, lo, hi = group_params(Wp[:, c0:c1], bits, sym)
        scales[:, gi] = s
        zeros[:, gi] = z
        codes[:, c0:c1] = quantize_values(Wp[:, c0:c1], s[:, None], z[:, None], bits, sym,
                                          lo[:, None], hi[:, None])
    return dict(codes=codes.astype(np.int64), scales=scales, zeros=zeros.astype(np.int64))


# ---------------------------------------------------------------------------
# Stage 5: back to the original column order, packing, losses
# ---------------------------------------------------------------------------
def g_index(perm, group_size):
    """g_idx[perm[p]] = p // g: the group of each original column."""
    n = len(perm)
    gw = _group_width(group_size, n)
    gidx = np.zeros(n, dtype=np.int64)
    gidx[np.asarray(perm)] = np.arange(n) // max(gw, 1)
    return gidx


def unpermute_codes(codes_p, perm):
    """Q[:, perm[p]] = codes_p[:, p]."""
    Q = np.zeros_like(codes_p)
    Q[:, np.asarray(perm)] = codes_p
    return Q


def dequantize_layer(Q, scales, zeros, gidx):
    """Q̂ [m, n] in original column order from codes, per-group scale and zero."""
    return (Q - zeros[:, gidx]) * scales[:, gidx]


def pack_codes(Q, bits):
    """qweight as uint32 words.

    bits <= 4: eight codes per word, column 8w+i in bits [4i, 4i+4).
    bits == 8: four codes per word, column 4w+i in bits [8i, 8i+8).
    The last word of a row is zero-padded.
    """
    Q = np.asarray(Q, dtype=np.int64)
    m, n = Q.shape
    per, width = (8, 4) if bits <= 4 else (4, 8)
    nw = (n + per - 1) // per
    out = np.zeros((m, nw), dtype=np.uint64)
    for j in range(n):
        out[:, j // per] |= (Q[:, j].astype(np.uint64) << np.uint64(width * (j % per)))
    return out.astype(np.uint32)


def unpack_codes(qweight, n, bits):
    per, width = (8, 4) if bits <= 4 else (4, 8)
    mask = (1 << width) - 1
    qw = np.asarray(qweight, dtype=np.uint64)
    Q = np.zeros((qw.shape[0], n), dtype=np.int64)
    for j in range(n):
        Q[:, j] = (qw[:, j // per] >> np.uint64(width * (j % per))) & np.uint64(mask)
    return Q


def loss_terms(W, Qhat, H, lam):
    """(½·tr(ΔW H_d ΔWᵀ), ‖ΔW‖²_F) with ΔW = W - Q̂ in original order, H_d = H + λI."""
    dW = np.asarray(W, dtype=np.float64) - Qhat
    Hd = np.asarray(H, dtype=np.float64) + lam * np.eye(dW.shape[1])
    return 0.5 * float(np.sum((dW @ Hd) * dW)), float(np.sum(dW * dW))


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------
def gptq_layer(W, H, key, bits, group_size, sym, desc_act, damp_percent,
               block=None, U=None, perm=None):
    """Full path on one layer: (damp, act-order, inverse factor, quantize, finalize).

    U/perm may be supplied (for a stage-wise comparison fed the GPU's own
    inverse factor); otherwise they are computed here from H and key.
    Returns the outputs in original column order plus both losses:
    loss0 = ½Σe² (equal to ½·tr(ΔW H_d ΔWᵀ)) and loss1 = ‖W - Q̂‖²_F.
    """
    W = np.asarray(W, dtype=np.float64)
    lam = None
    if U is None or perm is None:
        U, perm, lam = prepare(H, key, damp_percent, desc_act)
    perm = np.asarray(perm, dtype=np.int64)
    Wp = W[:, perm]
    res = gptq_quantize(Wp, U, bits, group_size, sym, block=block)
    Q = unpermute_codes(res["codes"], perm)
    gidx = g_index(perm, group_size)
    Qhat = dequantize_layer(Q, res["scales"], res["zeros"], gidx)
    loss1 = float(np.sum((W - Qhat) ** 2))
    return dict(codes=Q, codes_p=res["codes"], scales=res["scales"], zeros=res["zeros"],
                g_idx=gidx, perm=perm, U=U, lam=lam, err_p=res["err"],
                loss0=res["loss0"], loss1=loss1, qweight=pack_codes(Q, bits), Qhat=Qhat)
