"""Python binding of the C ABI: the same entry points, taking torch tensors.

Argument marshalling only: tensors become device pointers, sizes and strides
become integers, the stream is torch's current HIP stream.  Every step of the
path runs in the HIP kernels of libgptq_mi355x.so; a non-OK status raises
GptqError carrying the library's message.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import GptqConfig, lib


class GptqError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().gptq_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


@dataclass
class QuantConfig:
    """Quantizer settings (bits, group_size, sym, desc_act, damp_percent)."""
    bits: int = 4
    group_size: int = 128
    sym: bool = False
    desc_act: bool = True
    damp_percent: float = 0.01
    block_size: int = 128

    def c(self) -> GptqConfig:
        return GptqConfig(int(self.bits), int(self.group_size), int(bool(self.sym)),
                          int(bool(self.desc_act)), int(self.block_size), float(self.damp_percent))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.GPTQ_BF16
    if t.dtype == torch.float32:
        return _lib.GPTQ_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(status: int, where: str) -> None:
    if status != _lib.GPTQ_OK:
        raise GptqError(status, where)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- sizes
def gptq_hessian_workspace_bytes(n: int, tokens: int, x_dtype: int = _lib.GPTQ_BF16) -> int:
    return int(lib().gptq_hessian_workspace_bytes(n, tokens, x_dtype))


def gptq_prepare_workspace_bytes(n: int) -> int:
    return int(lib().gptq_prepare_workspace_bytes(n))


def gptq_quantize_workspace_bytes(m: int, n: int, cfg: QuantConfig) -> int:
    c = cfg.c()
    return int(lib().gptq_quantize_workspace_bytes(m, n, ctypes.byref(c)))


def gptq_qweight_words(n: int, bits: int) -> int:
    return int(lib().gptq_qweight_words(n, bits))


def gptq_num_groups(n: int, group_size: int) -> int:
    return int(lib().gptq_num_groups(n, group_size))


def gptq_last_error() -> str:
    return lib().gptq_last_error().decode(errors="replace")


# ---------------------------------------------------------------- stages
def gptq_hessian_accumulate(H: torch.Tensor, diag_key: Optional[torch.Tensor], X: torch.Tensor,
                            alpha: float = 2.0, workspace: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """H += alpha·XᵀX, diag_key += alpha·Σx² (fp64), for X [tokens, n] with unit column stride."""
    n = H.shape[0]
    if X.dim() != 2 or X.shape[1] != n or (X.shape[0] > 0 and X.stride(1) != 1):
        raise ValueError("X must be [tokens, n] with contiguous rows")
    code = _dtype_code(X)
    ws = _workspace(gptq_hessian_workspace_bytes(n, X.shape[0], code), H.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().gptq_hessian_accumulate(_ptr(H), _ptr(diag_key), n, _ptr(X), code, X.shape[0],
                                       X.stride(0) if X.shape[0] > 0 else n, float(alpha),
                                       _ptr(ws), nbytes, _stream(stream))
    _check(st, "gptq_hessian_accumulate")


def gptq_prepare_hinv(H: torch.Tensor, diag_key: Optional[torch.Tensor], damp_percent: float,
                      desc_act: bool, perm_out: torch.Tensor,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> float:
    """H (in place) -> U; fills perm_out; returns the damping λ."""
    n = H.shape[0]
    ws = _workspace(gptq_prepare_workspace_bytes(n), H.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    lam = ctypes.c_double(0.0)
    st = lib().gptq_prepare_hinv(_ptr(H), _ptr(diag_key), n, float(damp_percent), int(bool(desc_act)),
                                 _ptr(perm_out), _ptr(ws), nbytes, ctypes.byref(lam), _stream(stream))
    _check(st, "gptq_prepare_hinv")
    return lam.value


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, cfg: QuantConfig,
                        qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                        g_idx: torch.Tensor, loss: torch.Tensor, status: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue the quantization; never synchronises.  `status` (int32 [1] on
    the device, optional) receives 0 or GPTQ_ERR_NONFINITE in stream order:
    read it with check_status()."""
    if not W.is_contiguous():
        raise ValueError("W must be contiguous [m, n]")
    m, n = W.shape
    c = cfg.c()
    ws = _workspace(gptq_quantize_workspace_bytes(m, n, cfg), W.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().gptq_quantize_layer(_ptr(W), _dtype_code(W), m, n, _ptr(U), _ptr(perm), ctypes.byref(c),
                                   _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(g_idx), _ptr(loss),
                                   _ptr(status), _ptr(ws), nbytes, _stream(stream))
    _check(st, "gptq_quantize_layer")


def check_status(*outs) -> None:
    """Read the device status words of earlier quantizations (one host
    synchronisation for all of them) and raise GptqError for the first that
    is not GPTQ_OK.  Each argument is an output dict of quantize_layer /
    quantize_shared_input, or a list of them."""
    flat = []
    for o in outs:
        if isinstance(o, dict):
            flat.append(o)
        else:
            for x in o:
                flat.extend(x if isinstance(x, list) else [x])
    if not flat:
        return
    words = torch.cat([o["status"] for o in flat]).cpu().tolist()
    for w in words:
        if w != _lib.GPTQ_OK:
            lib().gptq_last_error()   # keeps the message API uniform
            raise GptqError(int(w), "gptq_quantize_layer (status word)")


# ---------------------------------------------------------------- linear (RTN) quantizer
@dataclass
class RtnConfig:
    """Settings of gptq_rtn_quantize: bits 2/3/4/8; group_size -1 (one group
    per output row) or >= 1; sym; clip_ratio in (0, 1]."""
    bits: int = 8
    group_size: int = -1
    sym: bool = True
    clip_ratio: float = 0.99

    def c(self) -> "_lib.GptqRtnConfig":
        return _lib.GptqRtnConfig(self.bits, self.group_size, int(self.sym), self.clip_ratio)


def gptq_rtn_workspace_bytes(m: int, n: int, cfg: RtnConfig) -> int:
    c = cfg.c()
    return int(lib().gptq_rtn_workspace_bytes(m, n, ctypes.byref(c)))


def _status_word(status: Optional[torch.Tensor], check: bool, device) -> Optional[torch.Tensor]:
    if status is None and check:
        status = torch.zeros(1, dtype=torch.int32, device=device)
    return status


def _read_status(status: torch.Tensor, where: str) -> None:
    """Synchronise on the device status word and raise on a non-OK status."""
    w = int(status.item())
    if w != _lib.GPTQ_OK:
        raise GptqError(w, f"{where} (status word: the input holds a NaN or Inf)")


def gptq_rtn_quantize(W: torch.Tensor, cfg: RtnConfig, qweight: torch.Tensor, scales: torch.Tensor,
                      zeros: torch.Tensor, err: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      stream=None, status: Optional[torch.Tensor] = None, check: bool = True) -> None:
    """Enqueue the quantizer (the call itself never synchronises).  check=True
    reads the device status word afterwards and raises on a NaN/Inf in W;
    check=False leaves it in `status` (int32 [1]) for the caller."""
    if not W.is_contiguous():
        raise ValueError("W must be contiguous [m, n]")
    m, n = W.shape
    c = cfg.c()
    ws = _workspace(gptq_rtn_workspace_bytes(m, n, cfg), W.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    status = _status_word(status, check, W.device)
    st = lib().gptq_rtn_quantize(_ptr(W), _dtype_code(W), m, n, ctypes.byref(c), _ptr(qweight),
                                 _ptr(scales), _ptr(zeros), _ptr(err), _ptr(status), _ptr(ws), nbytes,
                                 _stream(stream))
    _check(st, "gptq_rtn_quantize")
    if check and m > 0 and n > 0:
        _read_status(status, "gptq_rtn_quantize")


def rtn_quantize(W: torch.Tensor, cfg: RtnConfig) -> dict:
    """Allocate the outputs and run gptq_rtn_quantize on W [m, n]."""
    m, n = W.shape
    dev = W.device
    # sizes of an invalid config come back negative: allocate nothing and let
    # the library report the config
    words = max(gptq_qweight_words(n, cfg.bits), 0)
    groups = max(gptq_num_groups(n, cfg.group_size), 0)
    out = dict(
        qweight=torch.empty(m, words, dtype=torch.int32, device=dev),
        scales=torch.empty(m, groups, dtype=torch.float32, device=dev),
        zeros=torch.empty(m, groups, dtype=torch.int32, device=dev),
        err=torch.zeros(2, dtype=torch.float64, device=dev),
    )
    gptq_rtn_quantize(W, cfg, out["qweight"], out["scales"], out["zeros"], out["err"])
    return out


# ---------------------------------------------------------------- AWQ channel scaling
def gptq_awq_stats_workspace_bytes(n: int, tokens: int) -> int:
    return int(lib().gptq_awq_stats_workspace_bytes(n, tokens))


def gptq_awq_channel_stats(X: torch.Tensor, abs_sum: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> None:
    """abs_sum [n] fp64 += Σ_t |X[t]| for X [tokens, n] (bf16 or fp32) with contiguous rows."""
    if X.dim() != 2 or (X.shape[0] > 0 and X.stride(1) != 1):
        raise ValueError("X must be [tokens, n] with contiguous rows")
    tokens, n = X.shape
    ws = _workspace(gptq_awq_stats_workspace_bytes(n, tokens), X.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().gptq_awq_channel_stats(_ptr(X), _dtype_code(X), tokens, X.stride(0) if tokens > 0 else n, n,
                                      _ptr(abs_sum), _ptr(ws), nbytes, _stream(stream))
    _check(st, "gptq_awq_channel_stats")


def gptq_awq_workspace_bytes(m: int, n: int, cfg: RtnConfig) -> int:
    c = cfg.c()
    return int(lib().gptq_awq_workspace_bytes(m, n, ctypes.byref(c)))


def gptq_awq_quantize(W: torch.Tensor, abs_sum: torch.Tensor, tokens: int, protect: float, cfg: RtnConfig,
                      qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                      channel_scale: torch.Tensor, err: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      stream=None, status: Optional[torch.Tensor] = None, check: bool = True) -> None:
    """Enqueue the AWQ-scaled quantizer (never synchronises by itself);
    check as in gptq_rtn_quantize (NaN/Inf in W or in abs_sum)."""
    if not W.is_contiguous():
        raise ValueError("W must be contiguous [m, n]")
    m, n = W.shape
    c = cfg.c()
    ws = _workspace(gptq_awq_workspace_bytes(m, n, cfg), W.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    status = _status_word(status, check, W.device)
    st = lib().gptq_awq_quantize(_ptr(W), _dtype_code(W), m, n, _ptr(abs_sum), tokens, float(protect),
                                 ctypes.byref(c), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(channel_scale),
                                 _ptr(err), _ptr(status), _ptr(ws), nbytes, _stream(stream))
    _check(st, "gptq_awq_quantize")
    if check and m > 0 and n > 0:
        _read_status(status, "gptq_awq_quantize")


def awq_quantize(W: torch.Tensor, x_tiles, cfg: RtnConfig, protect: float = 2.0) -> dict:
    """Channel statistics over every X tile, then gptq_awq_quantize on W [m, n]."""
    m, n = W.shape
    dev = W.device
    abs_sum = torch.zeros(n, dtype=torch.float64, device=dev)
    tokens = 0
    for X in x_tiles:
        gptq_awq_channel_stats(X, abs_sum)
        tokens += X.shape[0]
    words = max(gptq_qweight_words(n, cfg.bits), 0)
    groups = max(gptq_num_groups(n, cfg.group_size), 0)
    out = dict(
        qweight=torch.empty(m, words, dtype=torch.int32, device=dev),
        scales=torch.empty(m, groups, dtype=torch.float32, device=dev),
        zeros=torch.empty(m, groups, dtype=torch.int32, device=dev),
        channel_scale=torch.empty(n, dtype=torch.float32, device=dev),
        err=torch.zeros(2, dtype=torch.float64, device=dev),
        abs_sum=abs_sum,
        tokens=tokens,
    )
    gptq_awq_quantize(W, abs_sum, tokens, protect, cfg, out["qweight"], out["scales"], out["zeros"],
                      out["channel_scale"], out["err"])
    return out


# ---------------------------------------------------------------- W4A16 product
def gptq_w4a16_packed_bytes(m: int, n: int, group_size: int) -> int:
    return int(lib().gptq_w4a16_packed_bytes(m, n, group_size))


def gptq_w4a16_pack(qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                    g_idx: torch.Tensor, n: int, bits: int, group_size: int,
                    packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The quantizer's output of an m x n weight -> the product's layout (uint8 tensor)."""
    m = qweight.shape[0]
    nbytes = gptq_w4a16_packed_bytes(m, n, group_size)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qweight.device)
    st = lib().gptq_w4a16_pack(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(g_idx), m, n, bits,
                               group_size, _ptr(packed), packed.numel() * packed.element_size(),
                               _stream(stream))
    _check(st, "gptq_w4a16_pack")
    return packed


def gptq_checkpoint_qweight_rows(n: int, bits: int) -> int:
    return int(lib().gptq_checkpoint_qweight_rows(n, bits))


def gptq_checkpoint_qzeros_words(m: int, bits: int) -> int:
    return int(lib().gptq_checkpoint_qzeros_words(m, bits))


def gptq_export_checkpoint(qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, n: int,
                           bits: int, group_size: int, zero_offset: int = 0, stream=None) -> dict:
    """The quantizer's output of an m x n weight -> the checkpoint tensors
    {"qweight": int32 [ceil(n·bits/32), m], "qzeros": int32 [G, ceil(m·bits/32)],
    "scales": float16 [G, m]} (g_idx is the quantizer's own)."""
    m = qweight.shape[0]
    G = gptq_num_groups(n, group_size)
    rows = gptq_checkpoint_qweight_rows(n, bits)
    zw = gptq_checkpoint_qzeros_words(m, bits)
    if G < 0 or rows < 0 or zw < 0:
        raise ValueError(f"bits={bits} group_size={group_size} n={n}")
    dev = qweight.device
    out = {"qweight": torch.empty(rows, m, dtype=torch.int32, device=dev),
           "qzeros": torch.empty(G, zw, dtype=torch.int32, device=dev),
           "scales": torch.empty(G, m, dtype=torch.float16, device=dev)}
    st = lib().gptq_export_checkpoint(_ptr(qweight), _ptr(scales), _ptr(zeros), m, n, bits, group_size,
                                      zero_offset, _ptr(out["qweight"]), _ptr(out["qzeros"]),
                                      _ptr(out["scales"]), _stream(stream))
    _check(st, "gptq_export_checkpoint")
    return out


def gptq_w4a16_workspace_bytes(tokens: int, m: int, n: int) -> int:
    return int(lib().gptq_w4a16_workspace_bytes(tokens, m, n))


def gptq_w4a16_matmul(X: torch.Tensor, packed: torch.Tensor, m: int, n: int, group_size: int,
                      Y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Y [tokens, m] fp32 = X [tokens, n] bf16 · Ŵᵀ from a packed weight."""
    if X.dim() != 2 or X.shape[1] != n or (X.shape[0] > 0 and X.stride(1) != 1):
        raise ValueError("X must be [tokens, n] with contiguous rows")
    tokens = X.shape[0]
    if Y is None:
        Y = torch.empty(tokens, m, dtype=torch.float32, device=X.device)
    ws = _workspace(gptq_w4a16_workspace_bytes(tokens, m, n), X.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().gptq_w4a16_matmul(_ptr(X), tokens, X.stride(0) if tokens > 0 else n, _ptr(packed), m, n,
                                 group_size, _ptr(Y), Y.stride(0) if tokens > 0 else m, _ptr(ws), nbytes,
                                 _stream(stream))
    _check(st, "gptq_w4a16_matmul")
    return Y


def gptq_w4a16_matmul_noalloc(X: torch.Tensor, packed: torch.Tensor, m: int, n: int, group_size: int,
                              Y: torch.Tensor, stream=None) -> torch.Tensor:
    """gptq_w4a16_matmul on the library's own device scratch (no workspace;
    the C call allocates nothing).  Y [tokens, m] fp32 must be given."""
    if X.dim() != 2 or X.shape[1] != n or (X.shape[0] > 0 and X.stride(1) != 1):
        raise ValueError("X must be [tokens, n] with contiguous rows")
    tokens = X.shape[0]
    st = lib().gptq_w4a16_matmul_noalloc(_ptr(X), tokens, X.stride(0) if tokens > 0 else n, _ptr(packed), m, n,
                                         group_size, _ptr(Y), Y.stride(0) if tokens > 0 else m, _stream(stream))
    _check(st, "gptq_w4a16_matmul_noalloc")
    return Y


# ---------------------------------------------------------------- whole layer
def alloc_outputs(m: int, n: int, cfg: QuantConfig, device) -> dict:
    words = gptq_qweight_words(n, cfg.bits)
    groups = gptq_num_groups(n, cfg.group_size)
    return dict(
        qweight=torch.empty(m, words, dtype=torch.int32, device=device),
        scales=torch.empty(m, groups, dtype=torch.float32, device=device),
        zeros=torch.empty(m, groups, dtype=torch.int32, device=device),
        g_idx=torch.empty(n, dtype=torch.int32, device=device),
        loss=torch.zeros(2, dtype=torch.float64, device=device),
        perm=torch.empty(n, dtype=torch.int32, device=device),
        status=torch.zeros(1, dtype=torch.int32, device=device),
    )


def quantize_layer(W: torch.Tensor, x_tiles, cfg: QuantConfig, alpha: float = 2.0,
                   keep_hessian: bool = False, check: bool = True) -> dict:
    """The three calls in order on one layer: accumulate every X tile into H,
    prepare U, quantize W.  Returns the outputs (and H/key if keep_hessian).
    check=False leaves the quantizer's status word unread (check_status()
    reads many at once), so the quantization adds no host synchronisation."""
    m, n = W.shape
    dev = W.device
    H = torch.zeros(n, n, dtype=torch.float32, device=dev)
    key = torch.zeros(n, dtype=torch.float64, device=dev)
    for X in x_tiles:
        gptq_hessian_accumulate(H, key, X, alpha)
    out = alloc_outputs(m, n, cfg, dev)
    if keep_hessian:
        out["H"] = H.clone()
        out["key"] = key.clone()
    lam = gptq_prepare_hinv(H, key, cfg.damp_percent, cfg.desc_act, out["perm"])
    out["U"] = H
    out["lam"] = lam
    gptq_quantize_layer(W, H, out["perm"], cfg, out["qweight"], out["scales"], out["zeros"],
                        out["g_idx"], out["loss"], out["status"])
    if check:
        check_status(out)
    return out


def quantize_shared_input(Ws, x_tiles, cfgs, alpha: float = 2.0, check: bool = True) -> list:
    """Linears that read the same input (q/k/v of one attention block, gate/up
    of one MLP) have one Hessian H = 2·XᵀX, and the inverse factor U and the
    column order depend only on H, the damping and act-order: accumulate H and
    prepare U once, then quantize every W under every config (for instance
    two bit widths).  All configs must share damp_percent and desc_act.
    The quantizations issue no host synchronisation; with check=True their
    status words are read once, after the last of them.

    Returns out[i][j] for W i under config j (the alloc_outputs dict), each
    identical to what quantize_layer gives for that W, X and config."""
    cfgs = list(cfgs)
    Ws = list(Ws)
    if not Ws or not cfgs:
        raise ValueError("need at least one weight and one config")
    n = Ws[0].shape[1]
    if any(W.dim() != 2 or W.shape[1] != n for W in Ws):
        raise ValueError("every W must be [m_i, n] with the same n")
    if any(c.damp_percent != cfgs[0].damp_percent or bool(c.desc_act) != bool(cfgs[0].desc_act)
           for c in cfgs):
        raise ValueError("configs sharing one U must agree on damp_percent and desc_act")
    dev = Ws[0].device
    H = torch.zeros(n, n, dtype=torch.float32, device=dev)
    key = torch.zeros(n, dtype=torch.float64, device=dev)
    for X in x_tiles:
        gptq_hessian_accumulate(H, key, X, alpha)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    lam = gptq_prepare_hinv(H, key, cfgs[0].damp_percent, cfgs[0].desc_act, perm)
    res = []
    for W in Ws:
        row = []
        for cfg in cfgs:
            o = alloc_outputs(W.shape[0], n, cfg, dev)
            o["perm"].copy_(perm)
            gptq_quantize_layer(W, H, perm, cfg, o["qweight"], o["scales"], o["zeros"], o["g_idx"],
                                o["loss"], o["status"])
            o["lam"] = lam
            row.append(o)
        res.append(row)
    if check:
        check_status(res)
    return res
