"""ctypes loader for libgptq_mi355x.so (the C ABI declared in include/gptq_mi355x.h).

There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq_mi355x.so")

GPTQ_OK = 0
GPTQ_ERR_INVALID_ARG = -1
GPTQ_ERR_UNSUPPORTED = -2
GPTQ_ERR_WORKSPACE = -3
GPTQ_ERR_NOT_PD = -4
GPTQ_ERR_NONFINITE = -5
GPTQ_ERR_HIP = -6
STATUS_NAMES = {
    GPTQ_OK: "GPTQ_OK", GPTQ_ERR_INVALID_ARG: "GPTQ_ERR_INVALID_ARG",
    GPTQ_ERR_UNSUPPORTED: "GPTQ_ERR_UNSUPPORTED", GPTQ_ERR_WORKSPACE: "GPTQ_ERR_WORKSPACE",
    GPTQ_ERR_NOT_PD: "GPTQ_ERR_NOT_PD", GPTQ_ERR_NONFINITE: "GPTQ_ERR_NONFINITE",
    GPTQ_ERR_HIP: "GPTQ_ERR_HIP",
}
GPTQ_BF16 = 0
GPTQ_FP32 = 1


class GptqConfig(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("desc_act", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("damp_percent", ctypes.c_double)]


class GptqRtnConfig(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("clip_ratio", ctypes.c_float)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_ST = ctypes.c_int  # gptq_status

SIGNATURES = {
    "gptq_hessian_workspace_bytes": (_SZ, [_I64, _I64, _I32]),
    "gptq_hessian_accumulate": (_ST, [_P, _P, _I64, _P, _I32, _I64, _I64, ctypes.c_float, _P, _SZ, _P]),
    "gptq_prepare_workspace_bytes": (_SZ, [_I64]),
    "gptq_prepare_hinv": (_ST, [_P, _P, _I64, ctypes.c_double, _I32, _P, _P, _SZ,
                                ctypes.POINTER(ctypes.c_double), _P]),
    "gptq_quantize_workspace_bytes": (_SZ, [_I64, _I64, ctypes.POINTER(GptqConfig)]),
    "gptq_quantize_layer": (_ST, [_P, _I32, _I64, _I64, _P, _P, ctypes.POINTER(GptqConfig), _P, _P,
                                  _P, _P, _P, _P, _P, _SZ, _P]),
    "gptq_rtn_workspace_bytes": (_SZ, [_I64, _I64, ctypes.POINTER(GptqRtnConfig)]),
    "gptq_rtn_quantize": (_ST, [_P, _I32, _I64, _I64, ctypes.POINTER(GptqRtnConfig), _P, _P, _P, _P,
                                _P, _P, _SZ, _P]),
    "gptq_awq_stats_workspace_bytes": (_SZ, [_I64, _I64]),
    "gptq_awq_channel_stats": (_ST, [_P, _I32, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "gptq_awq_workspace_bytes": (_SZ, [_I64, _I64, ctypes.POINTER(GptqRtnConfig)]),
    "gptq_awq_quantize": (_ST, [_P, _I32, _I64, _I64, _P, _I64, ctypes.c_float, ctypes.POINTER(GptqRtnConfig),
                                _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "gptq_w4a16_packed_bytes": (_SZ, [_I64, _I64, _I32]),
    "gptq_w4a16_pack": (_ST, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _SZ, _P]),
    "gptq_w4a16_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "gptq_w4a16_matmul": (_ST, [_P, _I64, _I64, _P, _I64, _I64, _I32, _P, _I64, _P, _SZ, _P]),
    "gptq_w4a16_noalloc_scratch_bytes": (_SZ, []),
    "gptq_w4a16_matmul_noalloc": (_ST, [_P, _I64, _I64, _P, _I64, _I64, _I32, _P, _I64, _P]),
    "gptq_checkpoint_qweight_rows": (_I64, [_I64, _I32]),
    "gptq_checkpoint_qzeros_words": (_I64, [_I64, _I32]),
    "gptq_export_checkpoint": (_ST, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P]),
    "gptq_qweight_words": (_I64, [_I64, _I32]),
    "gptq_num_groups": (_I64, [_I64, _I32]),
    "gptq_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m post_weight_quantization_14_amd.build` "
                "(or __graft_entry__.build()) first; there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
