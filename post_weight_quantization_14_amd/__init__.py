"""MI355X (gfx950) GPTQ layer quantization: Hessian accumulation, the damped
inverse factor with act-order, and block-wise column quantization with error
feedback, all in hand-written HIP kernels behind a C ABI
(include/gptq_mi355x.h).  This package is the thin Python binding."""
from ._lib import GPTQ_BF16, GPTQ_FP32, LIB_PATH, lib  # noqa: F401
from .gptq import (  # noqa: F401
    GptqError,
    QuantConfig,
    RtnConfig,
    alloc_outputs,
    awq_quantize,
    check_status,
    gptq_awq_channel_stats,
    gptq_awq_quantize,
    gptq_awq_stats_workspace_bytes,
    gptq_awq_workspace_bytes,
    gptq_checkpoint_qweight_rows,
    gptq_checkpoint_qzeros_words,
    gptq_export_checkpoint,
    gptq_hessian_accumulate,
    gptq_hessian_workspace_bytes,
    gptq_last_error,
    gptq_num_groups,
    gptq_prepare_hinv,
    gptq_prepare_workspace_bytes,
    gptq_quantize_layer,
    gptq_quantize_workspace_bytes,
    gptq_qweight_words,
    gptq_rtn_quantize,
    gptq_rtn_workspace_bytes,
    gptq_w4a16_matmul,
    gptq_w4a16_matmul_noalloc,
    gptq_w4a16_pack,
    gptq_w4a16_packed_bytes,
    gptq_w4a16_workspace_bytes,
    quantize_layer,
    quantize_shared_input,
    rtn_quantize,
)
