"""CPU oracle for the GPTQ layer-quantization path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product library.
It is plain float64 NumPy written from the pages; see ``gptq_oracle`` for the
citations and the readings taken where the pages are silent or garbled.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(worked example, hand cases, exact rational route, brute force, invariants).
"""
from .gptq_oracle import (  # noqa: F401
    NotPositiveDefinite,
    act_order,
    damp_and_permute,
    damping,
    dequantize_layer,
    dequantize_values,
    g_index,
    gptq_layer,
    gptq_quantize,
    group_params,
    hessian,
    hessian_accumulate,
    hessian_diagonal_accumulate,
    inverse_upper_factor,
    loss_terms,
    pack_codes,
    prepare,
    quantize_values,
    rtn_quantize,
    unpack_codes,
    unpermute_codes,
)
from .linear_quantizer import (  # noqa: F401,E402
    linear_codes,
    linear_grid,
    linear_quantize,
    percentile_linear,
)
from .quantized_matmul import (  # noqa: F401,E402
    dequant_matmul,
    dequantized_weight,
)
from .awq import (  # noqa: F401,E402
    awq_quantize,
    channel_abs_sum,
    channel_scale,
    lower_median,
)
from .checkpoint import (  # noqa: F401,E402
    bit_stream_codes,
    bit_stream_words,
    checkpoint_qweight_rows,
    checkpoint_qzeros_words,
    export_checkpoint,
    export_qweight_columns,
    export_qzeros,
    export_scales,
    import_checkpoint,
)
