"""QLoRA frozen-base linear layer for MI355X (gfx950).

The base weight is stored as packed 4-bit NF4 codes with double-quantised
block scales and is dequantised to bf16 tile by tile inside hand-written
HIP GEMMs; the LoRA path y += (alpha/r).(x.A^T).B^T rides on the same
MFMA accumulators.  The work sits behind the C ABI in include/qlora.h
(``libqlora.so``); this package is its thin Python binding plus the seeded
synthetic input generators.
"""

from . import workloads  # noqa: F401
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    Nf4Weight,
    PackedWeight,
    QloraError,
    dequantize,
    dequantize_f16,
    double_quant,
    double_quant_centred,
    dropout_keep_mask,
    lib,
    linear_bf16_bwd,
    linear_bf16_fwd,
    linear_bwd,
    linear_bwd_dropout,
    linear_bwd_dropout_rng,
    linear_bwd_f16,
    linear_fwd,
    linear_fwd_dropout,
    linear_fwd_dropout_rng,
    linear_fwd_f16,
    linear_fwd_noalloc,
    merge_adapter,
    nf4_levels,
    quantize_nf4,
    quantize_nf4_dq,
    quantize_nf4_dq_centred,
    quantize_weight,
    quantize_weight_centred,
    workspace_bytes,
)
