"""CPU oracle for the QLoRA frozen-base linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(the C-ABI library and its Python binding) never imports, links or calls
anything here, and this package imports nothing from the product.

What it computes (numpy, fp64 unless a step fixes another precision):

* ``nf4``   -- the 16 NF4 levels and their decision thresholds, the blockwise
  absmax quantiser (blocks of 64, two 4-bit codes per byte), the 8-bit
  double quantisation of the block scales (groups of 256) and the bit-exact
  dequantisation to bf16 (and, for the fp16 compute-type variant, to fp16).
* ``lora_linear`` -- the layer y = x.W'^T + (alpha/r).(x.A^T).B^T and its
  gradients dX, dA, dB on the decoded weight W', optionally with LoRA
  dropout on the adapter's input (the keep-mask is an input).
* ``philox`` -- Philox4x32-10 and the LoRA-dropout keep mask the library
  draws from it in-kernel (counter = mask byte and stream offset, key =
  seed; 16-bit draws against a threshold).
* ``dq_centred`` -- the paper-style variant of the scale encoding: block
  scales centred on their tensor mean and coded as symmetric signed 8-bit
  values per group of 256 (s' = fp32(fp32(q * step) + mean)).
* ``merge`` -- the adapter merged into a base weight for export,
  W_m = W_base + (alpha/r).B.A (fp32 and bf16 exports, re-quantisation, and
  the errors of the three ways to export).

Sources are cited by page title and section.  The pages state the format in
words only; every reading taken where they are silent is written at the
function that takes it.

Parity status: every function here is pinned by a CPU test in ``tests/``
against something other than itself (closed forms, brute force on tiny
inputs, library routines for special cases, adjoint identities, the pages'
storage figures).  The exact numeric values of the NF4 levels are fixed by
the construction reading, not by a table on the pages.
"""

from .nf4 import (  # noqa: F401
    P_MAX,
    BLOCK,
    GROUP,
    nf4_levels_f64,
    nf4_levels_f32,
    nf4_thresholds_f32,
    bf16_rne_bits,
    bf16_bits_to_f64,
    quantize_nf4,
    unpack_codes,
    double_quant,
    dequant_scales,
    dequant_nf4_bits,
    dequant_nf4_f16_bits,
    f16_rne_bits,
    f16_bits_to_f64,
    storage_bits_per_weight,
)
from .lora_linear import lora_linear_fwd, lora_linear_bwd, lora_scale, dropped_input  # noqa: F401
from .dq_centred import (  # noqa: F401
    centred_mean,
    double_quant_centred,
    dequant_scales_centred,
    dequant_nf4_centred_bits,
    dequant_nf4_centred_f16_bits,
)
from .merge import merge_adapter, merged_bf16_bits, requantize, merge_errors  # noqa: F401
from .philox import (  # noqa: F401
    philox4x32_10,
    dropout_threshold,
    realised_dropout,
    dropout_uniforms,
    dropout_keep_philox,
)
