"""fp64 oracle of merging a trained LoRA adapter into its base weight.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, by page title and section:

* "QLoRA -- the democratization event", the closing note on deployment:
  to ship a merged model the base is dequantised, the adapter merged into
  it, and the result possibly quantised again.
* "QLoRA" (infivelines.com), the unheaded note on the recipe's last step:
  merging the bf16 adapters into the 4-bit base and saving that loses
  precision a second time, so the merge should be made against the
  original (unquantised) weights.
* "QLoRA, and fine-tuning a 7B model on a free GPU", "Merging a QLoRA
  adapter": merging into the full-precision base is the usual practice; it
  is not the arithmetic that was trained (the adapter learned to correct
  the quantised base).

Reading: the pages give the merge in words.  The merged weight is the one
whose plain linear layer equals the adapted layer,

    W_m = W_base + s . B . A,      s = lora_alpha / r,

so that x . W_m^T = x . W_base^T + s . (x . A^T) . B^T.  W_base is either
the decoded 4-bit base W' (what the adapter was trained against) or the
original weight W0.  The exported values are W_m in fp32 and W_m rounded
once more to bf16 (round to nearest even, from the fp32 value).  The
"quantised again" path feeds the fp32 W_m through the same NF4 + double
quantisation as the base.
"""

from __future__ import annotations

import numpy as np

from .lora_linear import lora_scale
from .nf4 import (bf16_bits_to_f64, bf16_rne_bits, dequant_nf4_bits, double_quant,
                  quantize_nf4)


def merge_adapter(w_base, A, B, alpha: float) -> np.ndarray:
    """W_m = W_base + (alpha/r) . B . A in fp64.

    ``w_base`` [N, K] (any float dtype holding the exact base values),
    ``A`` [r, K], ``B`` [N, r].  ``A``/``B`` may be None (or r = 0): then
    W_m is the base itself.
    """
    w64 = np.asarray(w_base, dtype=np.float64)
    r = 0 if A is None else np.asarray(A).shape[0]
    if not r:
        return w64.copy()
    return w64 + lora_scale(alpha, r) * (np.asarray(B, dtype=np.float64)
                                         @ np.asarray(A, dtype=np.float64))


def merged_bf16_bits(w_m) -> np.ndarray:
    """The bf16 export of W_m: round to fp32, then to bf16 (both to nearest
    even); returns uint16 bit patterns."""
    return bf16_rne_bits(np.asarray(w_m, dtype=np.float64).astype(np.float32))


def requantize(w_m_f32) -> np.ndarray:
    """The merged fp32 weight quantised again (NF4, blocks of 64, scales
    double-quantised in groups of 256) and decoded back: the fp64 values a
    re-quantised export holds."""
    w = np.ascontiguousarray(w_m_f32, dtype=np.float32)
    _, packed, absmax = quantize_nf4(w)
    q, step = double_quant(absmax)
    return bf16_bits_to_f64(dequant_nf4_bits(packed, q, step, w.size)).reshape(w.shape)


def merge_errors(w0, A, B, alpha: float) -> dict:
    """The three exports of an adapter trained on the NF4 base of ``w0``,
    measured against the ideal merged weight T = W0 + s.B.A (fp64), as
    ||export - T||_F / ||T||_F:

    * ``clean``: merged into the original weights, exported in bf16;
    * ``once``:  merged into the decoded 4-bit base (fp32 export); its error
      is the base's quantisation error;
    * ``twice``: that merge quantised to 4 bits again and decoded.

    Also ``trained_shift``: ||W0 - W'||_F / ||T||_F, how far the clean merge
    moves the layer from the arithmetic the adapter was trained on; and
    ``update_kept``: the share of the update U = s.B.A that survives the
    second quantisation, <twice - W', U> / <U, U> (1 = all of it).
    """
    w0 = np.ascontiguousarray(w0, dtype=np.float32)
    _, packed, absmax = quantize_nf4(w0)
    q, step = double_quant(absmax)
    w_deq = bf16_bits_to_f64(dequant_nf4_bits(packed, q, step, w0.size)).reshape(w0.shape)
    target = merge_adapter(w0, A, B, alpha)
    norm = float(np.linalg.norm(target))
    m_once = merge_adapter(w_deq, A, B, alpha)
    clean = bf16_bits_to_f64(merged_bf16_bits(target))
    twice = requantize(m_once.astype(np.float32))

    def rel(a):
        return float(np.linalg.norm(a - target)) / norm

    upd = m_once - w_deq
    uu = float(np.sum(upd * upd))

    return {"clean": rel(clean), "once": rel(m_once.astype(np.float32).astype(np.float64)),
            "twice": rel(twice),
            "trained_shift": float(np.linalg.norm(w0.astype(np.float64) - w_deq)) / norm,
            "update_kept": float(np.sum((twice - w_deq) * upd)) / uu if uu else 1.0}
