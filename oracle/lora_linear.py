"""fp64 oracle of the frozen-base LoRA linear layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, by page title and section:

* "QLoRA -- the democratization event", the recipe: a frozen 4-bit base with
  16-bit LoRA adapters attached; gradients flow through the frozen 4-bit base
  into the adapters; the base never moves.
* "QLoRA -- Module 12.4", "Definition": gradients flow to the adapters; the
  quantised base stays frozen.  "Hugging Face + BitsAndBytes" and "QLoRA, and
  fine-tuning a 7B model on a free GPU", "Combining two ideas": the adapters
  are configured by a rank r and lora_alpha.

Reading: the pages defer the LoRA equation to another lesson.  The layer
taken here is the standard LoRA form on the decoded base W',

    y = x . W'^T + s . (x . A^T) . B^T,     s = lora_alpha / r,

with x [M, K], W' [N, K] (out x in, row-major), A [r, K], B [N, r].
The base is frozen, so the backward pass has no dW; it returns

    g  = dy . B                      [M, r]
    dX = dy . W' + s . g . A         [M, K]
    dB = s . dy^T . (x . A^T)        [N, r]
    dA = s . g^T . x                 [r, K]

Everything is fp64 on the exact input values (bf16 / fp32 inputs widen
exactly).  r = 0 means the layer has no adapter term.

LoRA dropout ("QLoRA -- Module 12.4", "Hugging Face + BitsAndBytes": the
adapter config sets lora_dropout; the pages give no formula).  Reading:
the standard LoRA dropout acts on the adapter's input only, with inverted
scaling: x~ = x * keep / (1 - p), keep in {0, 1} per element of x, and the
adapter term becomes s . (x~ . A^T) . B^T; the base term keeps x.  The
random draws are an input (``keep``), so the same mask serves the forward
pass and its backward, which then reads

    g  = dy . B
    dX = dy . W' + s . (g . A) * keep / (1 - p)
    dB = s . dy^T . (x~ . A^T)
    dA = s . g^T . x~
"""

from __future__ import annotations

import numpy as np


def lora_scale(alpha: float, r: int) -> float:
    """s = lora_alpha / r (0 when there is no adapter)."""
    return 0.0 if r == 0 else float(alpha) / float(r)


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def dropped_input(x, keep, p: float):
    """x~ = x * keep / (1 - p) in fp64 (x itself when keep is None)."""
    x64 = _f64(x)
    if keep is None:
        return x64
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must lie in [0, 1)")
    return x64 * np.asarray(keep, dtype=np.float64) / (1.0 - p)


def lora_linear_fwd(x, w_deq, A, B, alpha: float, keep=None, p: float = 0.0) -> np.ndarray:
    """y = x . W'^T + (alpha/r) . (x~ . A^T) . B^T in fp64.

    ``x`` [M, K], ``w_deq`` [N, K] (decoded base, any float dtype holding
    the exact values), ``A`` [r, K], ``B`` [N, r]; ``A``/``B`` may be None or
    have r = 0 for a base-only layer.  ``keep`` [M, K] (0/1) and ``p``: LoRA
    dropout on the adapter's input (x~ = x when keep is None).
    """
    x64, w64 = _f64(x), _f64(w_deq)
    y = x64 @ w64.T
    r = 0 if A is None else np.asarray(A).shape[0]
    if r:
        xa = dropped_input(x, keep, p) @ _f64(A).T
        y = y + lora_scale(alpha, r) * (xa @ _f64(B).T)
    return y


def lora_linear_bwd(x, dy, w_deq, A, B, alpha: float, keep=None, p: float = 0.0):
    """Gradients of the layer for upstream gradient ``dy`` [M, N], in fp64.

    Returns ``(dX, dA, dB)``; ``dA``/``dB`` are None when r = 0.  ``keep``
    and ``p`` as in the forward pass (the same mask).
    """
    dy64, w64 = _f64(dy), _f64(w_deq)
    dX = dy64 @ w64
    r = 0 if A is None else np.asarray(A).shape[0]
    if not r:
        return dX, None, None
    s = lora_scale(alpha, r)
    A64, B64 = _f64(A), _f64(B)
    xd = dropped_input(x, keep, p)
    g = dy64 @ B64
    gA = s * (g @ A64)
    if keep is not None:
        gA = gA * np.asarray(keep, dtype=np.float64) / (1.0 - p)
    dX = dX + gA
    xa = xd @ A64.T
    dB = s * (dy64.T @ xa)
    dA = s * (g.T @ xd)
    return dX, dA, dB
