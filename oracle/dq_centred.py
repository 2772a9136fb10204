"""Mean-centred 8-bit double quantisation of the block scales -- the
paper-style variant of the scale encoding.  TEST INFRASTRUCTURE ONLY (see
the package docstring).

Sources, by page title and section:

* "QLoRA -- the democratization event", the recipe (step 4): the base is
  loaded with double quantization, named after the QLoRA paper it cites.
* "QLoRA" (infivelines.com): the per-block scales are quantised again in
  blocks of 256.
* "QLoRA -- Module 12.4", "Design Details That Matter": double quant
  quantises the quantisation constants.

The pages give neither the 8-bit format nor any centring.  The paper the
recipe cites centres the first-level scales on their mean before the
second quantisation so that a symmetric 8-bit code can be used; this module
is that variant, and every step below is a reading (parity of the format
itself is unpinned by the pages; the pins in the tests are the definition's
own closed forms, exact rational arithmetic and invariants):

* mean: mu = fp32(T / n_blocks) where T is an fp64 sum in a fixed order --
  each group's (up to) 256 scales added in index order starting from 0,
  the group sums added in CHUNKS contiguous chunks of ceil(G / CHUNKS)
  groups (group order within a chunk), and the chunk sums added in chunk
  order.  (Every addend is a non-negative fp32 value held exactly in fp64;
  the order is fixed so that a parallel device reduction can give the same
  bits.)
* centred scale: d_b = fp32(s_b - mu), one fp32 subtraction.
* per group of 256 blocks (the last group holds only the real blocks):
  A = max_b |d_b|; step = fp32(A / 127) correctly rounded;
  q_b = clamp(round-half-even(fp32(d_b / step)), -127, 127), stored as a
  two's-complement byte; a group with A = 0 stores step 0 and q = 0.
* decoded scale: s'_b = fp32(fp32(q_b * step) + mu) -- a product and a sum,
  each rounded once (not fused).
* Storage: one byte per block, one fp32 step per group and one fp32 mean
  per tensor (the same bits per weight as the unsigned format plus 32 bits
  per tensor).  A decoded scale may come out slightly below zero for a
  block whose scale is within step / 2 of zero; the NF4 codes are those of
  the unsigned format (they depend only on the first-level scale).
"""

from __future__ import annotations

import numpy as np

from .nf4 import BLOCK, GROUP, bf16_rne_bits, f16_rne_bits, nf4_levels_f32, unpack_codes

CHUNKS = 1024   # chunks of the mean's second summation level
QMAX = 127      # the symmetric 8-bit code: q in [-127, 127]


def centred_mean(absmax: np.ndarray, blocksize2: int = GROUP) -> np.float32:
    """mu = fp32(T / n_blocks), T summed in fp64 in the fixed order above."""
    s = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    nb = s.size
    if nb == 0:
        return np.float32(0.0)
    ng = (nb + blocksize2 - 1) // blocksize2
    padded = np.zeros(ng * blocksize2, dtype=np.float64)   # +0.0 past the end adds nothing
    padded[:nb] = s.astype(np.float64)
    # np.add.accumulate runs strictly left to right: its last column is the
    # sequential sum of each row
    group_sums = np.add.accumulate(padded.reshape(ng, blocksize2), axis=1)[:, -1]
    per_chunk = (ng + CHUNKS - 1) // CHUNKS
    chunked = np.zeros(CHUNKS * per_chunk, dtype=np.float64)
    chunked[:ng] = group_sums
    chunk_sums = np.add.accumulate(chunked.reshape(CHUNKS, per_chunk), axis=1)[:, -1]
    total = np.add.accumulate(chunk_sums)[-1]
    return np.float32(total / np.float64(nb))


def double_quant_centred(absmax: np.ndarray, blocksize2: int = GROUP):
    """The block scales -> (q, step, mu): q uint8 [n_blocks] (two's
    complement of the signed code), step fp32 [ceil(n_blocks / 256)], mu
    fp32 scalar."""
    s = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    nb = s.size
    ng = (nb + blocksize2 - 1) // blocksize2
    mu = centred_mean(s, blocksize2)
    d = (s - mu).astype(np.float32)                         # fp32 subtraction
    padded = np.zeros(ng * blocksize2, dtype=np.float32)    # |0| adds nothing to the max
    padded[:nb] = np.abs(d)
    amax = padded.reshape(ng, blocksize2).max(axis=1)
    # fp64 quotients of fp32 operands round to the correctly rounded fp32
    # quotient (53 >= 2 * 24 + 2 bits)
    step = (amax.astype(np.float64) / float(QMAX)).astype(np.float32)
    group_of_block = np.arange(nb) // blocksize2
    st = step[group_of_block]
    live = st > 0
    safe = np.where(live, st, np.float32(1.0)).astype(np.float64)
    u = (d.astype(np.float64) / safe).astype(np.float32)
    q = np.clip(np.rint(u), -QMAX, QMAX)                     # rint: half to even
    q[~live] = 0
    return q.astype(np.int8).view(np.uint8), step, mu


def dequant_scales_centred(q: np.ndarray, step: np.ndarray, mu,
                           blocksize2: int = GROUP) -> np.ndarray:
    """s'_b = fp32(fp32(q_b * step_group(b)) + mu)."""
    qs = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1).view(np.int8)
    st = np.ascontiguousarray(step, dtype=np.float32).reshape(-1)
    group_of_block = np.arange(qs.size) // blocksize2
    prod = (qs.astype(np.float64) * st[group_of_block].astype(np.float64)).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)        # fp32 sum, rounded once


def _decoded_products(packed, q, step, mu, n, blocksize, blocksize2):
    codes = unpack_codes(packed, n)
    scale = dequant_scales_centred(q, step, mu, blocksize2)
    block_of_elem = np.arange(n) // blocksize
    levels = nf4_levels_f32().astype(np.float64)
    return (levels[codes] * scale[block_of_elem].astype(np.float64)).astype(np.float32)


def dequant_nf4_centred_bits(packed: np.ndarray, q: np.ndarray, step: np.ndarray, mu,
                             n: int, blocksize: int = BLOCK,
                             blocksize2: int = GROUP) -> np.ndarray:
    """w' = bf16_rne(fp32(L32[code] * s')) with s' the centred decoded scale
    (the dequantisation of the unsigned format with only s' changed)."""
    return bf16_rne_bits(_decoded_products(packed, q, step, mu, n, blocksize, blocksize2))


def dequant_nf4_centred_f16_bits(packed: np.ndarray, q: np.ndarray, step: np.ndarray, mu,
                                 n: int, blocksize: int = BLOCK,
                                 blocksize2: int = GROUP) -> np.ndarray:
    """The fp16 compute-type form: w' = fp16_rne(fp32(L32[code] * s'))."""
    return f16_rne_bits(_decoded_products(packed, q, step, mu, n, blocksize, blocksize2))
