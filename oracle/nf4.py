"""NF4 encoding oracle: levels, blockwise quantiser, double quantisation, dequant.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, by page title and section:

* "QLoRA" (infivelines.com): NF4 puts its 16 levels at quantiles of a normal
  distribution so that each level is about equally likely; every block of 64
  weights has its own scale so an outlier only affects its own block; the
  block scales are quantised again in blocks of 256, which brings the
  overhead to about 0.127 bits per weight; the base is dequantised to bf16
  one block at a time inside the matrix multiply.
* "QLoRA -- Module 12.4", "Design Details That Matter": NF4 = quantiles for
  normal weights; double quant = quantise the quantisation constants.
* "QLoRA, and fine-tuning a 7B model on a free GPU", "What each setting is
  doing": stored in 4 bits, computed in bfloat16, dequantised for each matmul.

Readings taken where the pages are silent (each is restated at its function):

* Level construction: 8 levels above zero, 7 below, plus an exact zero, each
  side at evenly spaced normal probabilities between 1/2 and P_MAX, scaled so
  the extremes are exactly -1 and +1.  Levels are built in fp64 and rounded
  once to fp32.  A weight's code is the index of the fp32 level nearest to
  u = w / absmax, ties going to the lower index; the fp32 decision
  thresholds that implement this exactly are the midpoints of neighbouring
  levels rounded towards -infinity.
* Quantiser: u = correctly rounded fp32 quotient w / absmax; the code is the
  number of thresholds strictly below u; a block whose absmax is 0 gets
  code 7 (the zero level) everywhere.
* Packing: two codes per byte, the even element in the low nibble; an odd
  tail is padded with code 7.
* Double quantisation: unsigned linear 8-bit codes per group of 256 scales,
  step = fp32(max / 255), q = min(255, round-half-even(fp32(scale / step))).
  A group whose step is 0 stores q = 0 everywhere.
* Dequantisation: s' = fp32(q * step); w' = bf16_rne(fp32(L32[code] * s')):
  one fp32 product, then round-to-nearest-even to bf16.
"""

from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

BLOCK = 64    # weights per absmax block ("QLoRA", infivelines.com)
GROUP = 256   # block scales per double-quantisation group (same page)

# Upper probability of the outermost level: the mean of the outermost
# equal-mass bin centres for 15 and 16 levels, (1 - 1/30) and (1 - 1/32).
P_MAX = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))

_STD_NORMAL = NormalDist(0.0, 1.0)


def _side_probabilities(count: int) -> list[float]:
    """``count`` probabilities evenly spaced from P_MAX towards 1/2, with 1/2
    itself left out (it would duplicate the zero level)."""
    return [P_MAX + (0.5 - P_MAX) * i / count for i in range(count)]


def nf4_levels_f64() -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending, spanning [-1, 1] with an exact 0.

    "QLoRA" (infivelines.com): the 16 levels sit at quantiles of a normal
    distribution.  Sixteen levels that include an exact zero cannot be
    symmetric about it, so this takes 8 positive levels (normal quantiles of
    8 probabilities evenly spaced from P_MAX down towards 1/2) and 7 negative
    ones (the mirrored quantiles of 7 such probabilities), adds 0, and
    divides everything by the quantile of P_MAX so the ends are exactly +-1.
    """
    positive = [_STD_NORMAL.inv_cdf(p) for p in _side_probabilities(8)]
    negative = [-_STD_NORMAL.inv_cdf(p) for p in _side_probabilities(7)]
    top = _STD_NORMAL.inv_cdf(P_MAX)
    levels = sorted(negative + [0.0] + positive)
    return np.array(levels, dtype=np.float64) / top


def nf4_levels_f32() -> np.ndarray:
    """The fp64 levels rounded once (round-to-nearest-even) to fp32."""
    return nf4_levels_f64().astype(np.float32)


def nf4_thresholds_f32() -> np.ndarray:
    """The 15 fp32 decision thresholds between neighbouring fp32 levels.

    Reading: a weight takes the level nearest to u, a tie going to the lower
    level.  For fp32 u that is "u > m_i" with m_i the exact midpoint of
    levels i and i+1.  m_i is exact in fp64 (the two levels' exponents are
    close), but may need one bit more than fp32 holds; rounding it towards
    -infinity gives the fp32 T_i with  u > T_i  <=>  u > m_i  for every fp32
    u, so the count of thresholds below u is the nearest-level index.
    """
    lv = nf4_levels_f32().astype(np.float64)
    mid = (lv[:-1] + lv[1:]) / 2.0
    t = mid.astype(np.float32)
    above = t.astype(np.float64) > mid
    t[above] = np.nextafter(t[above], np.float32(-np.inf))
    return t


# --------------------------------------------------------------------------
# bf16 helpers (the oracle's own; inputs are finite)
# --------------------------------------------------------------------------

def bf16_rne_bits(values_f32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; return the bits.

    bf16 keeps the upper 16 bits of the fp32 pattern.  The discarded low half
    rounds the kept part up when it exceeds 0x8000, or equals 0x8000 while
    the kept part is odd.  Adding 0x7FFF plus the kept part's lowest bit and
    then dropping the low 16 bits does exactly that (a carry into the
    exponent is the correct rounding up to the next binade or to infinity).
    """
    bits = np.ascontiguousarray(values_f32, dtype=np.float32).view(np.uint32)
    wide = bits.astype(np.uint64)
    kept_lsb = (wide >> 16) & 1
    return ((wide + 0x7FFF + kept_lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp64 exactly (bf16 -> fp32 is a shift)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_rne_bits(values_f32: np.ndarray) -> np.ndarray:
    """Round fp32 values to IEEE binary16 (round to nearest even, with
    subnormals and overflow to infinity) and return the bits -- numpy's
    float32 -> float16 conversion, which is that IEEE operation."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    with np.errstate(over="ignore"):
        return v.astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen binary16 bit patterns to fp64 exactly."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Level-1 quantiser: blockwise absmax, NF4 codes, nibble packing
# --------------------------------------------------------------------------

def quantize_nf4(w: np.ndarray, blocksize: int = BLOCK):
    """Blockwise NF4 quantisation of an fp32 tensor, flattened row-major.

    "QLoRA" (infivelines.com): each block of 64 weights carries its own
    scale, the block's largest magnitude, and each weight becomes the 4-bit
    index of the NF4 level nearest to weight / scale.

    Returns ``(codes, packed, absmax)``:
      codes  uint8 [n]            one code 0..15 per element
      packed uint8 [ceil(n/2)]    byte j = codes[2j] | codes[2j+1] << 4
      absmax fp32  [ceil(n/64)]   the exact per-block max |w|
    The last block may be partial; its absmax covers only real elements.
    """
    flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = flat.size
    n_blocks = (n + blocksize - 1) // blocksize
    thresholds = nf4_thresholds_f32()

    padded = np.zeros(n_blocks * blocksize, dtype=np.float32)
    padded[:n] = flat
    blocks = padded.reshape(n_blocks, blocksize)
    absmax = np.abs(blocks).max(axis=1).astype(np.float32)   # exact

    # u = fp32(w / absmax), correctly rounded: the fp64 quotient is rounded
    # once more to fp32, which equals direct correctly-rounded fp32 division
    # because 53 >= 2*24 + 2.
    safe = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float64)
    u = (blocks.astype(np.float64) / safe[:, None]).astype(np.float32)

    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for t in thresholds:                # count thresholds strictly below u
        codes += (u > t).astype(np.uint8)
    codes[absmax == 0, :] = 7           # all-zero block -> the zero level
    codes = codes.reshape(-1)[:n]

    return codes, pack_codes(codes), absmax


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, even element in the low nibble; an odd tail
    is padded with the zero level's code 7."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.array([7], dtype=np.uint8)])
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: the first ``n`` codes."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out[:n]


# --------------------------------------------------------------------------
# Level-2: double quantisation of the block scales
# --------------------------------------------------------------------------

def double_quant(absmax: np.ndarray, blocksize2: int = GROUP):
    """Quantise the fp32 block scales to 8 bits in groups of 256.

    "QLoRA" (infivelines.com) / "QLoRA -- Module 12.4", "Double quant": the
    quantisation constants are themselves quantised, in blocks of 256.  The
    8-bit format is not given; the reading here is an unsigned linear grid
    per group (scales are >= 0): step = fp32(group max / 255) and
    q = min(255, round-half-even(fp32(scale / step))), one fp32 step stored
    per group.  A group whose step is 0 stores q = 0 everywhere.

    Returns ``(q, step)``: uint8 [n_blocks], fp32 [ceil(n_blocks/256)].
    """
    s = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    nb = s.size
    ng = (nb + blocksize2 - 1) // blocksize2
    padded = np.zeros(ng * blocksize2, dtype=np.float32)
    padded[:nb] = s
    groups = padded.reshape(ng, blocksize2)

    gmax = groups.max(axis=1).astype(np.float64)
    step = (gmax / 255.0).astype(np.float32)          # correctly rounded
    live = step > 0
    safe = np.where(live, step, np.float32(1.0)).astype(np.float64)
    ratio = (groups.astype(np.float64) / safe[:, None]).astype(np.float32)
    q = np.minimum(np.rint(ratio), 255.0)             # rint: half to even
    q[~live, :] = 0
    return q.reshape(-1)[:nb].astype(np.uint8), step


def dequant_scales(q: np.ndarray, step: np.ndarray,
                   blocksize2: int = GROUP) -> np.ndarray:
    """s'_b = fp32(q_b * step_group(b)); the product is exact in fp64."""
    qq = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1)
    st = np.ascontiguousarray(step, dtype=np.float32).reshape(-1)
    group_of_block = np.arange(qq.size) // blocksize2
    return (qq.astype(np.float64) * st[group_of_block].astype(np.float64)
            ).astype(np.float32)


def dequant_nf4_bits(packed: np.ndarray, q: np.ndarray, step: np.ndarray,
                     n: int, blocksize: int = BLOCK,
                     blocksize2: int = GROUP) -> np.ndarray:
    """Dequantise to bf16 bit patterns, bit-exactly.

    "QLoRA" (infivelines.com): the stored base is dequantised to bf16.  The
    reading: w' = bf16_rne(fp32(L32[code] * s')) with s' the decoded block
    scale -- one fp32 product (exact in fp64, then rounded once), then a
    round-to-nearest-even to bf16.
    """
    codes = unpack_codes(packed, n)
    scale = dequant_scales(q, step, blocksize2)
    block_of_elem = np.arange(n) // blocksize
    levels = nf4_levels_f32().astype(np.float64)
    prod = (levels[codes] * scale[block_of_elem].astype(np.float64)
            ).astype(np.float32)
    return bf16_rne_bits(prod)


def dequant_nf4_f16_bits(packed: np.ndarray, q: np.ndarray, step: np.ndarray,
                         n: int, blocksize: int = BLOCK,
                         blocksize2: int = GROUP) -> np.ndarray:
    """Dequantise to fp16 bit patterns, bit-exactly: the fp16 compute-type
    variant.  "QLoRA: Fine-Tuning a 7B Model on a 16GB GPU" (digipro.cn),
    the flags paragraph: compute_dtype float16 dequantises to fp16 for the
    matrix multiplies.  Reading: as the bf16 dequantisation, with the one
    fp32 product rounded to binary16 (nearest even) instead:
    w' = fp16_rne(fp32(L32[code] * s')).
    """
    codes = unpack_codes(packed, n)
    scale = dequant_scales(q, step, blocksize2)
    block_of_elem = np.arange(n) // blocksize
    levels = nf4_levels_f32().astype(np.float64)
    prod = (levels[codes] * scale[block_of_elem].astype(np.float64)
            ).astype(np.float32)
    return f16_rne_bits(prod)


def storage_bits_per_weight(n: int, double_quantised: bool = True,
                            blocksize: int = BLOCK,
                            blocksize2: int = GROUP) -> float:
    """Bits stored per weight for ``n`` weights in this format.

    4-bit codes, plus per block either one fp32 scale (no double quant) or
    one 8-bit code, plus one fp32 step per group of 256 blocks.
    """
    n_blocks = math.ceil(n / blocksize)
    code_bits = 8 * math.ceil(n / 2)
    if double_quantised:
        scale_bits = 8 * n_blocks + 32 * math.ceil(n_blocks / blocksize2)
    else:
        scale_bits = 32 * n_blocks
    return (code_bits + scale_bits) / n
