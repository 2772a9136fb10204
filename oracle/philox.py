"""Counter-based random draws for LoRA dropout: Philox4x32-10 and the keep
mask it defines.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "QLoRA -- Module 12.4", "Hugging Face + BitsAndBytes": the adapter config
  sets lora_dropout (0.05).  The pages give neither the formula nor a
  generator; the layer oracle (``lora_linear``) takes the keep mask as an
  input.  This module defines where that mask comes from when the library
  draws it itself.
* The generator is Philox4x32 with ten rounds, as published by Salmon,
  Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
  (SC 2011), section on the Philox family.  Its state is a 128-bit counter
  (four 32-bit words X0..X3) and a 64-bit key (K0, K1).  One round takes
  the two 64-bit products M0 * X0 and M1 * X2 (M0 = 0xD2511F53,
  M1 = 0xCD9E8D57) and forms the new words
      X0' = hi(M1 * X2) ^ X1 ^ K0,   X1' = lo(M1 * X2),
      X2' = hi(M0 * X0) ^ X3 ^ K1,   X3' = lo(M0 * X0);
  between rounds the key advances by the Weyl constants (K0 += 0x9E3779B9,
  K1 += 0xBB67AE85, modulo 2^32).  The ten rounds' result is the output.

Readings taken for the keep mask:

* The packed mask has the library's layout: byte b = m * (K / 8) + k / 8 of
  an [M, K] activation holds the keep bits of elements 8 (k / 8) .. + 7 of
  row m, bit j for element 8 (k / 8) + j.
* Byte b is drawn by one Philox call with counter (b mod 2^32, b >> 32,
  offset mod 2^32, offset >> 32) and key (seed mod 2^32, seed >> 32): the
  output's eight 16-bit halves u_j = (X_{j/2} >> 16 (j mod 2)) & 0xFFFF are
  the uniforms of the byte's eight elements.  seed picks the stream, offset
  separates the draws of different steps or layers under one seed.
* Element j is kept iff u_j >= t, with t the integer nearest to 65536 p
  (ties to even).  The dropout probability is therefore realised as
  t / 65536 (0.05 -> 3277 / 65536 = 0.0500030518), and the inverted
  scaling uses that realised value: 1 / (1 - t / 65536).
"""

from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counters: np.ndarray, key) -> np.ndarray:
    """Philox4x32 with ten rounds on each row of ``counters`` ([n, 4] words,
    X0..X3) under the 64-bit ``key`` (K0, K1).  Returns [n, 4] uint32.

    The round and key schedule are the published ones (module docstring);
    the 32 x 32 -> 64-bit products are exact in uint64."""
    c = np.asarray(counters, dtype=np.uint64).reshape(-1, 4)
    x0, x1, x2, x3 = (c[:, i].copy() for i in range(4))
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for rnd in range(ROUNDS):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = m0 * x0
        p1 = m1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(k0), lo1,
                          hi0 ^ x3 ^ np.uint64(k1), lo0)
    return np.stack([x0, x1, x2, x3], axis=1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """t = the integer nearest to 65536 p (p taken as fp32; ties to even):
    a draw u in [0, 65535] is dropped iff u < t."""
    v = float(np.float32(p)) * 65536.0
    return int(round(v))


def realised_dropout(p: float) -> float:
    """The dropout probability the 16-bit draws realise: t / 65536."""
    return dropout_threshold(p) / 65536.0


def dropout_uniforms(M: int, K: int, seed: int, offset: int) -> np.ndarray:
    """The 16-bit draw of every element of an [M, K] activation (K a
    multiple of 8), as uint16 [M, K]."""
    assert K % 8 == 0
    nbytes = M * (K // 8)
    b = np.arange(nbytes, dtype=np.uint64)
    ctr = np.empty((nbytes, 4), dtype=np.uint64)
    ctr[:, 0] = b & _MASK32
    ctr[:, 1] = b >> np.uint64(32)
    ctr[:, 2] = int(offset) & 0xFFFFFFFF
    ctr[:, 3] = (int(offset) >> 32) & 0xFFFFFFFF
    out = philox4x32_10(ctr, (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF))
    halves = np.empty((nbytes, 8), dtype=np.uint16)
    for j in range(8):
        halves[:, j] = (out[:, j // 2] >> np.uint32(16 * (j % 2))) & np.uint32(0xFFFF)
    return halves.reshape(M, K)


def dropout_keep_philox(M: int, K: int, p: float, seed: int, offset: int) -> np.ndarray:
    """The keep mask [M, K] (uint8 0/1) drawn from Philox4x32-10 for dropout
    probability p under (seed, offset): element kept iff its draw >= t."""
    u = dropout_uniforms(M, K, seed, offset)
    return (u.astype(np.int64) >= dropout_threshold(p)).astype(np.uint8)
