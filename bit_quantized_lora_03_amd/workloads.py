"""Seeded synthetic inputs for the QLoRA linear layer (no method arithmetic).

The pages' workloads need trained checkpoints and a dataset (a 7B/8B chat
model, about 2,000 examples of ~512 tokens) that are not used here.  These
generators stand in for them with the same shapes and value distributions:

* base weights fp32 ~ N(0, sigma) (second parameter = standard deviation),
  optionally with a fraction of entries multiplied by 10 (heavy tails);
* activations ``x`` and upstream gradients ``dy`` bf16 ~ N(0, 1);
* LoRA factors ``A`` [r, K] and ``B`` [N, r] bf16 ~ N(0, 0.01).

bf16 values are the round-to-nearest-even of fp32 draws.  Every array has
its own PCG64 stream, ``numpy.random.default_rng([seed, index])``, so any
array can be drawn without drawing the others.  This module is the only
code that the oracle side and the HIP side share; it contains none of the
quantisation or layer arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional

import numpy as np


def _rng(seed: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(index)])


def normal_f32(seed: int, index: int, shape, sigma: float) -> np.ndarray:
    """fp32 N(0, sigma) draws (fp32 standard normals times fp32 sigma)."""
    z = _rng(seed, index).standard_normal(shape, dtype=np.float32)
    z *= np.float32(sigma)
    return z


def to_bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return uint16 patterns.

    Input preparation only: the generated bf16 inputs are these patterns.
    """
    u = np.ascontiguousarray(values_f32, dtype=np.float32).view(np.uint32)
    u64 = u.astype(np.uint64)
    return ((u64 + 0x7FFF + ((u64 >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """The exact fp32 values of bf16 patterns."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << 16).view(np.float32)


def weight_f32(seed: int, index: int, n: int, k: int, sigma: float,
               outlier_frac: float = 0.0) -> np.ndarray:
    """Base weight [n, k] fp32 ~ N(0, sigma); ``round(outlier_frac*n*k)``
    distinct positions (uniform, without replacement) are multiplied by 10."""
    w = normal_f32(seed, index, (n, k), sigma)
    if outlier_frac:
        count = int(round(outlier_frac * n * k))
        pos = _rng(seed, index + 1000).choice(n * k, size=count, replace=False)
        flat = w.reshape(-1)
        flat[pos] *= np.float32(10.0)
    return w


def keep_mask(seed: int, index: int, M: int, K: int, p: float) -> np.ndarray:
    """A LoRA-dropout keep mask [M, K] (uint8 0/1): each element kept with
    probability 1 - p, from its own seeded stream."""
    return (_rng(seed, index).random((M, K)) >= p).astype(np.uint8)


def pack_keep(keep: np.ndarray) -> np.ndarray:
    """[M, K] 0/1 -> the library's packed layout [M, K/8]: bit (k mod 8) of
    byte (m, k / 8) is keep[m, k]."""
    return np.packbits(np.ascontiguousarray(keep, dtype=np.uint8), axis=1, bitorder="little")


@dataclass
class Layer:
    """One linear layer's inputs.  Arrays are drawn lazily on first access."""
    name: str
    M: int
    N: int
    K: int
    r: int
    alpha: float
    seed: int
    base_index: int = 0
    w_sigma: float = 0.02
    outlier_frac: float = 0.0
    w_override: Optional[Callable[[], np.ndarray]] = None
    x_override: Optional[Callable[[], np.ndarray]] = None
    _cache: Dict[str, np.ndarray] = field(default_factory=dict, repr=False)

    # stream indices within the layer (x/dy/A/B/W)
    def _get(self, key, make):
        if key not in self._cache:
            self._cache[key] = make()
        return self._cache[key]

    @property
    def w(self) -> np.ndarray:
        """fp32 [N, K] base weight (out x in)."""
        if self.w_override is not None:
            return self._get("w", self.w_override)
        return self._get("w", lambda: weight_f32(
            self.seed, self.base_index + 0, self.N, self.K, self.w_sigma,
            self.outlier_frac))

    @property
    def x_bits(self) -> np.ndarray:
        """bf16 [M, K] activations."""
        if self.x_override is not None:
            return self._get("x", self.x_override)
        return self._get("x", lambda: to_bf16_bits(normal_f32(
            self.seed, self.base_index + 1, (self.M, self.K), 1.0)))

    @property
    def A_bits(self) -> np.ndarray:
        """bf16 [r, K] LoRA down-projection."""
        return self._get("A", lambda: to_bf16_bits(normal_f32(
            self.seed, self.base_index + 2, (self.r, self.K), 0.01)))

    @property
    def B_bits(self) -> np.ndarray:
        """bf16 [N, r] LoRA up-projection."""
        return self._get("B", lambda: to_bf16_bits(normal_f32(
            self.seed, self.base_index + 3, (self.N, self.r), 0.01)))

    @property
    def dy_bits(self) -> np.ndarray:
        """bf16 [M, N] upstream gradient."""
        return self._get("dy", lambda: to_bf16_bits(normal_f32(
            self.seed, self.base_index + 4, (self.M, self.N), 1.0)))

    def f32(self, name: str) -> np.ndarray:
        """Exact fp32 values of a bf16 input ('x', 'A', 'B' or 'dy')."""
        return bf16_bits_as_f32(getattr(self, name + "_bits"))

    def drop(self):
        self._cache.clear()


def layer(M, N, K, r, alpha, seed, name="custom", w_sigma=0.02,
          outlier_frac=0.0, base_index=0) -> Layer:
    return Layer(name, M, N, K, r, alpha, seed, base_index, w_sigma,
                 outlier_frac)


# ---------------------------------------------------------------------------
# The five workloads (shapes of the pages' 7B / 65B-class models)
# ---------------------------------------------------------------------------

def tiny_256() -> Layer:
    """Single 256x256 linear, M=16 tokens, LoRA r=8 alpha=16, seed 0."""
    return layer(16, 256, 256, 8, 16.0, seed=0, name="linear256_m16_r8")


def q_proj_4096() -> Layer:
    """7B-attention q_proj 4096x4096 with 0.1 % outliers x10, M=512 tokens
    (batch 1 x seq 512), LoRA r=16 alpha=32."""
    return layer(512, 4096, 4096, 16, 32.0, seed=1, name="q_proj4096_m512_r16",
                 outlier_frac=0.001)


def mlp_7b():
    """7B MLP: gate and up 4096->11008, down 11008->4096, M=2048 tokens
    (batch 4 x seq 512), LoRA r=16 alpha=32 on all three.  Gate and up share
    one activation; down has its own."""
    seed = 2
    gate = layer(2048, 11008, 4096, 16, 32.0, seed, "mlp_gate", base_index=0)
    up = layer(2048, 11008, 4096, 16, 32.0, seed, "mlp_up", base_index=10)
    down = layer(2048, 4096, 11008, 16, 32.0, seed, "mlp_down", base_index=20)
    shared = lambda: to_bf16_bits(normal_f32(seed, 100, (2048, 4096), 1.0))
    gate.x_override = shared
    up.x_override = shared
    return [gate, up, down]


DECODE_ROTATION = 16


def decode_8192(M: int, j: int = 0) -> Layer:
    """Decode-like 8192x8192 base, M in {1, 4, 16}, LoRA r=64 alpha=16, fwd
    only.  ``j`` picks one of 16 independent weights (a rotation set larger
    than the on-package cache); x/A/B do not depend on ``j``."""
    seed = 3
    L = layer(M, 8192, 8192, 64, 16.0, seed, f"decode8192_m{M}_w{j}")
    L.w_override = lambda: weight_f32(seed, 1000 + j, 8192, 8192, 0.02)
    L.x_override = lambda: to_bf16_bits(normal_f32(seed, 200 + M, (M, 8192), 1.0))
    return L


def layer_65b() -> Layer:
    """65B-class 8192->22016 with double quant, W ~ N(0, 0.015), M=4096
    tokens (batch 8 x seq 512), LoRA r=64 alpha=16; quantise + fwd + bwd."""
    return layer(4096, 22016, 8192, 64, 16.0, seed=4, name="up65b_m4096_r64",
                 w_sigma=0.015)


WORKLOADS = {
    "linear256_m16_r8": tiny_256,
    "q_proj4096_m512_r16": q_proj_4096,
    "up65b_m4096_r64": layer_65b,
}
