"""Host tests of the comparison helpers the GPU parity tests use."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import bf16_floor, check_close_bf16, half_ulp_bf16


def _bf16(v: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f64(oracle.bf16_rne_bits(np.asarray(v, dtype=np.float32)))


def test_half_ulp_bf16_values():
    # bf16 keeps 8 significant bits: spacing 2^-7 on [1, 2), 2^-8 on [0.5, 1)
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([1.99]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([0.75]))[0] == 2.0 ** -9
    assert half_ulp_bf16(np.array([-3.0]))[0] == 2.0 ** -7


def test_half_ulp_bounds_bf16_rounding():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))
    x = x.astype(np.float32).astype(np.float64)
    assert np.all(np.abs(_bf16(x) - x) <= half_ulp_bf16(x))
    # and it is attained: values halfway between two bf16 numbers
    mid = 1.0 + 2.0 ** -8
    assert abs(_bf16(np.array([mid]))[0] - mid) == half_ulp_bf16(np.array([mid]))[0]


def _outlier_case():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(4096) * 0.01
    ref[17] = 2.26  # a x10 outlier whose half-ulp is a large share of the rms
    return ref


def test_floor_decides_and_exact_rounding_passes():
    ref = _outlier_case()
    assert bf16_floor(ref) > 2e-2
    check_close_bf16("y", _bf16(ref), ref)


def test_floor_decides_and_a_two_ulp_miss_fails():
    ref = _outlier_case()
    got = _bf16(ref)
    got[17] += 4 * half_ulp_bf16(np.array([got[17]]))[0] + 2e-2 * np.sqrt(np.mean(ref ** 2))
    with pytest.raises(AssertionError):
        check_close_bf16("y", got, ref)


def test_plain_bar_when_floor_is_small():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal(4096)
    assert bf16_floor(ref) <= 2e-2
    got = ref.copy()
    got[5] += 0.03 * np.sqrt(np.mean(ref ** 2))
    with pytest.raises(AssertionError):
        check_close_bf16("y", got, ref)
