"""Pins for the oracle's NF4 level table and thresholds (CPU only).

The pages fix: 16 levels at normal quantiles, each about equally likely
("QLoRA", infivelines.com); the format is 4-bit with an exact zero and range
[-1, 1].  These tests check the oracle's table against those properties
using the normal CDF from ``math.erfc`` -- a different function from the
quantile routine the oracle builds the levels with.
"""

import math

import numpy as np
import pytest

import oracle


def phi(z: float) -> float:
    """Standard normal CDF from the complementary error function."""
    return 0.5 * math.erfc(-z / math.sqrt(2.0))


def phi_inverse_bisect(p: float) -> float:
    """Quantile by bisection on ``phi`` (independent of the oracle's routine)."""
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_sixteen_strictly_increasing_levels_with_exact_ends_and_zero():
    for L in (oracle.nf4_levels_f64(), oracle.nf4_levels_f32()):
        assert L.shape == (16,)
        assert np.all(np.diff(L) > 0)
        assert L[0] == -1.0 and L[15] == 1.0 and L[7] == 0.0
        # 8 levels above zero, 7 below
        assert (L > 0).sum() == 8 and (L < 0).sum() == 7


def test_levels_sit_at_evenly_spaced_normal_probabilities():
    """Phi(level * q_top) must step evenly from 1/2 to P_MAX on each side."""
    L = oracle.nf4_levels_f64()
    top = phi_inverse_bisect(oracle.P_MAX)
    pm = oracle.P_MAX
    # positive side: levels 8..15 -> 1/2 + (P_MAX - 1/2) * (j+1)/8
    for j in range(8):
        want = 0.5 + (pm - 0.5) * (j + 1) / 8
        assert abs(phi(L[8 + j] * top) - want) < 1e-12
    # negative side: levels 0..6 -> Phi(-L) = P_MAX - (P_MAX - 1/2) * i/7
    for i in range(7):
        want = pm - (pm - 0.5) * i / 7
        assert abs(phi(-L[i] * top) - want) < 1e-12


def test_p_max_is_mean_of_outer_bin_centres():
    assert oracle.P_MAX == pytest.approx(0.5 * ((1 - 1 / 30) + (1 - 1 / 32)), abs=0)
    assert oracle.P_MAX == pytest.approx(0.9677083333333333, abs=1e-15)


def test_fp32_levels_are_the_rounded_fp64_levels():
    L64 = oracle.nf4_levels_f64()
    L32 = oracle.nf4_levels_f32()
    for a, b in zip(L64, L32):
        b = float(b)
        # b is the fp32 nearest to a: its neighbours are farther away
        up = float(np.nextafter(np.float32(b), np.float32(np.inf)))
        dn = float(np.nextafter(np.float32(b), np.float32(-np.inf)))
        assert abs(a - b) <= abs(a - up) and abs(a - b) <= abs(a - dn)


def test_thresholds_separate_levels_and_are_round_down_midpoints():
    L = oracle.nf4_levels_f32().astype(np.float64)
    T = oracle.nf4_thresholds_f32()
    assert T.shape == (15,) and T.dtype == np.float32
    for i in range(15):
        m = (L[i] + L[i + 1]) / 2
        t = float(T[i])
        assert L[i] < t < L[i + 1]
        assert t <= m
        nxt = float(np.nextafter(np.float32(t), np.float32(np.inf)))
        assert nxt > m          # t is the largest fp32 not above the midpoint


def test_equal_occupancy_in_quantile_space():
    """Nearest-level cells of z / q_top for z ~ N(0,1) each hold about 1/16.

    "QLoRA" (infivelines.com): each level is about equally likely.  The exact
    cell masses are computed with the normal CDF and must lie within
    [0.85, 1.15] / 16; a Monte Carlo of 10^6 draws agrees with them to 5 sigma.
    """
    T = oracle.nf4_thresholds_f32().astype(np.float64)
    top = phi_inverse_bisect(oracle.P_MAX)
    edges = [-math.inf] + [t * top for t in T] + [math.inf]
    masses = np.array([phi(edges[i + 1]) - phi(edges[i]) for i in range(16)])
    assert masses.sum() == pytest.approx(1.0, abs=1e-12)
    assert np.all(masses > 0.85 / 16) and np.all(masses < 1.15 / 16)

    n = 1_000_000
    z = np.random.default_rng(12345).standard_normal(n)
    u = np.clip(z / top, -1, 1).astype(np.float32)
    codes = np.zeros(n, dtype=np.int64)
    for t in oracle.nf4_thresholds_f32():
        codes += u > t
    counts = np.bincount(codes, minlength=16) / n
    sigma = np.sqrt(masses * (1 - masses) / n)
    assert np.all(np.abs(counts - masses) < 5 * sigma)


def test_levels_independent_of_quantile_routine():
    """Rebuild the levels from the bisection quantile; they agree to 1e-12."""
    top = phi_inverse_bisect(oracle.P_MAX)
    pm = oracle.P_MAX
    pos = [phi_inverse_bisect(pm + (0.5 - pm) * i / 8) for i in range(8)]
    neg = [-phi_inverse_bisect(pm + (0.5 - pm) * i / 7) for i in range(7)]
    rebuilt = np.array(sorted(neg + [0.0] + pos)) / top
    assert np.max(np.abs(rebuilt - oracle.nf4_levels_f64())) < 1e-12
