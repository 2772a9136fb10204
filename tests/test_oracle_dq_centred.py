"""Pins of the oracle's mean-centred double quantisation (CPU only).

* A hand-worked group: scales 1, 2, 3, 4 -> mean 2.5, codes -127, -42, 42,
  127, step the fp32 nearest 1.5 / 127 (checked with exact rationals).
* The mean is the fp32 nearest the exact rational mean of the fp32 scales
  (tensors with one group, many groups, and more groups than the summation
  has chunks).
* Reconstruction: every decoded scale lies within step / 2 (plus the
  roundings the definition makes) of its scale; each live group's largest
  |scale - mean| takes code +-127; no code is -128.
* Special cases: a constant tensor is reconstructed exactly; all-zero
  scales give zero codes and steps; a group symmetric about the mean gets
  antisymmetric codes.
* The decoded scale is a product and a sum each rounded once (exact
  rational arithmetic on cases where a fused multiply-add would differ),
  and the bf16 dequantisation is the element formula by brute force.
* Planted mistakes (grid 255 instead of 127, no centring, a fused
  decode) fail these pins.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.dq_centred as dqc


def _nearest_f32(x: Fraction) -> np.float32:
    """The fp32 value nearest the rational x (ties to even mantissa)."""
    f = np.float32(float(x))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - x)
        key = (err, int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def _exact_mean(s: np.ndarray) -> Fraction:
    # every fp32 value is an integer multiple of 2^-149
    ints = (np.asarray(s, dtype=np.float32).astype(np.float64) * 2.0 ** 149)
    total = sum(int(v) for v in ints)  # exact: the fp64 scaling is exact for fp32 inputs
    return Fraction(total, s.size * (1 << 149))


def test_hand_worked_group():
    s = np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32)
    q, step, mu = oracle.double_quant_centred(s)
    assert mu == np.float32(2.5)
    assert list(q.view(np.int8)) == [-127, -42, 42, 127]
    assert step.shape == (1,)
    assert step[0] == _nearest_f32(Fraction(3, 254))
    sp = oracle.dequant_scales_centred(q, step, mu)
    # s'_0 = fp32(fp32(-127 step) + 2.5): here 127 step rounds to exactly 1.5
    assert sp[0] == np.float32(1.0) and sp[3] == np.float32(4.0)


@pytest.mark.parametrize("nb,seed", [(37, 0), (256, 1), (5000, 2), (256 * 1500 + 77, 3),
                                     (256 * 2100, 4)])
def test_mean_is_the_nearest_fp32_of_the_exact_mean(nb, seed):
    rng = np.random.default_rng(seed)
    s = np.abs(rng.standard_normal(nb) * 0.05).astype(np.float32) + np.float32(0.01)
    s[::97] *= np.float32(30.0)                      # heavy tail
    assert oracle.centred_mean(s) == _nearest_f32(_exact_mean(s))


def _absmax_of_weight(seed=5, n=1024 * 4096, sigma=0.02, outliers=True):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n) * sigma).astype(np.float32)
    if outliers:
        w[rng.integers(0, n, n // 1000)] *= 10
    return np.abs(w.reshape(-1, 64)).max(axis=1).astype(np.float32)


def test_reconstruction_bound_and_extreme_codes():
    s = _absmax_of_weight()
    q, step, mu = oracle.double_quant_centred(s)
    sp = oracle.dequant_scales_centred(q, step, mu).astype(np.float64)
    qs = q.view(np.int8).astype(np.int64)
    g = np.arange(s.size) // 256
    st = step[g].astype(np.float64)
    d = (s - mu).astype(np.float32).astype(np.float64)
    ulp = lambda v: np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)
    bound = st * (0.5 + 127 * 2.0 ** -24) + ulp(d) / 2 + ulp(qs * st) / 2 + ulp(sp) / 2
    assert np.all(np.abs(sp - s) <= bound)
    assert np.all(np.abs(qs) <= 127)
    for gi in range(step.size):
        if step[gi] > 0:
            assert np.abs(qs[g == gi]).max() == 127


def test_constant_zero_and_symmetric_cases():
    c = np.full(700, 0.75, dtype=np.float32)
    q, step, mu = oracle.double_quant_centred(c)
    assert mu == np.float32(0.75) and np.all(step == 0) and np.all(q == 0)
    assert np.array_equal(oracle.dequant_scales_centred(q, step, mu), c)

    z = np.zeros(300, dtype=np.float32)
    q, step, mu = oracle.double_quant_centred(z)
    assert mu == 0 and np.all(step == 0) and np.all(q == 0)
    assert np.all(oracle.dequant_scales_centred(q, step, mu) == 0)

    deltas = np.array([0.25, 0.5, 0.125, 0.375], dtype=np.float32)
    s = np.concatenate([2.0 + deltas, 2.0 - deltas]).astype(np.float32)
    q, step, mu = oracle.double_quant_centred(s)
    assert mu == np.float32(2.0)
    qs = q.view(np.int8)
    assert np.array_equal(qs[:4], -qs[4:])


def test_decoded_scale_rounds_product_and_sum_separately():
    rng = np.random.default_rng(7)
    found = 0
    for _ in range(4000):
        qv = int(rng.integers(-127, 128))
        step = np.float32(rng.uniform(1e-4, 1e-2))
        mu = np.float32(rng.uniform(0.01, 0.1))
        two = _nearest_f32(Fraction(float(_nearest_f32(qv * Fraction(float(step))))) +
                           Fraction(float(mu)))
        fused = _nearest_f32(qv * Fraction(float(step)) + Fraction(float(mu)))
        if two != fused:
            got = oracle.dequant_scales_centred(np.array([qv], dtype=np.int8).view(np.uint8),
                                                np.array([step], dtype=np.float32), mu)
            assert got[0] == two
            found += 1
            if found == 20:
                break
    assert found == 20


def test_dequant_bits_by_brute_force():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal(256) * 0.03).astype(np.float32)
    codes, packed, absmax = oracle.quantize_nf4(w)
    q, step, mu = oracle.double_quant_centred(absmax)
    bits = oracle.dequant_nf4_centred_bits(packed, q, step, mu, w.size)
    lv = oracle.nf4_levels_f32()
    qs = q.view(np.int8)
    for i in range(w.size):
        b = i // 64
        sp = _nearest_f32(Fraction(float(_nearest_f32(int(qs[b]) * Fraction(float(step[0]))))) +
                          Fraction(float(mu)))
        prod = _nearest_f32(Fraction(float(lv[codes[i]])) * Fraction(float(sp)))
        u = int(np.array(prod, dtype=np.float32).view(np.uint32))
        # bf16 round-to-nearest-even of the fp32 bits
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        assert int(bits[i]) == r, i


def test_centring_tightens_the_scales_of_a_normal_weight():
    """The point of the variant: on scales of normal weights (a narrow band
    far from zero) the symmetric code over [mean - A, mean + A] has a finer
    step than the unsigned one over [0, max].  (With outlier blocks the
    band is one-sided and the centred code is the coarser one: checked
    too.)"""
    s = _absmax_of_weight(seed=9, outliers=False)
    qc, stc, mu = oracle.double_quant_centred(s)
    qu, stu = oracle.double_quant(s)
    err_c = np.abs(oracle.dequant_scales_centred(qc, stc, mu).astype(np.float64) - s).mean()
    err_u = np.abs(oracle.dequant_scales(qu, stu).astype(np.float64) - s).mean()
    assert err_c < 0.8 * err_u
    s = _absmax_of_weight(seed=9, outliers=True)
    qc, stc, mu = oracle.double_quant_centred(s)
    qu, stu = oracle.double_quant(s)
    err_c = np.abs(oracle.dequant_scales_centred(qc, stc, mu).astype(np.float64) - s).mean()
    err_u = np.abs(oracle.dequant_scales(qu, stu).astype(np.float64) - s).mean()
    assert err_c > err_u


@pytest.mark.parametrize("plant", ["grid 255", "no centring", "fused decode"])
def test_planted_mistakes_are_caught(monkeypatch, plant):
    if plant == "grid 255":
        monkeypatch.setattr(dqc, "QMAX", 255)
        with pytest.raises(AssertionError):
            test_hand_worked_group()
    elif plant == "no centring":
        monkeypatch.setattr(dqc, "centred_mean", lambda s, blocksize2=256: np.float32(0.0))
        with pytest.raises(AssertionError):
            test_hand_worked_group()
    else:
        def fused(q, step, mu, blocksize2=256):
            qs = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1).view(np.int8)
            st = np.ascontiguousarray(step, dtype=np.float32).reshape(-1)
            g = np.arange(qs.size) // blocksize2
            return (qs.astype(np.float64) * st[g].astype(np.float64) +
                    np.float64(mu)).astype(np.float32)
        monkeypatch.setattr(dqc, "dequant_scales_centred", fused)
        monkeypatch.setattr(oracle, "dequant_scales_centred", fused)
        with pytest.raises(AssertionError):
            test_decoded_scale_rounds_product_and_sum_separately()
