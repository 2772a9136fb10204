"""Pins for the oracle's adapter merge (CPU only).

W_m = W_base + (alpha/r).B.A is pinned by a pure-Python triple loop on tiny
shapes, by the layer identity x.W_m^T = the adapted layer's forward output
(the forward oracle is pinned on its own), by a one-entry closed form that
catches a transposed or mis-scaled update, and by the zero adapter.  The
bf16 export is pinned on hand-picked values, including one where rounding
straight from fp64 and rounding through fp32 differ; re-quantisation on a
weight that already lies on the NF4 grid with unit block scales.
"""

import numpy as np
import pytest

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def triple_loop_merge(W, A, B, alpha):
    N, K, r = len(W), len(W[0]), len(A)
    s = alpha / r
    return np.array([[W[n][k] + s * sum(B[n][j] * A[j][k] for j in range(r))
                      for k in range(K)] for n in range(N)])


@pytest.mark.parametrize("N,K,r,alpha", [(3, 5, 2, 4.0), (4, 4, 1, 1.0), (2, 7, 3, 9.0)])
def test_merge_equals_triple_loop(N, K, r, alpha):
    W, A, B = rand((N, K), 1), rand((r, K), 2), rand((N, r), 3)
    ref = triple_loop_merge(W.tolist(), A.tolist(), B.tolist(), alpha)
    assert np.allclose(oracle.merge_adapter(W, A, B, alpha), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,N,K,r,alpha", [(5, 6, 8, 2, 16.0), (3, 9, 4, 4, 8.0)])
def test_merged_weight_reproduces_the_adapted_layer(M, N, K, r, alpha):
    """x.W_m^T equals y = x.W^T + (alpha/r).(x.A^T).B^T of the forward oracle."""
    x, W = rand((M, K), 4), rand((N, K), 5)
    A, B = rand((r, K), 6), rand((N, r), 7)
    W_m = oracle.merge_adapter(W, A, B, alpha)
    assert np.allclose(x @ W_m.T, oracle.lora_linear_fwd(x, W, A, B, alpha),
                       rtol=1e-12, atol=1e-12)


def test_one_entry_update_lands_at_row_of_B_column_of_A():
    """A[0, 2] = 1, B[5, 0] = 1: only W_m[5, 2] moves, by exactly alpha/r.
    A transposed update or a wrong scale moves another entry or another
    amount."""
    N, K, r, alpha = 8, 6, 2, 6.0
    W = rand((N, K), 8)
    A = np.zeros((r, K)); A[0, 2] = 1.0
    B = np.zeros((N, r)); B[5, 0] = 1.0
    d = oracle.merge_adapter(W, A, B, alpha) - W
    expect = np.zeros((N, K)); expect[5, 2] = 3.0
    assert np.array_equal(d, expect)


def test_zero_adapter_returns_the_base():
    W = rand((4, 6), 9)
    assert np.array_equal(oracle.merge_adapter(W, None, None, 8.0), W)
    assert np.array_equal(oracle.merge_adapter(W, np.zeros((0, 6)), np.zeros((4, 0)), 8.0), W)
    assert np.array_equal(oracle.merge_adapter(W, rand((2, 6), 10), np.zeros((4, 2)), 8.0), W)


def test_bf16_export_rounds_through_fp32_to_nearest_even():
    one = 1.0
    vals = np.array([
        one,                        # exact -> 0x3F80
        one + 2.0 ** -7,            # exact bf16 neighbour of 1 -> 0x3F81
        one + 2.0 ** -8,            # tie between 1 and 1+2^-7 -> even (1.0)
        one + 3 * 2.0 ** -8,        # tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
        one + 2.0 ** -8 + 2.0 ** -30,  # fp32 rounds this onto the tie -> 1.0
        -2.5,                       # exact -> 0xC020
    ])
    got = oracle.merged_bf16_bits(vals)
    assert got.tolist() == [0x3F80, 0x3F81, 0x3F80, 0x3F82, 0x3F80, 0xC020]


def test_requantize_keeps_a_weight_on_the_grid():
    """Every block holds the 16 levels (so its absmax is 1) four times over:
    quantised again and decoded, each value comes back as bf16 of its level."""
    lv = oracle.nf4_levels_f32()
    w = np.tile(lv, 4 * 256).reshape(64, 256)
    back = oracle.requantize(w)
    expect = oracle.bf16_bits_to_f64(oracle.bf16_rne_bits(w))
    assert np.array_equal(back, expect)


def test_requantize_reduces_to_the_scaled_grid():
    """A power-of-two multiple of the grid decodes as bf16 of that multiple
    (the scales then double-quantise exactly: q = 255 in every block)."""
    lv = oracle.nf4_levels_f32()
    w = (np.tile(lv, 4 * 256) * np.float32(0.25)).reshape(128, 128)
    back = oracle.requantize(w)
    expect = oracle.bf16_bits_to_f64(oracle.bf16_rne_bits(w))
    assert np.max(np.abs(back - expect)) <= 2.0 ** -8 * 0.25


def test_three_exports_order_as_the_pages_say():
    """Merging into the 4-bit base and quantising again loses precision
    twice: twice > once (the base's own quantisation error) > clean (bf16
    rounding of the ideal merge).  ``once`` is the trained-shift measure."""
    rng = np.random.default_rng(12)
    N, K, r, alpha = 128, 512, 16, 32.0
    w0 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((r, K)) * 0.01
    B = rng.standard_normal((N, r)) * 0.01
    e = oracle.merge_errors(w0, A, B, alpha)
    assert e["twice"] > 1.05 * e["once"]
    assert e["once"] > 10 * e["clean"]
    assert abs(e["once"] - e["trained_shift"]) < 1e-3 * e["once"]
