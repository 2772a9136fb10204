"""Pins for the oracle's LoRA dropout (CPU only).

The mask is an input, so the layer stays linear in x, A and B for a fixed
mask: the adjoint identities pin the backward against the forward, as for
the layer without dropout.  The forward is pinned by a pure-Python triple
loop; the limits p = 0 with every element kept (the layer without dropout,
exactly) and nothing kept (the base alone); and the inverted scaling by
its mean: over many masks, E[x~] = x.
"""

import numpy as np
import pytest

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def mask(shape, seed, p):
    return (np.random.default_rng(seed).random(shape) >= p).astype(np.uint8)


def triple_loop_fwd(x, W, A, B, alpha, keep, p):
    M, K, N, r = len(x), len(x[0]), len(W), len(A)
    s = alpha / r
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        xd = [x[m][k] * keep[m][k] / (1.0 - p) for k in range(K)]
        xa = [sum(xd[k] * A[j][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            y[m][n] = (sum(x[m][k] * W[n][k] for k in range(K))
                       + s * sum(xa[j] * B[n][j] for j in range(r)))
    return np.array(y)


@pytest.mark.parametrize("M,N,K,r,alpha,p", [(3, 5, 7, 2, 4.0, 0.25), (4, 3, 6, 3, 9.0, 0.05)])
def test_forward_equals_triple_loop(M, N, K, r, alpha, p):
    x, W = rand((M, K), 1), rand((N, K), 2)
    A, B = rand((r, K), 3), rand((N, r), 4)
    keep = mask((M, K), 5, p)
    ref = triple_loop_fwd(x.tolist(), W.tolist(), A.tolist(), B.tolist(), alpha,
                          keep.tolist(), p)
    got = oracle.lora_linear_fwd(x, W, A, B, alpha, keep=keep, p=p)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_p0_with_everything_kept_is_the_layer_without_dropout():
    M, N, K, r, alpha = 5, 7, 9, 3, 6.0
    x, W, A, B, dy = rand((M, K), 6), rand((N, K), 7), rand((r, K), 8), rand((N, r), 9), \
        rand((M, N), 10)
    ones = np.ones((M, K), dtype=np.uint8)
    assert np.array_equal(oracle.lora_linear_fwd(x, W, A, B, alpha, keep=ones, p=0.0),
                          oracle.lora_linear_fwd(x, W, A, B, alpha))
    for u, v in zip(oracle.lora_linear_bwd(x, dy, W, A, B, alpha, keep=ones, p=0.0),
                    oracle.lora_linear_bwd(x, dy, W, A, B, alpha)):
        assert np.array_equal(u, v)


def test_nothing_kept_leaves_the_base_alone():
    """keep = 0: y = x.W^T, dX = dy.W, dA = dB = 0 -- dropout acts on the
    adapter's input only, never on the base term."""
    M, N, K, r, alpha, p = 4, 6, 8, 2, 4.0, 0.3
    x, W, A, B, dy = rand((M, K), 11), rand((N, K), 12), rand((r, K), 13), rand((N, r), 14), \
        rand((M, N), 15)
    zero = np.zeros((M, K), dtype=np.uint8)
    assert np.allclose(oracle.lora_linear_fwd(x, W, A, B, alpha, keep=zero, p=p), x @ W.T,
                       rtol=1e-13, atol=1e-13)
    dX, dA, dB = oracle.lora_linear_bwd(x, dy, W, A, B, alpha, keep=zero, p=p)
    assert np.allclose(dX, dy @ W, rtol=1e-13, atol=1e-13)
    assert np.all(dA == 0) and np.all(dB == 0)


def test_inverted_scaling_keeps_the_mean():
    """Averaged over many masks drawn with P(keep) = 1 - p, x~ = x; without
    the 1/(1 - p) factor the mean would be (1 - p) x."""
    p = 0.25
    x = rand((4, 5), 16)
    rng = np.random.default_rng(17)
    n = 40000
    acc = np.zeros_like(x)
    for _ in range(n // 1000):
        keep = (rng.random((1000,) + x.shape) >= p)
        acc += oracle.dropped_input(x[None], keep, p).sum(axis=0)
    mean = acc / n
    # standard error of each mean: |x| sqrt(p / (1 - p) / n)
    se = np.abs(x) * np.sqrt(p / (1 - p) / n)
    assert np.all(np.abs(mean - x) <= 5 * se + 1e-12)


def _case(seed, M=6, N=10, K=12, r=3, alpha=6.0, p=0.2):
    x, W = rand((M, K), seed), rand((N, K), seed + 1)
    A, B = rand((r, K), seed + 2), rand((N, r), seed + 3)
    dy = rand((M, N), seed + 4)
    keep = mask((M, K), seed + 5, p)
    return x, W, A, B, dy, alpha, keep, p


@pytest.mark.parametrize("seed", [60, 70])
def test_adjoint_identity_for_x(seed):
    x, W, A, B, dy, alpha, keep, p = _case(seed)
    dX, _, _ = oracle.lora_linear_bwd(x, dy, W, A, B, alpha, keep=keep, p=p)
    v = rand(x.shape, seed + 9)
    jv = oracle.lora_linear_fwd(v, W, A, B, alpha, keep=keep, p=p)
    lhs, rhs = np.sum(dy * jv), np.sum(dX * v)
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


@pytest.mark.parametrize("seed", [60, 70])
def test_adjoint_identity_for_A(seed):
    x, W, A, B, dy, alpha, keep, p = _case(seed)
    _, dA, _ = oracle.lora_linear_bwd(x, dy, W, A, B, alpha, keep=keep, p=p)
    V = rand(A.shape, seed + 9)
    jv = oracle.lora_linear_fwd(x, np.zeros_like(W), V, B, alpha, keep=keep, p=p)
    lhs, rhs = np.sum(dy * jv), np.sum(dA * V)
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


@pytest.mark.parametrize("seed", [60, 70])
def test_adjoint_identity_for_B(seed):
    x, W, A, B, dy, alpha, keep, p = _case(seed)
    _, _, dB = oracle.lora_linear_bwd(x, dy, W, A, B, alpha, keep=keep, p=p)
    V = rand(B.shape, seed + 9)
    jv = oracle.lora_linear_fwd(x, np.zeros_like(W), A, V, alpha, keep=keep, p=p)
    lhs, rhs = np.sum(dy * jv), np.sum(dB * V)
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))
