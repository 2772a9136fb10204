"""GPU parity of the layer with LoRA dropout on the adapter's input (keep
mask passed in, packed 8 bits per byte) against the fp64 oracle, through
the C ABI.

Bar: max|T_gpu - T_oracle| <= 2e-2 * rms(T_oracle) for y, dX, dA, dB; for
the bf16 outputs y and dX, the output's own rounding floor where that is
larger (one seeded case: an outlier-driven dX element of 2.26 has a bf16
half-ulp of 2.3 % of rms).
Exact cases: with nothing kept the layer is its base alone (y, dX equal
the base-only calls bit for bit, dA = dB = 0); with everything kept and
p = 0 the forward equals the layer without dropout bit for bit.
"""

import numpy as np
import pytest

import oracle
import bit_quantized_lora_03_amd as q
from bit_quantized_lora_03_amd import workloads
from tests.gpu_util import OracleLayer, bf16_values, check_close, check_close_bf16, dev, host

pytestmark = pytest.mark.gpu

# (M, N, K, r, alpha, p): few tokens (the decode path), the small and the MFMA
# down-projection kernels, the three gradient kernels (r <= 16, <= 32,
# > 32), both dX tiles, split-K and whole-tile schedules, ragged tails
SHAPES = [
    (1, 64, 64, 8, 16.0, 0.05),
    (16, 256, 256, 8, 16.0, 0.05),
    (4, 256, 2048, 64, 16.0, 0.05),      # few tokens: x staged in LDS, 4 A splits
    (29, 320, 1024, 32, 64.0, 0.1),      # few tokens: x in registers, ragged M
    (13, 192, 4096, 16, 32.0, 0.3),      # few tokens: x by DMA ring, 8 A splits
    (300, 320, 448, 16, 32.0, 0.05),
    (257, 512, 320, 24, 48.0, 0.1),
    (513, 384, 256, 64, 16.0, 0.05),
    (33, 192, 1024, 128, 32.0, 0.3),
    (600, 256, 512, 256, 8.0, 0.05),
    (1024, 1024, 768, 16, 32.0, 0.05),
    (200, 4096, 512, 32, 64.0, 0.05),
    (1000, 4096, 1024, 64, 16.0, 0.05),  # split down-projections, 4 token tiles
    (2100, 8192, 256, 32, 64.0, 0.1),    # dy.B split, 8 token tiles
    (100, 28672, 128, 64, 16.0, 0.1),    # the gradient kernel's 128-column tiles
]


def _case(M, N, K, r, alpha, p, seed=19):
    L = workloads.layer(M, N, K, r, alpha, seed=seed, outlier_frac=0.001)
    keep = workloads.keep_mask(seed, 50, M, K, p)
    return L, keep


def _ids(shapes):
    return [str(s) for s in shapes]


@pytest.mark.parametrize("shape", SHAPES, ids=_ids(SHAPES))
def test_dropout_forward_parity(cuda, shape):
    import torch
    M, N, K, r, alpha, p = shape
    print(f"dropout fwd {shape}", flush=True)
    L, keep = _case(*shape)
    ol = OracleLayer(L.w)
    y = q.linear_fwd_dropout(ol.to_device(), dev(L.x_bits), dev(L.A_bits), dev(L.B_bits), alpha,
                             dev(workloads.pack_keep(keep)), p)
    torch.cuda.synchronize()
    ref = oracle.lora_linear_fwd(L.f32("x"), ol.w_deq, L.f32("A"), L.f32("B"), alpha,
                                 keep=keep, p=p)
    check_close_bf16("y", bf16_values(host(y)), ref)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids(SHAPES))
def test_dropout_backward_parity(cuda, shape):
    import torch
    M, N, K, r, alpha, p = shape
    print(f"dropout bwd {shape}", flush=True)
    L, keep = _case(*shape)
    ol = OracleLayer(L.w)
    dx, dA, dB = q.linear_bwd_dropout(ol.to_device(), dev(L.x_bits), dev(L.dy_bits),
                                      dev(L.A_bits), dev(L.B_bits), alpha,
                                      dev(workloads.pack_keep(keep)), p)
    torch.cuda.synchronize()
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                           L.f32("B"), alpha, keep=keep, p=p)
    check_close_bf16("dX", bf16_values(host(dx)), rdx)
    check_close("dA", host(dA), rdA)
    check_close("dB", host(dB), rdB)


@pytest.mark.parametrize("shape", [(300, 320, 448, 16, 32.0), (600, 256, 512, 64, 16.0),
                                   (40, 192, 1024, 24, 48.0)],
                         ids=["r16", "r64_tile256", "r24_small"])
def test_dropout_zero_base_isolates_the_masked_adapter(cuda, shape):
    """W = 0: y and dX are the dropped adapter terms alone, at their own
    scale (the mask on dX's adapter term is otherwise hidden by the base)."""
    import torch
    M, N, K, r, alpha = shape
    p = 0.2
    L, keep = _case(M, N, K, r, alpha, p)
    L.w_override = lambda: np.zeros((N, K), dtype=np.float32)
    ol = OracleLayer(L.w)
    pw, kp = ol.to_device(), dev(workloads.pack_keep(keep))
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    y = q.linear_fwd_dropout(pw, x, A, B, alpha, kp, p)
    dx, dA, dB = q.linear_bwd_dropout(pw, x, dy, A, B, alpha, kp, p)
    torch.cuda.synchronize()
    ry = oracle.lora_linear_fwd(L.f32("x"), ol.w_deq, L.f32("A"), L.f32("B"), alpha,
                                keep=keep, p=p)
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                           L.f32("B"), alpha, keep=keep, p=p)
    check_close("y(W=0)", bf16_values(host(y)), ry)
    check_close("dX(W=0)", bf16_values(host(dx)), rdx)
    check_close("dA(W=0)", host(dA), rdA)
    check_close("dB(W=0)", host(dB), rdB)
    # dropped positions of dX carry nothing at all
    assert np.all(bf16_values(host(dx))[keep == 0] == 0)


@pytest.mark.parametrize("M", [16, 40, 600])
def test_nothing_kept_is_the_base_alone(cuda, M):
    import torch
    N, K, r, alpha = 256, 512, 16, 32.0
    L, _ = _case(M, N, K, r, alpha, 0.05)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    kp = dev(np.zeros((M, K // 8), dtype=np.uint8))
    y = q.linear_fwd_dropout(pw, x, A, B, alpha, kp, 0.05)
    dx, dA, dB = q.linear_bwd_dropout(pw, x, dy, A, B, alpha, kp, 0.05)
    y0 = q.linear_fwd(pw, x, None, None, alpha)
    dx0, _, _ = q.linear_bwd(pw, None, dy, None, None, alpha)
    torch.cuda.synchronize()
    # (few tokens: the adapter epilogue adds scale * 0 to the same sums)
    assert np.array_equal(host(y), host(y0))
    assert np.array_equal(host(dx), host(dx0))
    assert np.all(host(dA) == 0) and np.all(host(dB) == 0)


@pytest.mark.parametrize("M", [16, 300])
def test_everything_kept_at_p0_is_the_plain_layer(cuda, M):
    import torch
    N, K, r, alpha = 320, 448, 16, 32.0
    L, _ = _case(M, N, K, r, alpha, 0.0)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    kp = dev(np.full((M, K // 8), 0xFF, dtype=np.uint8))
    y = q.linear_fwd_dropout(pw, x, A, B, alpha, kp, 0.0)
    y0 = q.linear_fwd(pw, x, A, B, alpha)
    _, dA, dB = q.linear_bwd_dropout(pw, x, dy, A, B, alpha, kp, 0.0)
    _, dA0, dB0 = q.linear_bwd(pw, x, dy, A, B, alpha)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), host(y0))
    assert np.array_equal(host(dA), host(dA0))
    assert np.array_equal(host(dB), host(dB0))
