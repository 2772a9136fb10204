"""GPU parity of LoRA dropout with the keep bits drawn by the library
(Philox4x32-10 from (seed, offset), no mask argument), through the C ABI.

* The drawn mask (qlora_dropout_keep_mask) is bit-exact against the
  oracle's generator, at ragged sizes, large seeds and offsets, and the
  65B-class activation [4096, 8192].
* The layer with drawn bits equals the layer with the same bits passed in
  (qlora_linear_*_dropout with p = t / 65536) bit for bit: the same
  arithmetic on the same bits, so a wrong draw or a wrong stored mask in
  the backward shows as a difference.
* The layer is within 2e-2 rms of the fp64 oracle fed the oracle's mask
  and realised p (the output's own bf16 rounding floor where larger).
Outputs sit between guard bytes.
"""

import numpy as np
import pytest

import oracle
import bit_quantized_lora_03_amd as q
from bit_quantized_lora_03_amd import workloads
from tests.gpu_util import (Guarded, OracleLayer, bf16_values, check_close, check_close_bf16,
                            dev, host)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,p,seed,offset", [
    (1, 8, 0.05, 0, 0),
    (3, 200, 0.05, 1, 2),
    (37, 1024, 0.3, (1 << 64) - 1, (1 << 63) + 11),
    (512, 4096, 0.05, 0x1234_5678_9ABC_DEF0, 7),
    (4096, 8192, 0.05, 4, 1),                 # the 65B-class layer's x
])
def test_drawn_mask_is_bit_exact(cuda, M, K, p, seed, offset):
    import torch
    print(f"mask M={M} K={K} p={p} seed={seed} offset={offset}", flush=True)
    g = Guarded((M, K // 8), torch.uint8)
    q.dropout_keep_mask(M, K, p, seed, offset, keep=g.t)
    g.check("keep mask")
    got = host(g.t)
    want = workloads.pack_keep(oracle.dropout_keep_philox(M, K, p, seed, offset))
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} bytes differ"


# (M, N, K, r, alpha, p): the small down-projection kernel (M r <= 16384)
# and the MFMA one, one and several rank chunks (the first chunk's blocks
# store the drawn bytes), the three gradient kernels, ragged tails
SHAPES = [
    (1, 64, 64, 8, 16.0, 0.05),
    (16, 512, 4096, 64, 16.0, 0.05),     # few tokens: x by DMA ring, 8 A splits
    (29, 320, 1024, 32, 64.0, 0.1),      # few tokens: x in registers, ragged M
    (300, 320, 448, 16, 32.0, 0.05),
    (257, 512, 320, 24, 48.0, 0.1),
    (513, 384, 256, 64, 16.0, 0.05),
    (600, 256, 512, 128, 8.0, 0.05),     # MFMA kernel, two rank chunks of 64
    (33, 192, 1024, 256, 32.0, 0.3),     # small kernel, 32 rank groups
    (1024, 1024, 768, 16, 32.0, 0.05),
    (1000, 4096, 1024, 64, 16.0, 0.05),  # split down-projections, 4 token tiles
    (2304, 320, 4096, 16, 32.0, 0.05),   # 8 token tiles, x.A^T split 8 ways
]


def _layer(M, N, K, r, alpha, seed=23):
    return workloads.layer(M, N, K, r, alpha, seed=seed, outlier_frac=0.001)


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_drawn_dropout_equals_passed_mask_and_oracle(cuda, shape):
    import torch
    M, N, K, r, alpha, p = shape
    seed, offset = 977 + M, 3 * r
    print(f"drawn dropout {shape} seed={seed} offset={offset}", flush=True)
    L = _layer(M, N, K, r, alpha)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    p_real = oracle.realised_dropout(p)

    # drawn in the kernels
    y = Guarded((M, N), torch.int16)
    q.linear_fwd_dropout_rng(pw, x, A, B, alpha, p, seed, offset, y=y.t)
    gx = Guarded((M, K), torch.int16)
    gA = Guarded((r, K), torch.float32)
    gB = Guarded((N, r), torch.float32)
    ws = Guarded((q.workspace_bytes(9, M, N, K, r),), torch.uint8)
    q.linear_bwd_dropout_rng(pw, x, dy, A, B, alpha, p, seed, offset, dA=gA.t, dB=gB.t, dx=gx.t,
                             workspace=ws.t)
    torch.cuda.synchronize()
    for g, name in ((y, "y"), (gx, "dX"), (gA, "dA"), (gB, "dB"), (ws, "workspace")):
        g.check(name)

    # the same bits passed in
    keep_d = q.dropout_keep_mask(M, K, p, seed, offset)
    y2 = q.linear_fwd_dropout(pw, x, A, B, alpha, keep_d, p_real)
    dx2, dA2, dB2 = q.linear_bwd_dropout(pw, x, dy, A, B, alpha, keep_d, p_real)
    torch.cuda.synchronize()
    for name, a, b in (("y", y.t, y2), ("dX", gx.t, dx2), ("dA", gA.t, dA2), ("dB", gB.t, dB2)):
        ha, hb = host(a), host(b)
        assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8)), \
            f"{name}: drawn and passed-in masks differ ({np.count_nonzero(ha != hb)} elements)"

    # the oracle with its own draws
    keep = oracle.dropout_keep_philox(M, K, p, seed, offset)
    ry = oracle.lora_linear_fwd(L.f32("x"), ol.w_deq, L.f32("A"), L.f32("B"), alpha,
                                keep=keep, p=p_real)
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                           L.f32("B"), alpha, keep=keep, p=p_real)
    check_close_bf16("y", bf16_values(host(y.t)), ry)
    check_close_bf16("dX", bf16_values(host(gx.t)), rdx)
    check_close("dA", host(gA.t), rdA)
    check_close("dB", host(gB.t), rdB)


def test_drawn_dropout_65b_layer(cuda):
    """The 65B-class layer (M 4096, 22016 x 8192, r 64) with p = 0.05: the
    drawn layer equals the passed-in mask bit for bit (y, dX, dA, dB)."""
    import torch
    L = workloads.layer_65b()
    M, N, K, r, alpha = L.M, L.N, L.K, L.r, L.alpha
    p, seed, offset = 0.05, 4, 1
    pw = q.quantize_weight(dev(L.w))
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    y = q.linear_fwd_dropout_rng(pw, x, A, B, alpha, p, seed, offset)
    dx, dA, dB = q.linear_bwd_dropout_rng(pw, x, dy, A, B, alpha, p, seed, offset)
    keep_d = q.dropout_keep_mask(M, K, p, seed, offset)
    p_real = oracle.realised_dropout(p)
    y2 = q.linear_fwd_dropout(pw, x, A, B, alpha, keep_d, p_real)
    dx2, dA2, dB2 = q.linear_bwd_dropout(pw, x, dy, A, B, alpha, keep_d, p_real)
    torch.cuda.synchronize()
    for name, a, b in (("y", y, y2), ("dX", dx, dx2), ("dA", dA, dA2), ("dB", dB, dB2)):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("M", [16, 300])
def test_no_dropout_limit_equals_the_plain_layer(cuda, M):
    """p = 0 keeps every element: the drawn forward equals the layer without
    dropout bit for bit (same kernels, same scale).  The backward's
    masked dX kernel adds the adapter rows before the base (so its rounding
    order differs): dX, dA and dB are checked against the oracle without
    dropout."""
    import torch
    N, K, r, alpha = 320, 448, 16, 32.0
    L = _layer(M, N, K, r, alpha)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    y = q.linear_fwd_dropout_rng(pw, x, A, B, alpha, 0.0, 5, 5)
    dx, dA, dB = q.linear_bwd_dropout_rng(pw, x, dy, A, B, alpha, 0.0, 5, 5)
    y0 = q.linear_fwd(pw, x, A, B, alpha)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                           L.f32("B"), alpha)
    check_close("dX", bf16_values(host(dx)), rdx)
    check_close("dA", host(dA), rdA)
    check_close("dB", host(dB), rdB)
