"""GPU parity of the fused forward and backward passes against the fp64
oracle, through the C ABI.  The GEMMs are fed the oracle's packed weight,
so their parity does not depend on the GPU quantiser (tested separately).

Bar: max|T_gpu - T_oracle| <= 2e-2 * rms(T_oracle) for y, dX, dA, dB (for
the bf16 outputs y and dX, or their own rounding floor where one large
element puts that above 2e-2).
Exact cases: one-hot probes read back the decoded weight bit for bit.
"""

import numpy as np
import pytest

import oracle
import bit_quantized_lora_03_amd as q
from bit_quantized_lora_03_amd import workloads
from tests.gpu_util import (Guarded, OracleLayer, bf16_values, check_close, check_close_bf16, dev,
                            host)

pytestmark = pytest.mark.gpu

# (M, N, K, r, alpha): several tiles and ragged tails in every dimension the
# kernels tile (256-wide n/m/k tiles, 64-wide k/n steps, 2r adapter columns)
SHAPES = [
    (1, 64, 64, 8, 16.0),
    (16, 256, 256, 8, 16.0),
    (300, 320, 448, 16, 32.0),
    (257, 512, 320, 24, 48.0),
    (513, 384, 256, 64, 16.0),
    (33, 192, 1024, 128, 32.0),
    (5, 128, 192, 256, 8.0),
    (70, 448, 640, 0, 1.0),
    # the two adapter down-projections of the backward (over K and over N)
    # with very different reduction lengths: N >> K and N << K
    (200, 4096, 512, 32, 64.0),
    (96, 256, 4096, 16, 32.0),
    # the down-projection's token tiles and reduction splits: 8 tiles with
    # x.A^T split (dy.B not), 4 tiles with both split, 8 tiles with only
    # dy.B split (ragged token blocks in each)
    (2304, 320, 4096, 16, 32.0),
    (1000, 4096, 1024, 64, 16.0),
    (2100, 8192, 256, 32, 64.0),
]


def _layer(M, N, K, r, alpha, seed=11):
    return workloads.layer(M, N, K, r, alpha, seed=seed, outlier_frac=0.001)


def _run_fwd(L, ol, pw=None):
    """The forward with y and the workspace between guard bytes."""
    import torch
    pw = pw or ol.to_device()
    x = dev(L.x_bits)
    A = dev(L.A_bits) if L.r else None
    B = dev(L.B_bits) if L.r else None
    y = Guarded((L.M, L.N), torch.int16)
    ws = Guarded((max(1, q.workspace_bytes(0, L.M, L.N, L.K, L.r)),), torch.uint8)
    q.linear_fwd(pw, x, A, B, L.alpha, y=y.t, workspace=ws.t)
    torch.cuda.synchronize()
    y.check("y")
    ws.check("forward workspace")
    return bf16_values(host(y.t))


def _ref_fwd(L, ol, rows=None):
    xs = L.f32("x") if rows is None else L.f32("x")[rows]
    A = L.f32("A") if L.r else None
    B = L.f32("B") if L.r else None
    return oracle.lora_linear_fwd(xs, ol.w_deq, A, B, L.alpha)


def _run_bwd(L, ol, need_dx=True, accumulate=False, dA0=None, dB0=None):
    """The backward with dX, dA, dB and the workspace between guard bytes."""
    import torch
    pw = ol.to_device()
    x = dev(L.x_bits)
    dy = dev(L.dy_bits)
    A = dev(L.A_bits) if L.r else None
    B = dev(L.B_bits) if L.r else None
    gx = Guarded((L.M, L.K), torch.int16) if need_dx else None
    gA = gB = None
    if L.r:
        gA = Guarded((L.r, L.K), torch.float32, None if dA0 is None else dev(dA0.copy()))
        gB = Guarded((L.N, L.r), torch.float32, None if dB0 is None else dev(dB0.copy()))
    ws = Guarded((max(1, q.workspace_bytes(1, L.M, L.N, L.K, L.r)),), torch.uint8)
    dx, dA, dB = q.linear_bwd(pw, x, dy, A, B, L.alpha, need_dx=need_dx,
                              dA=gA.t if gA else None, dB=gB.t if gB else None,
                              accumulate=accumulate, workspace=ws.t,
                              dx=gx.t if gx else None)
    torch.cuda.synchronize()
    for g, name in ((gx, "dX"), (gA, "dA"), (gB, "dB"), (ws, "backward workspace")):
        if g is not None:
            g.check(name)
    return (bf16_values(host(dx)) if dx is not None else None,
            host(dA) if dA is not None else None, host(dB) if dB is not None else None)


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_forward_parity(cuda, shape):
    M, N, K, r, alpha = shape
    print(f"fwd {shape}", flush=True)
    L = _layer(*shape)
    ol = OracleLayer(L.w)
    check_close_bf16("y", _run_fwd(L, ol), _ref_fwd(L, ol))


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_backward_parity(cuda, shape):
    M, N, K, r, alpha = shape
    print(f"bwd {shape}", flush=True)
    L = _layer(*shape)
    ol = OracleLayer(L.w)
    dx, dA, dB = _run_bwd(L, ol)
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq,
                                           L.f32("A") if r else None,
                                           L.f32("B") if r else None, alpha)
    check_close_bf16("dX", dx, rdx)
    if r:
        check_close("dA", dA, rdA)
        check_close("dB", dB, rdB)


@pytest.mark.parametrize("shape", [(100, 28672, 128, 16, 32.0), (100, 28672, 128, 32, 64.0),
                                   (70, 27648, 1024, 64, 16.0)],
                         ids=["r16", "r32", "r64-two-jobs"])
def test_wide_gradient_tiles(cuda, shape):
    """Enough G columns for the gradient kernel's 128-column tiles (four
    waves, 256-byte runs per token row): 224 blocks, the dA job's first
    block after the dB job's last, ragged tokens; dX, dA and dB against the
    oracle, the accumulate mode on the last shape."""
    M, N, K, r, alpha = shape
    L = _layer(M, N, K, r, alpha)
    ol = OracleLayer(L.w)
    rng = np.random.default_rng(3)
    acc = r == 64
    dA0 = rng.standard_normal((r, K)).astype(np.float32) if acc else None
    dB0 = rng.standard_normal((N, r)).astype(np.float32) if acc else None
    dx, dA, dB = _run_bwd(L, ol, accumulate=acc, dA0=dA0, dB0=dB0)
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                           L.f32("B"), L.alpha)
    check_close_bf16("dX", dx, rdx)
    check_close("dA", dA.astype(np.float64) - (dA0 if acc else 0), rdA)
    check_close("dB", dB.astype(np.float64) - (dB0 if acc else 0), rdB)


def test_backward_accumulate_and_skip_dx(cuda):
    L = _layer(100, 256, 320, 16, 32.0)
    ol = OracleLayer(L.w)
    rng = np.random.default_rng(1)
    dA0 = rng.standard_normal((16, 320)).astype(np.float32)
    dB0 = rng.standard_normal((256, 16)).astype(np.float32)
    dx, dA, dB = _run_bwd(L, ol, need_dx=False, accumulate=True, dA0=dA0, dB0=dB0)
    assert dx is None
    _, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                         L.f32("B"), L.alpha)
    check_close("dA - dA0", dA.astype(np.float64) - dA0, rdA)
    check_close("dB - dB0", dB.astype(np.float64) - dB0, rdB)


@pytest.mark.parametrize("N,K,step", [(320, 448, 3), (4096, 4096, 517)],
                         ids=["tiled", "few-token"])
def test_one_hot_probes_are_bit_exact(cuda, N, K, step):
    """Base only, x = one-hot rows e_k: y[m, :] = W'[:, k_m] bit for bit (one
    exact bf16 product per output; at 4096 x 4096 with 8 rows, the few-token
    path over four chunks with x in registers).  dy = e_n: dX[m, :] =
    W'[n_m, :]."""
    import torch
    L = _layer(1, N, K, 0, 1.0)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    ks = np.arange(0, K, step)
    x = np.zeros((ks.size, K), dtype=np.uint16)
    x[np.arange(ks.size), ks] = 0x3F80                     # bf16 1.0
    y = host(q.linear_fwd(pw, dev(x), None, None, 1.0))
    ns = np.arange(0, N, 2 if N < 1024 else 263)
    dy = np.zeros((ns.size, N), dtype=np.uint16)
    dy[np.arange(ns.size), ns] = 0x3F80
    dx, _, _ = q.linear_bwd(pw, None, dev(dy), None, None, 1.0)
    dx = host(dx)
    torch.cuda.synchronize()
    wbits = oracle.dequant_nf4_bits(ol.packed, ol.q, ol.step, N * K).reshape(N, K)
    assert np.array_equal(y, wbits[:, ks].T)
    assert np.array_equal(dx, wbits[ns, :])


@pytest.mark.parametrize("shape", [
    (129, 256, 512, 16, 32.0),    # few outputs: 8 x 8 tiles, bf16 dot products
    (40, 192, 1024, 24, 48.0),    # ... three rank groups, ragged tokens
    (33, 256, 2048, 128, 16.0),   # ... sixteen rank groups
    (2304, 320, 448, 16, 32.0),   # more outputs: 16 x 16 MFMA tiles
    (600, 128, 384, 64, 16.0),    # ... four 16-column groups per block
    (2304, 320, 4096, 16, 32.0),  # 8 token tiles, x.A^T split 8 ways
    (1000, 4096, 1024, 64, 16.0), # 4 token tiles, both reductions split
    (2100, 8192, 256, 32, 64.0),  # 8 token tiles, dy.B split
], ids=[str(s) for s in [(129, 256, 512, 16), (40, 192, 1024, 24), (33, 256, 2048, 128),
                         (2304, 320, 448, 16), (600, 128, 384, 64), (2304, 320, 4096, 16),
                         (1000, 4096, 1024, 64), (2100, 8192, 256, 32)]])
def test_zero_base_isolates_the_adapter_path(cuda, shape):
    """W = 0: y and dX are the adapter terms alone (x.A^T and dy.B through
    both down-projection kernels), tested at their own scale, with dA, dB."""
    M, N, K, r, alpha = shape
    L = _layer(M, N, K, r, alpha)
    L.w_override = lambda: np.zeros((N, K), dtype=np.float32)
    ol = OracleLayer(L.w)
    assert np.all(ol.w_deq == 0)
    check_close("y(W=0)", _run_fwd(L, ol), _ref_fwd(L, ol))
    dx, dA, dB = _run_bwd(L, ol)
    rdx, rdA, rdB = oracle.lora_linear_bwd(L.f32("x"), L.f32("dy"), ol.w_deq, L.f32("A"),
                                           L.f32("B"), L.alpha)
    check_close("dX(W=0)", dx, rdx)
    check_close("dA(W=0)", dA, rdA)
    check_close("dB(W=0)", dB, rdB)


@pytest.mark.parametrize("shape", [(300, 320, 448, 16, 32.0), (13, 512, 4096, 64, 16.0)],
                         ids=["tiled", "few-tokens"])
def test_deterministic(cuda, shape):
    """Three runs of the same call give the same bits (every reduction has
    a fixed order, split partials included)."""
    import torch
    L = _layer(*shape)
    ol = OracleLayer(L.w)
    a = [_run_fwd(L, ol) for _ in range(3)]
    assert np.array_equal(a[0], a[1]) and np.array_equal(a[0], a[2])
    d = [_run_bwd(L, ol) for _ in range(3)]
    for run in d[1:]:
        for u, v in zip(d[0], run):
            assert np.array_equal(u, v)
    torch.cuda.synchronize()


def test_empty_token_batch(cuda):
    import torch
    L = _layer(1, 128, 128, 8, 16.0)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    x = torch.zeros((0, 128), dtype=torch.int16, device="cuda")
    y = q.linear_fwd(pw, x, dev(L.A_bits), dev(L.B_bits), 16.0)
    assert y.shape == (0, 128)
    dA0 = np.full((8, 128), 5.0, dtype=np.float32)
    dx, dA, dB = q.linear_bwd(pw, x, torch.zeros((0, 128), dtype=torch.int16, device="cuda"),
                              dev(L.A_bits), dev(L.B_bits), 16.0, dA=dev(dA0))
    torch.cuda.synchronize()
    assert np.all(host(dA) == 0) and np.all(host(dB) == 0)


@pytest.mark.parametrize("shape", [(300, 320, 448, 16, 32.0), (8, 256, 512, 64, 16.0),
                                   (8, 4096, 4096, 16, 16.0), (1000, 4096, 1024, 64, 16.0)],
                         ids=["main", "decode-x-in-lds", "decode-x-in-registers",
                              "split-down-projection"])
def test_graph_replay_matches_eager(cuda, shape):
    """The whole fwd + bwd captured in one HIP graph: every replay (with
    eager work and synchronisations between replays) equals the eager run
    bit for bit."""
    import torch
    L = _layer(*shape)
    ol = OracleLayer(L.w)
    pw = ol.to_device()
    x, dy, A, B = dev(L.x_bits), dev(L.dy_bits), dev(L.A_bits), dev(L.B_bits)
    y0 = q.linear_fwd(pw, x, A, B, L.alpha)
    dx0, dA0, dB0 = q.linear_bwd(pw, x, dy, A, B, L.alpha)
    torch.cuda.synchronize()
    eager = [host(t) for t in (y0, dx0, dA0, dB0)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.linear_fwd(pw, x, A, B, L.alpha)
        q.linear_bwd(pw, x, dy, A, B, L.alpha)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = q.linear_fwd(pw, x, A, B, L.alpha)
        dx, dA, dB = q.linear_bwd(pw, x, dy, A, B, L.alpha)
    for rep in range(4):
        for t in (y, dx, dA, dB):
            t.zero_()                                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in (y, dx, dA, dB)]
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), f"replay {rep} differs from eager"
