"""The allocation-free forward, qlora_linear_fwd_noalloc, against the forward
with a caller workspace, qlora_linear_fwd, through the C ABI.  Both run the
same kernels on the same inputs, so y must be bit-identical.  Each sequence
makes two allocation-free calls in a row on one GPU, the second on a
smaller input: the static scratch then holds the first call's contents when
the second runs.  y sits between guard bytes, and the device's free memory
must not drop across the two calls."""

import numpy as np
import pytest

import bit_quantized_lora_03_amd as q
from bit_quantized_lora_03_amd import workloads
from tests.gpu_util import Guarded, dev, host

pytestmark = pytest.mark.gpu

SEQUENCES = {
    # tiled GEMM with 2-way split partials and the adapter products, then the
    # few-token path with its adapter partial planes
    "q_proj_then_decode": [(512, 4096, 4096, 16, 32.0), (16, 2048, 2048, 64, 16.0)],
    # the 65B-class layer (tail-split and down-projection partials, 54 MiB
    # of scratch), then a ragged small layer on the tiled path
    "up65b_then_ragged": [(4096, 22016, 8192, 64, 16.0), (300, 320, 448, 16, 32.0)],
    # the largest workload need (66.25 MiB), then a base-only ragged call
    "mlp_down_then_base_only": [(2048, 4096, 11008, 16, 32.0), (70, 448, 640, 0, 1.0)],
    # weights in the mean-centred scale format: the tiled path, then the
    # few-token path
    "centred_tiled_then_decode": [(512, 4096, 4096, 16, 32.0), (8, 1024, 2048, 32, 64.0)],
}
CENTRED = {"centred_tiled_then_decode"}


def _setup(shape, seed, centred=False):
    import torch
    M, N, K, r, alpha = shape
    L = workloads.layer(M, N, K, r, alpha, seed=seed, outlier_frac=0.001)
    pw = (q.quantize_weight_centred if centred else q.quantize_weight)(dev(L.w))
    x = dev(L.x_bits)
    A = dev(L.A_bits) if r else None
    B = dev(L.B_bits) if r else None
    y = Guarded((M, N), torch.int16)
    return L, pw, x, A, B, y


@pytest.mark.parametrize("name", list(SEQUENCES))
def test_noalloc_forward_equals_workspace_forward(cuda, name):
    import torch
    calls = [_setup(shape, 70 + i, name in CENTRED) for i, shape in enumerate(SEQUENCES[name])]
    # the references first: they also load every kernel the calls use (the
    # runtime reserves memory for a kernel's code on its first launch)
    refs = [host(q.linear_fwd(pw, x, A, B, L.alpha)) for L, pw, x, A, B, _ in calls]
    # a first allocation-free call on this GPU that uses the scratch
    Lw, pww, xw, Aw, Bw, yw = _setup((40, 256, 256, 8, 16.0), 69)
    q.linear_fwd_noalloc(pww, xw, Aw, Bw, Lw.alpha, y=yw.t)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    # two allocation-free calls in a row, the second on a smaller input
    for i, (L, pw, x, A, B, y) in enumerate(calls):
        print(f"{name}: allocation-free call {i}: M={L.M} N={L.N} K={L.K} r={L.r}", flush=True)
        q.linear_fwd_noalloc(pw, x, A, B, L.alpha, y=y.t)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    for i, ((L, pw, x, A, B, y), want) in enumerate(zip(calls, refs)):
        y.check(f"y of call {i}")
        got = host(y.t)
        print(f"  call {i}: {np.count_nonzero(got != want)} of {got.size} elements differ",
              flush=True)
        assert np.array_equal(got, want), f"{name}: call {i} differs from the workspace call"
    # the two calls reserved no device memory
    assert free0 - free1 < (1 << 20), (free0, free1)
