"""q4_gemm_no_alloc (the library's static scratch instead of a workspace)
through the C ABI: two calls in a row, the second on a smaller layer, each
bit-identical to q4_gemm with a caller-owned workspace (same plan, same
kernels), and both within the W4A16 parity bar against the oracle."""

import numpy as np
import pytest
import torch

import quantized_linear_layers_amd as ql
import workloads as wl
from oracle import w4a16 as ow4

pytestmark = pytest.mark.gpu


def _layer(w, M, K, N):
    W = wl.weight(w, K, N)
    wq, s, z = ql.q4_quantize_host(torch.from_numpy(W))
    return W, ql.q4_pack(wq, s, z, N, K, device="cuda"), wl.activations(w, M, K, N)


def test_no_alloc_matches_workspace_entry_point():
    w = wl.WORKLOADS["mid_m_7b"]
    for (M, K, N) in ((128, 11008, 4096), (32, 11008, 4096)):      # the second call is smaller
        assert ql.q4_gemm_plan(M, N, K)[2] > 1                       # the plan uses the scratch
        W, blob, X = _layer(w, M, K, N)
        Xd = X.cuda()
        Y0 = ql.q4_gemm(Xd, blob, N)                                 # caller-owned workspace
        Y1 = torch.full((M, N), float("nan"), dtype=X.dtype, device="cuda")
        ql.launcher("q4_gemm_no_alloc", Xd, X.dtype, M, K, N, blob, blob.numel(), 128, Y1)()
        torch.cuda.synchronize()
        assert torch.equal(Y0, Y1)
        q, s, z = ow4.quantize_w4(W)
        Y64 = ow4.w4a16_linear(wl.as_f64(X), q, s, z)
        Yd = wl.as_f64(Y1.cpu())
        assert np.abs(Yd - Y64).max() / np.abs(Y64).max() <= 1e-2


def test_no_alloc_without_scratch_and_binding():
    """A decode-sized layer (no split, the scratch untouched) and the binding's
    wrapper, which takes a caller-given output."""
    w = wl.WORKLOADS["decode_7b"]
    W, blob, X = _layer(w, 4, 4096, 4096)
    Xd = X.cuda()
    Y = torch.empty((4, 4096), dtype=X.dtype, device="cuda")
    ql.q4_gemm_no_alloc(Xd, blob, 4096, Y)
    torch.cuda.synchronize()
    assert torch.equal(Y, ql.q4_gemm(Xd, blob, 4096))
