"""Fused RMSNorm + per-token int8 quantization on the GPU against the oracle.

Bar: codes, zero points and fp32 scales bit-exact.  Both sides take every
step that decides a code in the same precision (the mean square as the
correctly rounded fp64 sum of the exact squares, rounded once to fp32, then
IEEE fp32 steps in a fixed order).  The device sums with an error-free
transformation (a double-fp64 running sum), which gives the correctly rounded
sum in any order unless the exact sum lies within about n^2 * 2^-106 of an
fp64 rounding boundary; the rows built to sit on and next to an fp32 boundary
of the mean square (tests/rmsnorm_rows.py) check exactly that case.
"""

import numpy as np
import pytest
import torch

import quantized_linear_layers_amd as ql
import workloads as wl
from oracle import rmsnorm as orn
from oracle import w8a8 as ow8

pytestmark = pytest.mark.gpu
TOL = 1e-2


def check(X, gamma, eps, symmetric=False):
    """X [M, K] and gamma [K] CPU 16-bit tensors."""
    Aq, s_a, azp = ql.i8_rmsnorm_quant_per_token(X.cuda(), gamma.cuda(), eps, symmetric=symmetric)
    torch.cuda.synchronize()
    Xf, gf = wl.as_f64(X), wl.as_f64(gamma)
    if symmetric:
        Aq_o, s_o = orn.rmsnorm_quant_per_token(Xf, gf, eps, asym=False)
        assert azp is None
    else:
        Aq_o, s_o, azp_o = orn.rmsnorm_quant_per_token(Xf, gf, eps)
        assert np.array_equal(azp.cpu().numpy(), azp_o)
    assert np.array_equal(s_a.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(Aq.cpu().numpy(), Aq_o)
    return Aq, s_a, azp


def rows(r, M, K, dtype, scale=1.0, mean=0.0):
    return torch.from_numpy((r.standard_normal((M, K)) * scale + mean).astype(np.float32)).to(dtype)


# ---------------------------------------------------------------- the W8A8 workload's activations

@pytest.mark.parametrize("symmetric", [False, True])
def test_w8a8_workload_rows(symmetric):
    w = wl.WORKLOADS["w8a8_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    check(wl.activations(w, M, K, N), wl.norm_weight(w, K), 1e-5, symmetric)


def test_fused_front_feeds_the_w8a8_gemm():
    """RMSNorm + quant, then i8_gemm_scaled, against the oracle's RMSNorm,
    quantization and exact integer product (the whole W8A8 path with the
    norm in front)."""
    w = wl.WORKLOADS["w8a8_prefill"]
    M, K, N = 256, 4096, 1024
    X = wl.activations(w, M, K, N)
    gamma = wl.norm_weight(w, K)
    Bq, s_b = ow8.quant_weight_per_channel_sym(wl.weight(w, K, N))
    adj = ow8.azp_adj(Bq)
    bias = wl.bias(w, N)
    Aq, s_a, azp = check(X, gamma, 1e-5)
    out = ql.i8_gemm_scaled(Aq, torch.from_numpy(Bq).cuda(), s_a, torch.from_numpy(s_b).cuda(), azp,
                            torch.from_numpy(adj).cuda(), bias.cuda())
    torch.cuda.synchronize()
    Aq_o, s_o, azp_o = orn.rmsnorm_quant_per_token(wl.as_f64(X), wl.as_f64(gamma), 1e-5)
    _, out64 = ow8.w8a8_linear(Aq_o, Bq, s_o, s_b, azp_o, adj, wl.as_f64(bias))
    e = float(np.abs(wl.as_f64(out.cpu()) - out64).max() / np.abs(out64).max())
    assert e <= TOL, f"relative error {e:.3e}"
    # and the quantized path stays close to the unquantized normalized layer
    y64 = orn.rms_norm64(wl.as_f64(X), wl.as_f64(gamma), 1e-5)
    ref = y64 @ (Bq.astype(np.float64) * s_b[:, None].astype(np.float64)).T + wl.as_f64(bias)
    assert float(np.abs(out64 - ref).max() / np.abs(ref).max()) < 2e-2


# ---------------------------------------------------------------- shapes and edges

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("K", [8, 24, 2056, 4104, 16384, 20480])
@pytest.mark.parametrize("M", [1, 3, 17])
def test_ragged(M, K, dtype):
    r = np.random.default_rng(M * 100003 + K)
    X = rows(r, M, K, dtype, 2.0, 0.1)
    gamma = rows(r, 1, K, dtype, 0.3, 1.0)[0]
    check(X, gamma, 1e-6)
    check(X, gamma, 1e-6, symmetric=True)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_edge_rows(dtype):
    K = 256
    r = np.random.default_rng(7)
    big = 60000.0 if dtype == torch.float16 else 1.0e19     # the mean square stays below the fp32 maximum
    X = torch.stack([
        torch.zeros(K),                                     # all zero: y = 0, the scale floor
        torch.full((K,), 3.0),                              # constant row
        torch.full((K,), -big),                             # at the top of the dtype's range
        torch.from_numpy(r.standard_normal(K).astype(np.float32) * 1e-6),   # tiny values
        torch.from_numpy(np.where(np.arange(K) == 5, 100.0, 1e-3).astype(np.float32)),  # one spike
    ]).to(dtype)
    gamma = rows(r, 1, K, dtype, 0.5, 1.0)[0]
    for eps in (1e-6, 1.0):
        check(X, gamma, eps)
        check(X, gamma, eps, symmetric=True)


@pytest.mark.parametrize("row", ["tie", "straddle_first", "straddle_second"])
def test_mean_square_at_an_fp32_boundary(row):
    """Rows whose mean square is an fp32 midpoint (ties to even) or lies just
    above one by less than the fp64 rounding of the sum (rounds up): the tiny
    squares sit in the first 8-value piece of 96 threads' rows, or in their
    second piece after a first piece of large values."""
    from tests import rmsnorm_rows as rr
    x = {"tie": lambda: rr.tie_row()[0],
         "straddle_first": lambda: rr.straddle_row()[0],
         "straddle_second": lambda: rr.straddle_row(tiny_start=2048, big_from=0)[0]}[row]()
    X = torch.from_numpy(np.stack([x, x[::-1].copy()]).astype(np.float32)).to(torch.float16)
    assert np.array_equal(wl.as_f64(X)[0], x)               # the row is exact in fp16
    gamma = torch.ones(rr.K, dtype=torch.float16)
    check(X, gamma, 1e-6)
    check(X, gamma, 1e-6, symmetric=True)


def test_gamma_signs_and_zeros():
    K = 512
    r = np.random.default_rng(8)
    X = rows(r, 4, K, torch.float16)
    g = r.standard_normal(K).astype(np.float32)
    g[::7] = 0.0
    check(X, torch.from_numpy(g).to(torch.float16), 1e-5)


def test_repeat_calls_identical():
    w = wl.WORKLOADS["w8a8_prefill"]
    X = wl.activations(w, 64, 4096, 4096).cuda()
    gamma = wl.norm_weight(w, 4096).cuda()
    a = ql.i8_rmsnorm_quant_per_token(X, gamma, 1e-5)
    b = ql.i8_rmsnorm_quant_per_token(X, gamma, 1e-5)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_empty_batch():
    gamma = torch.ones(64, dtype=torch.float16, device="cuda")
    Aq, s_a, azp = ql.i8_rmsnorm_quant_per_token(torch.empty((0, 64), dtype=torch.float16, device="cuda"), gamma,
                                                 1e-5)
    assert Aq.shape == (0, 64) and s_a.shape == (0,) and azp.shape == (0,)
