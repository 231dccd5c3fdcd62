"""Seeded random shapes for the device entry points, against the oracle.

The fixed-shape tests pin the workloads and the edges someone thought of
(ragged tails, tile and plan boundaries, extreme codes).  This sweep draws
further shapes from a seeded generator, so that combinations nobody listed
(a plan, a tile shape, a K split and ragged M, N and K at once) are checked
as well; the few-token W8A8 shapes (up to 64 tokens) are drawn separately,
so that the kernel that serves them gets its own sample.  Every case runs the
same checks as the fixed-shape tests of its entry point: W4A16 within the
1e-2 gate and the element-wise rounding bound, the int8 accumulator
bit-exact and its fp16/bf16 output within the epilogue bound, FP8 within the
gate, quantized codes and scales bit-exact.  Sizes are kept where the
oracle's fp64 products take about a second.
"""

import numpy as np
import pytest
import torch

from oracle import fp8 as of8
from oracle import w8a8 as ow8
from tests import test_gpu_fp8 as t8f
from tests import test_gpu_w4a16 as t4
from tests import test_gpu_w8a8 as t8

pytestmark = pytest.mark.gpu


def _log_uniform(r, lo, hi):
    return int(np.exp(r.uniform(np.log(lo), np.log(hi + 1))))


def _w4_cases(n=30):
    r = np.random.default_rng(2024)
    cases = []
    for i in range(n):
        M = int(r.integers(1, 17)) if i % 3 == 0 else _log_uniform(r, 17, 400)   # decode kernel / GEMM plans
        K = 128 * int(r.integers(1, 25))
        N = _log_uniform(r, 1, 1500) if i % 2 else int(r.integers(200, 3001))
        cases.append((i, M, K, N))
    return cases


@pytest.mark.parametrize("case,M,K,N", _w4_cases())
def test_w4a16_random_shape(case, M, K, N):
    """q4_gemm on a random layer; every fourth case without a workspace (the
    plan that does not split K), the others with one."""
    r = np.random.default_rng(10_000 + case)
    dtype = torch.bfloat16 if case % 2 else torch.float16
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    t4.check(W, X, workspace=case % 4 != 3)


def _w8_shape(r, large):
    if large:                                # grids of 256 x 128 tiles past half the compute units
        M, N = int(r.integers(600, 2601)), int(r.integers(900, 2201))
    else:
        M, N = _log_uniform(r, 1, 2600), _log_uniform(r, 1, 2200)
    K = 16 * int(r.integers(1, 200))
    while M * N * K > 2e9:                   # keep the oracle's product to about a second
        K = max(16, (K // 32) * 16)
    return M, N, K


def _w8_cases(n=24, seed=4048):
    r = np.random.default_rng(seed)
    return [(i,) + _w8_shape(r, i % 2 == 0) for i in range(n)]


@pytest.mark.parametrize("case,M,N,K", _w8_cases())
def test_int8_gemm_random_shape(case, M, N, K):
    """i8_gemm_scaled with the epilogue variant chosen by the case: per-token
    zero points or none, per-tensor or per-row/column scales, bias or not,
    fp16 or bf16 output."""
    r = np.random.default_rng(20_000 + case)
    Aq, s_a, azp, Bq, s_b = t8._operands(M, N, K, 30_000 + case)
    adj = ow8.azp_adj(Bq)
    out_dtype = torch.bfloat16 if case % 2 else torch.float16
    bias = None
    if case % 3 != 2:
        bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).to(out_dtype)
    if case % 4 == 1:
        s_a, s_b = s_a[:1], s_b[:1]
    if case % 5 == 4:
        azp, adj = None, None                 # symmetric activations
    t8.check_gemm(Aq, Bq, s_a, s_b, azp, adj, bias, out_dtype=out_dtype)


@pytest.mark.parametrize("case,M,N,K", _w8_cases(16, seed=5055))
def test_fp8_gemm_random_shape(case, M, N, K):
    r = np.random.default_rng(40_000 + case)
    Aq, s_a = of8.quant_per_token_fp8((r.standard_normal((M, K)) + 0.3).astype(np.float32))
    Bq, s_b = of8.quant_weight_per_channel_fp8((r.standard_normal((N, K)) * 0.02).astype(np.float32))
    out_dtype = torch.bfloat16 if case % 2 else torch.float16
    bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).to(out_dtype) if case % 3 else None
    t8f.check_gemm(Aq, Bq, s_a, s_b, bias, out_dtype=out_dtype)


def _few_token_cases(n, seed):
    """Shapes for the few-token W8A8 kernel: up to 64 tokens, N drawn so that
    M N stays within 2^19 (the range that kernel serves above 16 tokens)."""
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = _log_uniform(r, 1, 64)
        N = _log_uniform(r, 1, max(1, min(20000, (1 << 19) // M)))
        K = 16 * int(r.integers(1, 300))
        cases.append((i, M, N, K))
    return cases


@pytest.mark.parametrize("case,M,N,K", _few_token_cases(16, 7070))
def test_int8_gemm_few_tokens_random_shape(case, M, N, K):
    r = np.random.default_rng(60_000 + case)
    Aq, s_a, azp, Bq, s_b = t8._operands(M, N, K, 70_000 + case)
    out_dtype = torch.bfloat16 if case % 2 else torch.float16
    bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).to(out_dtype) if case % 3 else None
    if case % 4 == 3:
        s_a, s_b = s_a[:1], s_b[:1]
    t8.check_gemm(Aq, Bq, s_a, s_b, azp, ow8.azp_adj(Bq), bias, out_dtype=out_dtype)


@pytest.mark.parametrize("case,M,N,K", _few_token_cases(8, 8080))
def test_fp8_gemm_few_tokens_random_shape(case, M, N, K):
    r = np.random.default_rng(80_000 + case)
    Aq, s_a = of8.quant_per_token_fp8((r.standard_normal((M, K)) + 0.3).astype(np.float32))
    Bq, s_b = of8.quant_weight_per_channel_fp8((r.standard_normal((N, K)) * 0.02).astype(np.float32))
    out_dtype = torch.bfloat16 if case % 2 else torch.float16
    bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).to(out_dtype) if case % 3 else None
    t8f.check_gemm(Aq, Bq, s_a, s_b, bias, out_dtype=out_dtype)


def _quant_cases(n=16):
    r = np.random.default_rng(6060)
    return [(i, _log_uniform(r, 1, 300), 8 * _log_uniform(r, 1, 2600)) for i in range(n)]


@pytest.mark.parametrize("case,M,K", _quant_cases())
def test_quant_random_shape(case, M, K):
    """Per-token int8 (asymmetric and symmetric) and FP8 quantization of random
    rows: codes, zero points and scales bit-exact."""
    r = np.random.default_rng(50_000 + case)
    dtype = torch.bfloat16 if case % 2 else torch.float16
    X = torch.from_numpy((r.standard_normal((M, K)) * 2 + 0.4).astype(np.float32)).to(dtype)
    t8.check_quant(X)
    t8.check_quant(X, symmetric=True)
    t8f.check_quant(X)


def test_random_cases_cover_the_plans():
    """The drawn shapes reach both W4A16 kernels and both int8 tile shapes."""
    ms = [c[1] for c in _w4_cases()]
    assert min(ms) <= 16 < max(ms)
    small = [2 * ((M + 255) // 256) * ((N + 127) // 128) <= 256 for _, M, N, _ in _w8_cases()]
    assert any(small) and not all(small)
    few = [M for _, M, N, _ in _few_token_cases(16, 7070)]
    assert min(few) <= 16 < max(few)
