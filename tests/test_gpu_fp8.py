"""W8A8 with FP8 (E4M3) codes: parity on the GPU.

f8_quant_per_token: codes and fp32 scales bit-exact with the oracle (both
divide in IEEE fp32 and round once to E4M3, nearest even, saturating).
f8_gemm_scaled: output within max|out - out64| / max|out64| <= 1e-2 of the
oracle's exact FP8 product and fp64 epilogue.  The GEMM's inputs are the
oracle's own quantized operands.
"""

import numpy as np
import pytest
import torch

import quantized_linear_layers_amd as ql
import workloads as wl
from oracle import fp8 as of8

pytestmark = pytest.mark.gpu
TOL = 1e-2


def cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_quant(X):
    Aq, s_a = ql.f8_quant_per_token(X.cuda())
    torch.cuda.synchronize()
    Aq_o, s_o = of8.quant_per_token_fp8(wl.as_f64(X).astype(np.float32))
    assert np.array_equal(s_a.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(Aq.cpu().numpy(), Aq_o)


def check_gemm(Aq, Bq, s_a, s_b, bias=None, out_dtype=torch.float16, tol=TOL):
    out = ql.f8_gemm_scaled(cu(Aq), cu(Bq), cu(s_a), cu(s_b), None if bias is None else bias.cuda(),
                            out_dtype=out_dtype)
    torch.cuda.synchronize()
    out64 = of8.fp8_linear(Aq, Bq, s_a, s_b, None if bias is None else wl.as_f64(bias))
    od = wl.as_f64(out.cpu())
    e = float(np.abs(od - out64).max() / np.abs(out64).max())
    assert e <= tol, f"relative error {e:.3e}"


def _codes(r, shape):
    """Random E4M3 codes over the whole finite range (no NaN codes)."""
    c = r.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01
    return c


# ---------------------------------------------------------------- the workload

def test_fp8_prefill_workload():
    w = wl.WORKLOADS["w8a8_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    X = wl.activations(w, M, K, N)
    check_quant(X)
    Aq, s_a = of8.quant_per_token_fp8(wl.as_f64(X).astype(np.float32))
    Bq, s_b = of8.quant_weight_per_channel_fp8(wl.weight(w, K, N))
    check_gemm(Aq, Bq, s_a, s_b, wl.bias(w, N))
    # end to end from the device quantizer: same codes, same product
    Aq_d, s_a_d = ql.f8_quant_per_token(X.cuda())
    out = ql.f8_gemm_scaled(Aq_d, cu(Bq), s_a_d, cu(s_b), wl.bias(w, N).cuda())
    torch.cuda.synchronize()
    ref = of8.fp8_linear(Aq, Bq, s_a, s_b, wl.as_f64(wl.bias(w, N)))
    assert float(np.abs(wl.as_f64(out.cpu()) - ref).max() / np.abs(ref).max()) <= TOL


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("M,K,dtype", [(1, 8, torch.float16), (3, 136, torch.bfloat16), (17, 4096, torch.float16),
                                       (64, 11008, torch.bfloat16), (5, 24576, torch.float16)])
def test_quant_shapes(M, K, dtype):
    r = np.random.default_rng(M * K)
    X = torch.from_numpy((r.standard_normal((M, K)) * r.choice([1e-3, 1.0, 50.0], size=(M, 1)))
                         .astype(np.float32)).to(dtype)
    check_quant(X)


def test_quant_extremes():
    """Zero rows (the 1e-5 floor), tiny rows (subnormal codes), a row whose
    values sit on exact E4M3 points and midpoints after scaling."""
    K = 256
    X = np.zeros((5, K), np.float32)
    X[1] = np.linspace(-1e-6, 1e-6, K)
    X[2] = np.random.default_rng(2).standard_normal(K) * 1e-3
    vals = np.sort(of8.E4M3_VALUES[:0x7F])
    X[3, :127] = vals
    X[3, 127:253] = ((vals[:-1] + vals[1:]) / 2)[:126]
    X[3, 255] = 448.0                                   # scale exactly 1
    X[4] = -X[3]
    for dtype in (torch.float16, torch.bfloat16):
        check_quant(torch.from_numpy(X).to(dtype))


# ---------------------------------------------------------------- GEMM

# 128 x 128 tiles on small grids (the first five), 256 x 128 tiles otherwise
@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (5, 40, 48), (130, 72, 96), (256, 384, 512), (300, 260, 1040),
                                   (2100, 2050, 1040)])
def test_gemm_ragged(M, N, K):
    r = np.random.default_rng(M + N + K)
    Aq, s_a = of8.quant_per_token_fp8(r.standard_normal((M, K)).astype(np.float32))
    Bq, s_b = of8.quant_weight_per_channel_fp8((r.standard_normal((N, K)) * 0.02).astype(np.float32))
    bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).half()
    check_gemm(Aq, Bq, s_a, s_b, bias)


# few tokens: the decode kernel (one 128-byte group per MFMA, fp32 sums
# added across the waves in wave order; up to 64 tokens while M N <= 2^19)
@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (1, 4096, 4096), (5, 100, 1040), (8, 8200, 528), (16, 4096, 4112),
                                   (12, 1, 272), (13, 12000, 2064), (8, 16400, 272), (16, 28672, 400),
                                   (2, 33000, 144), (20, 4096, 2064), (64, 8192, 400), (30, 17000, 528)])
def test_gemm_decode(M, N, K):
    r = np.random.default_rng(3 * M + N + K)
    Aq, s_a = of8.quant_per_token_fp8(r.standard_normal((M, K)).astype(np.float32))
    Bq, s_b = of8.quant_weight_per_channel_fp8((r.standard_normal((N, K)) * 0.02).astype(np.float32))
    bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).half()
    check_gemm(Aq, Bq, s_a, s_b, bias)
    check_gemm(Aq, Bq, s_a[:1], s_b[:1], None, out_dtype=torch.bfloat16)


def test_gemm_decode_all_codes():
    """Every E4M3 code on both sides (random over the whole finite range) with
    few tokens."""
    r = np.random.default_rng(21)
    M, N, K = 16, 300, 2048
    Aq, Bq = _codes(r, (M, K)), _codes(r, (N, K))
    check_gemm(Aq, Bq, np.full(M, 1e-3, np.float32), np.full(N, 1e-3, np.float32))


@pytest.mark.parametrize("M,N", [(96, 136), (2100, 2050)])                 # 128 x 128 and 256 x 128 tiles
def test_gemm_all_codes_and_epilogue_variants(M, N):
    """Random codes over the whole E4M3 range (subnormals, both signs), then
    per-tensor scales, no bias and a bf16 output."""
    K = 256
    r = np.random.default_rng(11)
    Aq, Bq = _codes(r, (M, K)), _codes(r, (N, K))
    # |D| can reach 448 * 448 * K (about 5e7): scales keep the output inside fp16
    s_a = (r.uniform(0.5, 2, M) * 1e-3).astype(np.float32)
    s_b = (r.uniform(0.5, 2, N) * 1e-3).astype(np.float32)
    check_gemm(Aq, Bq, s_a, s_b)
    check_gemm(Aq, Bq, s_a[:1], s_b[:1])
    b16 = torch.from_numpy(np.linspace(-1e5, 1e5, N).astype(np.float32)).to(torch.bfloat16)
    check_gemm(Aq, Bq, s_a, s_b, b16, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("M,N", [(64, 64), (2304, 2048)])                 # 128 x 128 and 256 x 128 tiles
def test_gemm_extreme_codes(M, N):
    """All codes at +-448: D = -448 * 448 * K exactly (49 * 2**24 for K = 4096)."""
    K = 4096
    Aq = np.full((M, K), 0x7E, np.uint8)
    Bq = np.full((N, K), 0xFE, np.uint8)
    s_a = np.full(M, 2.0 ** -20, np.float32)
    s_b = np.full(N, 2.0 ** -10, np.float32)
    out = ql.f8_gemm_scaled(cu(Aq), cu(Bq), cu(s_a), cu(s_b))
    torch.cuda.synchronize()
    assert np.all(out.cpu().float().numpy() == np.float32(-448.0 * 448.0 * K * 2.0 ** -30))
