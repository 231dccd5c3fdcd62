"""W8A8 parity on the GPU.

i8_quant_per_token: codes, zero points and fp32 scales bit-exact with the
oracle (both decide the codes in IEEE fp32 with round-half-to-even).
i8_gemm_scaled: the int32 corrected accumulator (raw_out) bit-exact with the
oracle's exact integer product, the fp16/bf16 output within
max|out - out64| / max|out64| <= 1e-2 and, element by element, within the
bound of the epilogue's own roundings (epilogue_bound).  The GEMM's inputs
are the oracle's own quantized operands.
"""

import numpy as np
import pytest
import torch

import quantized_linear_layers_amd as ql
import workloads as wl
from oracle import w8a8 as ow8

pytestmark = pytest.mark.gpu
TOL = 1e-2


def cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_quant(X, symmetric=False):
    Aq, s_a, azp = ql.i8_quant_per_token(X.cuda(), symmetric=symmetric)
    torch.cuda.synchronize()
    Xf = wl.as_f64(X).astype(np.float32)
    if symmetric:
        Aq_o, s_o = ow8.quant_per_token_sym(Xf)
        assert azp is None
    else:
        Aq_o, s_o, azp_o = ow8.quant_per_token_asym(Xf)
        assert np.array_equal(azp.cpu().numpy(), azp_o)
    assert np.array_equal(s_a.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(Aq.cpu().numpy(), Aq_o)


def epilogue_bound(C, s_a, s_b, bias, out64, out_dtype):
    """Element-wise bound of the fused epilogue's float output: the int32 C
    is exact, then at most four fp32 roundings (C to fp32, the two scale
    products, the bias add), each within 2^-24 of a magnitude at most
    |s_a s_b C| + |bias|, and one rounding to the output type (half an ulp:
    at most 2^-11 |out| for fp16 and 2^-8 |out| for bf16, plus half the
    fp16 subnormal spacing).  The fp32 term takes 5 units instead of 4 to
    cover the output rounding's share of the fp32 error."""
    sa = np.broadcast_to(np.asarray(s_a, np.float64).reshape(-1, 1), out64.shape)
    sb = np.broadcast_to(np.asarray(s_b, np.float64).reshape(1, -1), out64.shape)
    mag = np.abs(sa * sb * C.astype(np.float64))
    if bias is not None:
        mag = mag + np.abs(wl.as_f64(bias)).reshape(1, -1)
    half_ulp = (2.0 ** -11 * np.abs(out64) + 2.0 ** -25) if out_dtype == torch.float16 else 2.0 ** -8 * np.abs(out64)
    return half_ulp + 5 * 2.0 ** -24 * mag


def check_epilogue_bound(o, C, s_a, s_b, bias, out64, out_dtype):
    err = np.abs(wl.as_f64(o.cpu()) - out64)
    b = epilogue_bound(C, s_a, s_b, bias, out64, out_dtype)
    worst = np.unravel_index(np.argmax(err / b), err.shape)
    assert (err <= b).all(), f"element {worst}: |err| {err[worst]:.3e} exceeds the epilogue bound {b[worst]:.3e}"


def check_gemm(Aq, Bq, s_a, s_b, azp=None, adj=None, bias=None, out_dtype=torch.float16):
    """With raw_out (per-element epilogue, the int32 accumulator kept) and
    without it (tiles wholly inside Y stage their outputs through LDS and
    store rows: the path the throughput figures time): both against the
    oracle."""
    args = (cu(Aq), cu(Bq), cu(s_a), cu(s_b), None if azp is None else cu(azp), None if adj is None else cu(adj),
            None if bias is None else bias.cuda())
    out, raw = ql.i8_gemm_scaled(*args, out_dtype=out_dtype, raw=True)
    out_fast = ql.i8_gemm_scaled(*args, out_dtype=out_dtype)
    torch.cuda.synchronize()
    C, out64 = ow8.w8a8_linear(Aq, Bq, s_a, s_b, azp, adj, None if bias is None else wl.as_f64(bias))
    assert np.array_equal(raw.cpu().numpy().astype(np.int64), C)
    for o in (out, out_fast):
        od = wl.as_f64(o.cpu())
        e = float(np.abs(od - out64).max() / np.abs(out64).max())
        assert e <= TOL, f"relative error {e:.3e}"
        check_epilogue_bound(o, C, s_a, s_b, bias, out64, out_dtype)


# ---------------------------------------------------------------- the workload

def test_w8a8_prefill_workload():
    w = wl.WORKLOADS["w8a8_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    X = wl.activations(w, M, K, N)
    check_quant(X)
    Aq, s_a, azp = ow8.quant_per_token_asym(wl.as_f64(X).astype(np.float32))
    Bq, s_b = ow8.quant_weight_per_channel_sym(wl.weight(w, K, N))
    check_gemm(Aq, Bq, s_a, s_b, azp, ow8.azp_adj(Bq), wl.bias(w, N))


# ---------------------------------------------------------------- variants and edges

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,K", [(1, 8), (3, 40), (7, 4096), (5, 20000), (64, 1000)])
@pytest.mark.parametrize("symmetric", [False, True])
def test_quant_shapes(M, K, dtype, symmetric):
    r = np.random.default_rng(M * 31 + K)
    Xf = (r.standard_normal((M, K)) * 3 + 0.5).astype(np.float32)
    X = torch.from_numpy(Xf).to(dtype)
    check_quant(X, symmetric)


def test_quant_degenerate_rows():
    X = torch.zeros((4, 64), dtype=torch.float16)
    X[1] = 2.0                     # constant positive row: mn = 0
    X[2] = -3.0                    # constant negative row: mx = 0
    X[3, 5] = 65504.0              # fp16 max
    check_quant(X)
    check_quant(X, symmetric=True)


def _operands(M, N, K, seed):
    r = np.random.default_rng(seed)
    Xf = (r.standard_normal((M, K)) + 0.3).astype(np.float32)
    Aq, s_a, azp = ow8.quant_per_token_asym(Xf)
    Bq, s_b = ow8.quant_weight_per_channel_sym((r.standard_normal((N, K)) * 0.02).astype(np.float32))
    return Aq, s_a, azp, Bq, s_b


# the GEMM takes 128 x 128 tiles when 256 x 128 ones would fill at most half
# the compute units (the first five shapes, and 1024 x 4096: exactly 128 of
# them) and 256 x 128 tiles otherwise (1025 x 4096: 160)
SMALL_AND_LARGE = [(1, 16, 16), (5, 40, 48), (130, 72, 96), (256, 384, 512), (300, 260, 1040), (2100, 2050, 1040),
                   (4097, 1000, 528), (1024, 4096, 272), (1025, 4096, 272)]


@pytest.mark.parametrize("M,N,K", SMALL_AND_LARGE)
def test_gemm_ragged(M, N, K):
    Aq, s_a, azp, Bq, s_b = _operands(M, N, K, M + N + K)
    bias = torch.from_numpy(np.random.default_rng(1).standard_normal(N).astype(np.float32) * 0.1).half()
    check_gemm(Aq, Bq, s_a, s_b, azp, ow8.azp_adj(Bq), bias)


# Up to 16 tokens, and up to 64 while M N <= 2^19, take the decode kernel: 16
# output channels per workgroup up to N = 16384, 32 up to 32768, 64 beyond
# (16400, 20000, 28672 and 33000 columns), K in 128-byte groups split among 4
# waves (ragged K, K shorter than the waves, N not a multiple of 16, 8, 16,
# 32 or 64 staged activation rows); 64 x 8193 is just past the rule (tiled
# GEMM)
DECODE = [(1, 16, 16), (1, 4096, 4096), (3, 100, 1040), (8, 8200, 528), (9, 1000, 4112), (16, 4096, 4096),
          (16, 8192, 1024), (2, 17, 48), (13, 12000, 2064), (16, 1, 272), (8, 16400, 272), (16, 28672, 400),
          (2, 33000, 144), (17, 4096, 1040), (33, 2000, 4112), (64, 8192, 528), (48, 100, 2064), (24, 20000, 272),
          (64, 8193, 272)]


@pytest.mark.parametrize("M,N,K", DECODE)
def test_gemm_decode(M, N, K):
    Aq, s_a, azp, Bq, s_b = _operands(M, N, K, 7 * M + N + K)
    bias = torch.from_numpy(np.random.default_rng(2).standard_normal(N).astype(np.float32) * 0.1).half()
    check_gemm(Aq, Bq, s_a, s_b, azp, ow8.azp_adj(Bq), bias)


def test_gemm_decode_variants_and_extremes():
    """The decode kernel's epilogue variants, all codes at the int8 extremes
    (Dq = 128 * 127 * K exactly), and zero points past 24 bits."""
    M, N, K = 11, 520, 4096
    Aq, s_a, azp, Bq, s_b = _operands(M, N, K, 8)
    adj = ow8.azp_adj(Bq)
    check_gemm(Aq, Bq, s_a, s_b)
    check_gemm(Aq, Bq, s_a[:1], s_b[:1], None, (5 * adj).astype(np.int32))
    b16 = torch.from_numpy(np.linspace(-1, 1, N).astype(np.float32)).to(torch.bfloat16)
    check_gemm(Aq, Bq, s_a, s_b, azp, adj, b16, out_dtype=torch.bfloat16)
    check_gemm(np.full((M, K), -128, np.int8), np.full((N, K), -127, np.int8), np.full(M, 1e-3, np.float32),
               np.full(N, 1e-4, np.float32))
    r = np.random.default_rng(9)
    wide = (r.integers(-1, 2, M) * ((1 << 23) + r.integers(0, 1 << 20, M))).astype(np.int32)
    Bz = np.zeros((N, K), np.int8)
    Bz[:, :3] = r.integers(-1, 2, (N, 3))
    check_gemm(Aq, Bz, np.full(M, 1e-6, np.float32), np.full(N, 1e-2, np.float32), wide, ow8.azp_adj(Bz))


@pytest.mark.parametrize("M,N,K", [(96, 136, 256), (2100, 2050, 256)])    # 128 x 128 and 256 x 128 tiles
def test_gemm_epilogue_variants(M, N, K):
    Aq, s_a, azp, Bq, s_b = _operands(M, N, K, 5)
    adj = ow8.azp_adj(Bq)
    check_gemm(Aq, Bq, s_a, s_b)                                   # symmetric, no bias
    check_gemm(Aq, Bq, s_a[:1], s_b[:1])                           # per-tensor scales
    check_gemm(Aq, Bq, s_a, s_b, None, (17 * adj).astype(np.int32))   # per-tensor zero point folded in
    b16 = torch.from_numpy(np.linspace(-1, 1, N).astype(np.float32)).to(torch.bfloat16)
    check_gemm(Aq, Bq, s_a, s_b, azp, adj, b16, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("M,N", [(64, 64), (2304, 2048)])                 # 128 x 128 and 256 x 128 tiles
def test_gemm_extreme_codes(M, N):
    """All codes at the int8 extremes: Dq reaches 128 * 127 * K exactly."""
    K = 4096
    Aq = np.full((M, K), -128, np.int8)
    Bq = np.full((N, K), -127, np.int8)
    s_a = np.full(M, 1e-3, np.float32)
    s_b = np.full(N, 1e-4, np.float32)
    check_gemm(Aq, Bq, s_a, s_b)


@pytest.mark.parametrize("M,N", [(256, 256), (2048, 2304)])               # 128 x 128 and 256 x 128 tiles
def test_gemm_wide_zero_points(M, N):
    """Zero points and column sums past 24 bits (the epilogue then forms
    azp * azp_adj with a 32-bit multiply): still exact.  Full tiles of either
    shape, so the row-staged store path is the one checked without raw_out."""
    K = 512
    r = np.random.default_rng(11)
    Aq = r.integers(-128, 128, (M, K)).astype(np.int8)
    Bq = np.zeros((N, K), np.int8)
    Bq[:, :3] = r.integers(-1, 2, (N, 3))          # column sums in -3..3
    azp = (r.integers(-1, 2, M) * ((1 << 23) + r.integers(0, 1 << 20, M))).astype(np.int32)
    s_a = np.full(M, 1e-6, np.float32)
    s_b = np.full(N, 1e-2, np.float32)
    adj = ow8.azp_adj(Bq)
    check_gemm(Aq, Bq, s_a, s_b, azp, adj)
    wide_adj = adj.astype(np.int64) + (1 << 24)    # a column sum past 24 bits, any zero points
    check_gemm(Aq, Bq, s_a, s_b, (azp % 64).astype(np.int32), wide_adj.astype(np.int32))


def test_gemm_operand_over_4gib():
    """Aq past 4 GiB (M*K > 2^32): the main loop's copies then take 64-bit
    row addresses instead of 32-bit lane offsets from the operand's base.
    Aq is drawn on the device from a seeded generator; sampled rows (among
    them the first and the last tile's) are checked against the oracle: the
    int32 accumulator bit-exact, both output paths within the tolerance."""
    M, N, K = (1 << 20) + 7, 160, 4112            # ragged M, N and K
    assert M * K > 0xFFFFFFFF
    g = torch.Generator(device="cuda").manual_seed(11)
    Aq = torch.randint(-128, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    r = np.random.default_rng(12)
    Bq, s_b = ow8.quant_weight_per_channel_sym((r.standard_normal((N, K)) * 0.02).astype(np.float32))
    s_a = (r.random(M) * 0.01 + 1e-3).astype(np.float32)
    azp = r.integers(-128, 128, M).astype(np.int32)
    adj = ow8.azp_adj(Bq)
    bias = torch.from_numpy(r.standard_normal(N).astype(np.float32) * 0.1).half()
    args = (Aq, cu(Bq), cu(s_a), cu(s_b), cu(azp), cu(adj), bias.cuda())
    out, raw = ql.i8_gemm_scaled(*args, raw=True)
    out_fast = ql.i8_gemm_scaled(*args)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M // 2, M - 257, M - 8, M - 1], r.integers(0, M, 24)]))
    ri = torch.from_numpy(rows).cuda()
    C, out64 = ow8.w8a8_linear(Aq.index_select(0, ri).cpu().numpy(), Bq, s_a[rows], s_b, azp[rows], adj,
                               wl.as_f64(bias))
    assert np.array_equal(raw.index_select(0, ri).cpu().numpy().astype(np.int64), C)
    for o in (out, out_fast):
        os_ = o.index_select(0, ri)
        od = wl.as_f64(os_.cpu())
        e = float(np.abs(od - out64).max() / np.abs(out64).max())
        assert e <= TOL, f"relative error {e:.3e}"
        check_epilogue_bound(os_, C, s_a[rows], s_b, bias, out64, torch.float16)
    del Aq, raw, out, out_fast
    torch.cuda.empty_cache()


def test_gemm_small_tiles_operand_over_4gib():
    """The 128 x 128 tiles with Aq past 4 GiB (a few rows of a very long K,
    ragged against the 64-byte blocks): 64-bit row addresses in that tile's
    main loop too.  Sampled rows against the oracle, as above."""
    M, N, K = 259, 16, (1 << 24) + 48
    assert M * K > 0xFFFFFFFF
    g = torch.Generator(device="cuda").manual_seed(13)
    Aq = torch.randint(-128, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    r = np.random.default_rng(14)
    Bq = r.integers(-127, 128, (N, K)).astype(np.int8)
    s_a = (r.random(M) * 0.01 + 1e-3).astype(np.float32)
    s_b = (r.random(N) * 1e-4 + 1e-5).astype(np.float32)
    azp = r.integers(-128, 128, M).astype(np.int32)
    adj = ow8.azp_adj(Bq)
    args = (Aq, cu(Bq), cu(s_a), cu(s_b), cu(azp), cu(adj), None)
    out, raw = ql.i8_gemm_scaled(*args, raw=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 200, M - 1])
    ri = torch.from_numpy(rows).cuda()
    C, out64 = ow8.w8a8_linear(Aq.index_select(0, ri).cpu().numpy(), Bq, s_a[rows], s_b, azp[rows], adj)
    assert np.array_equal(raw.index_select(0, ri).cpu().numpy().astype(np.int64), C)
    os_ = out.index_select(0, ri)
    assert float(np.abs(wl.as_f64(os_.cpu()) - out64).max() / np.abs(out64).max()) <= TOL
    check_epilogue_bound(os_, C, s_a[rows], s_b, None, out64, torch.float16)
    del Aq, raw, out
    torch.cuda.empty_cache()


def test_launcher_matches_the_binding():
    """The pre-marshalled launcher (used for tight launch loops) gives the
    same bytes as the checked binding, for the quant and the GEMM entry
    points, on two calls in a row."""
    w = wl.WORKLOADS["w8a8_prefill"]
    M, K, N = 300, 1024, 384
    X = wl.activations(w, M, K, N).cuda()
    Aq, s_a, azp = ql.i8_quant_per_token(X)
    Aq2, s_a2, azp2 = torch.empty_like(Aq), torch.empty_like(s_a), torch.empty_like(azp)
    lq = ql.launcher("i8_quant_per_token", X, X.dtype, M, K, Aq2, s_a2, azp2)
    Bq, s_b = ql.i8_quant_weight_host(torch.from_numpy(wl.weight(w, K, N)))
    adj = ql.i8_azp_adj(Bq)
    Bq, s_b, adj = Bq.cuda(), s_b.cuda(), adj.cuda()
    bias = wl.bias(w, N).cuda()
    out = ql.i8_gemm_scaled(Aq, Bq, s_a, s_b, azp, adj, bias)
    out2 = torch.empty_like(out)
    lg = ql.launcher("i8_gemm_scaled", Aq2, Bq, M, N, K, s_a2, M, s_b, N, azp2, adj, bias, out2, out.dtype, None)
    for _ in range(2):
        lq()
        lg()
        torch.cuda.synchronize()
        assert torch.equal(Aq2, Aq) and torch.equal(azp2, azp)
        assert torch.equal(s_a2.view(torch.int32), s_a.view(torch.int32))
        assert torch.equal(out2, out)
        for t in (Aq2, s_a2, azp2, out2):
            t.zero_()
