"""The oracle against closed forms, invariants, library routines and brute
force (CPU only).  Each test names the mistake it is there to catch."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics as nu
from oracle import w4a16 as w4
from oracle import w8a8 as w8


RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- rounding

def test_bf16_matches_torch_cast():
    """bf16 rounding from fp32 equals torch's cast (a library routine), ties included."""
    x = RNG.standard_normal(200000).astype(np.float32) * np.float32(37.0)
    # exact ties: fp32 values half-way between two bf16 numbers, both parities
    base = RNG.integers(0x3F000000, 0x4F000000, 4096, dtype=np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    big = np.array([3.3895314e38, 3.40e38, -3.40e38, 1e-39, -1e-40, 0.0], np.float32)
    for v in (x, ties, big):
        ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
        got = nu.to_bf16(v.astype(np.float64))
        assert np.array_equal(got, ref, equal_nan=True)


def test_bf16_bits_round_trip():
    v = nu.to_bf16(RNG.standard_normal(1000))
    assert np.array_equal(nu.bf16_from_bits(nu.bf16_bits(v)), v)


def test_f16_rounds_once_from_f64():
    """fp64 -> fp16 is one rounding: a value just above a tie (invisible in fp32) rounds up."""
    one_ulp = 2.0 ** -10
    x = 1.0 + one_ulp / 2 + 2.0 ** -40          # fp32 would drop the 2**-40 and tie to even (1.0)
    assert float(nu.to_f16(x)) == 1.0 + one_ulp


def test_signed_nibble_all_codes():
    for n in range(16):
        assert int(nu.signed_nibble(n)) == (n if n < 8 else n - 16)


# ---------------------------------------------------------------- W4 quantizer

def _w(N, K, std=0.02, seed=0):
    return (np.random.default_rng(seed).standard_normal((N, K)) * std).astype(np.float32)


def test_w4_quantizer_ranges_and_error_bound():
    """Codes and zeros are 4-bit; every weight is within one scale step of its
    dequantized value (rounding <= s/2, plus <= s/2 for the rounded zero point);
    each group's extreme values land on codes 0 and 15 (+-1).  A wrong sign of z
    or a scale of range/16 breaks these."""
    W = _w(64, 512)
    q, s16, z = w4.quantize_w4(W)
    assert q.max() <= 15 and z.max() <= 15
    Wd = w4.dequantize_w4(q, s16, z)
    s_full = np.repeat(s16.astype(np.float64).T, 128, axis=1)
    assert np.all(np.abs(Wd - W) <= s_full * 1.001)
    Wg = W.reshape(64, 4, 128)
    qg = q.reshape(64, 4, 128).astype(int)
    qmin = np.take_along_axis(qg, Wg.argmin(axis=2)[..., None], 2)[..., 0]
    qmax = np.take_along_axis(qg, Wg.argmax(axis=2)[..., None], 2)[..., 0]
    assert np.all(qmin <= 1) and np.all(qmax >= 14)
    # real zero is exact: w = 0 quantizes to code z and dequantizes to 0
    W0 = W.copy()
    W0[:, 5] = 0.0
    q0, s0, z0 = w4.quantize_w4(W0)
    assert np.array_equal(q0[:, 5], z0[0, :])
    assert np.all(w4.dequantize_w4(q0, s0, z0)[:, 5] == 0.0)


def test_w4_quantizer_degenerate_and_one_sided_groups():
    W = np.zeros((3, 256), np.float32)
    W[1, :128] = 0.5                 # positive constant group: mn = 0, z = 0, codes 15
    W[2, 128:] = -0.25               # negative constant group: mx = 0, z = 15, codes 0
    q, s16, z = w4.quantize_w4(W)
    assert s16[0, 0] == np.float16(np.float32(1e-5) / np.float32(15))   # clamped range (an fp16 subnormal)
    assert np.all(q[0] == z[:, 0].repeat(128))
    assert z[0, 1] == 0 and np.all(q[1, :128] == 15)
    assert z[1, 2] == 15 and np.all(q[2, 128:] == 0)
    Wd = w4.dequantize_w4(q, s16, z)
    assert np.allclose(Wd, W, rtol=2e-3, atol=0)


def test_w4_constant_group_closed_form():
    """Positive constant groups are represented (almost) exactly, so the whole
    layer reduces to Y[m, n] = sum_g a[g, n] * sum_{k in g} x[m, k].  Catches a
    wrong group index (k % G instead of k // group) and a transposed product."""
    N, K, M = 5, 512, 3
    a = np.random.default_rng(7).uniform(0.1, 1.0, (K // 128, N)).astype(np.float32)
    W = np.repeat(a.T, 128, axis=1)                        # W[n, k] = a[k // 128, n]
    X = np.random.default_rng(8).standard_normal((M, K))
    q, s16, z = w4.quantize_w4(W)
    Y = w4.w4a16_linear(X, q, s16, z)
    Xs = X.reshape(M, K // 128, 128).sum(axis=2)           # [M, G]
    Y_closed = Xs @ a.astype(np.float64)                    # [M, N]
    assert np.allclose(Y, Y_closed, rtol=2e-3, atol=2e-3 * np.abs(Y_closed).max())


def test_w4_bruteforce_exact_rationals():
    """Tiny layer: the fp64 oracle equals an exact rational triple loop."""
    N, K, M = 3, 256, 2
    W = _w(N, K, seed=3)
    q, s16, z = w4.quantize_w4(W)
    X = nu.to_f16(np.random.default_rng(4).standard_normal((M, K))).astype(np.float64)
    Y = w4.w4a16_linear(X, q, s16, z)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 128
                acc += Fraction(float(X[m, k])) * Fraction(float(s16[g, n])) * (int(q[n, k]) - int(z[g, n]))
            assert abs(float(acc) - Y[m, n]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_w4_group_equal_K_is_per_channel():
    """group = K: one (s, z) per output channel, the per-channel special case."""
    W = _w(4, 256, seed=5)
    q, s16, z = w4.quantize_w4(W, group=256)
    assert s16.shape == (1, 4)
    for n in range(4):
        mn, mx = min(W[n].min(), 0), max(W[n].max(), 0)
        s = np.float16(np.float32(mx - mn) / np.float32(15))
        assert s16[0, n] == s


def test_w4_symmetric_zero8_is_signed_form():
    """Unsigned codes q with z = 8 dequantize exactly like the signed nibbles
    whose two's-complement pattern is q XOR 8 (that is, q - 8) with z = 0."""
    q = np.arange(16, dtype=np.uint8).repeat(8)[None, :]
    s = np.full((1, 1), np.float16(0.02))
    z8 = np.full((1, 1), 8, np.uint8)
    a = w4.dequantize_w4(q, s, z8, group=128)
    b = float(s[0, 0]) * nu.signed_nibble(q ^ 8).astype(np.float64)
    assert np.array_equal(a, b)


def test_pack_round_trip_and_bit_positions():
    q = np.random.default_rng(9).integers(0, 16, (7, 64)).astype(np.uint8)
    words = w4.pack_canonical(q)
    assert words.shape == (8, 7)
    assert np.array_equal(w4.unpack_canonical(words), q)
    # code i of word j sits at bits 4i of words[j, n], k = 8 j + i
    for n, j, i in [(0, 0, 0), (3, 5, 7), (6, 7, 4)]:
        assert (int(words[j, n]) >> (4 * i)) & 0xF == q[n, 8 * j + i]


def test_w4_error_matches_uniform_rounding_model():
    """[LQ] "误差从哪来：舍入与截断" (where the error comes from): rounding error is
    roughly uniform on [-s/2, s/2], so the weight MSE is about mean(s**2) / 12.
    A scale off by a factor (range/16, range/7) or a misplaced zero point moves
    the measured MSE far from the model."""
    W = _w(64, 1024, seed=11)
    q, s16, z = w4.quantize_w4(W)
    err = w4.dequantize_w4(q, s16, z) - W
    s_full = np.repeat(s16.astype(np.float64).T, 128, axis=1)
    ratio = np.mean(err ** 2) / np.mean(s_full ** 2 / 12)
    assert 0.85 < ratio < 1.15


# ---------------------------------------------------------------- W8A8

def test_int_gemm_bruteforce_and_extremes():
    A = RNG.integers(-128, 128, (5, 37)).astype(np.int8)
    B = RNG.integers(-127, 128, (6, 37)).astype(np.int8)
    D = w8.int_gemm(A, B)
    for m in range(5):
        for n in range(6):
            assert D[m, n] == sum(int(A[m, k]) * int(B[n, k]) for k in range(37))
    K = 4096
    A = np.full((2, K), -128, np.int8)
    B = np.full((3, K), -127, np.int8)
    assert np.all(w8.int_gemm(A, B) == 128 * 127 * K)


def test_azp_identity_on_integers():
    """sum_k (a_k - z) b_k == sum_k a_k b_k - z * sum_k b_k, exactly."""
    M, N, K = 4, 5, 300
    A = RNG.integers(-128, 128, (M, K)).astype(np.int8)
    B = RNG.integers(-127, 128, (N, K)).astype(np.int8)
    azp = RNG.integers(-128, 128, M).astype(np.int32)
    adj = w8.azp_adj(B)
    C = w8.corrected_accumulator(w8.int_gemm(A, B), azp, adj)
    for m in range(M):
        for n in range(N):
            assert C[m, n] == sum((int(A[m, k]) - int(azp[m])) * int(B[n, k]) for k in range(K))
    assert np.array_equal(adj, np.array([sum(int(v) for v in B[n]) for n in range(N)]))
    # per-tensor form: azp_adj pre-multiplied by the scalar zero point
    z = 17
    C2 = w8.corrected_accumulator(w8.int_gemm(A, B), None, z * adj)
    C3 = w8.corrected_accumulator(w8.int_gemm(A, B), np.full(M, z, np.int32), adj)
    assert np.array_equal(C2, C3)


def test_epilogue_equals_explicit_dequant_product():
    """s_a s_b (Dq - azp azp_adj) + bias equals dequantizing both operands
    explicitly and multiplying (the epilogue algebra of the vLLM page)."""
    M, N, K = 6, 7, 128
    A = RNG.integers(-128, 128, (M, K)).astype(np.int8)
    B = RNG.integers(-127, 128, (N, K)).astype(np.int8)
    azp = RNG.integers(-128, 128, M).astype(np.int32)
    s_a = RNG.uniform(0.001, 0.05, M)
    s_b = RNG.uniform(0.0001, 0.001, N)
    bias = RNG.standard_normal(N)
    _, out = w8.w8a8_linear(A, B, s_a, s_b, azp, w8.azp_adj(B), bias)
    Ad = s_a[:, None] * (A.astype(np.float64) - azp[:, None])
    Bd = s_b[:, None] * B.astype(np.float64)
    ref = Ad @ Bd.T + bias[None, :]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # scalar scales broadcast; missing bias is zero
    _, o2 = w8.w8a8_linear(A, B, s_a[:1], s_b[:1], azp, w8.azp_adj(B), None)
    assert np.allclose(o2, (s_a[0] * (A - azp[:, None].astype(np.float64))) @ (s_b[0] * B.astype(np.float64)).T)


def test_per_token_asym_invariants():
    X = nu.to_f16(RNG.standard_normal((16, 512)) + 0.3).astype(np.float32)
    X[3] = 0.0                                  # all-zero row: clamped range
    X[4] = np.abs(X[4])                         # non-negative row: mn = 0
    X[5] = np.abs(X[5]) + np.float32(2.0)       # a row far from 0: the range is widened to contain it
    Aq, s_a, azp = w8.quant_per_token_asym(X)
    assert azp.min() >= -128 and azp.max() <= 127
    deq = s_a[:, None].astype(np.float64) * (Aq.astype(np.float64) - azp[:, None])
    assert np.all(np.abs(deq - X) <= s_a[:, None] * 1.0001)
    for m in range(16):
        if X[m].min() < 0:
            assert Aq[m, np.argmin(X[m])] == -128
        if X[m].max() > 0:
            assert Aq[m, np.argmax(X[m])] >= 126
    # real zero is exact: x = 0 maps to code azp
    assert np.all(Aq[3] == azp[3])
    assert azp[4] == -128
    # [LQ] "线性量化": z is an integer code so that real 0 lies on a tick; for
    # a row far from 0 that needs the widened range [0, max]
    assert azp[5] == -128 and s_a[5] == np.float32(X[5].max() / np.float32(255))
    assert s_a[3] == np.float32(np.float32(1e-5) / np.float32(255))


def test_per_token_sym_and_weight_quant_invariants():
    X = RNG.standard_normal((8, 256)).astype(np.float32)
    Aq, s_a = w8.quant_per_token_sym(X)
    assert np.all(np.abs(Aq.astype(int)).max(axis=1) == 127)
    assert np.all(np.abs(Aq * s_a[:, None].astype(np.float64) - X) <= s_a[:, None] * 0.5001)
    W = RNG.standard_normal((8, 256)).astype(np.float32) * np.float32(0.02)
    Bq, s_b = w8.quant_weight_per_channel_sym(W)
    assert np.all(np.abs(Bq.astype(int)).max(axis=1) == 127)
    assert Bq.min() >= -127


def test_w8a8_end_to_end_close_to_float():
    """The quantized layer tracks X·Wᵀ + bias (the page's example stays within 0.012)."""
    X = nu.to_f16(RNG.standard_normal((32, 512)) + 0.3).astype(np.float32)
    W = (RNG.standard_normal((48, 512)) * 0.02).astype(np.float32)
    bias = RNG.standard_normal(48) * 0.1
    Aq, s_a, azp = w8.quant_per_token_asym(X)
    Bq, s_b = w8.quant_weight_per_channel_sym(W)
    _, out = w8.w8a8_linear(Aq, Bq, s_a, s_b, azp, w8.azp_adj(Bq), bias)
    ref = X.astype(np.float64) @ W.astype(np.float64).T + bias
    assert np.abs(out - ref).max() / np.abs(ref).max() < 0.02


def test_corrected_accumulator_needs_adj():
    with pytest.raises(ValueError):
        w8.corrected_accumulator(np.zeros((1, 1), np.int64), np.zeros(1, np.int32), None)


# ---------------------------------------------------------------- FP8 E4M3

def test_fp8_all_codes_round_trip_and_order():
    from oracle import fp8
    codes = np.arange(256, dtype=np.uint8)
    v = fp8.e4m3_decode(codes)
    ok = ~np.isnan(v)
    assert np.array_equal(fp8.e4m3_encode(v[ok]), codes[ok])
    pos = np.sort(v[(codes < 0x80) & ok])
    assert np.all(np.diff(pos) > 0) and pos[0] == 0.0
    assert np.isnan(fp8.e4m3_decode(fp8.e4m3_encode(np.nan)))


def test_fp8_rounding_ties_even_and_saturation():
    from oracle import fp8
    vals = np.sort(fp8.E4M3_VALUES[:0x7F])               # non-negative finite, ascending
    for lo, hi in zip(vals[:-1], vals[1:]):
        mid = (lo + hi) / 2
        c_lo, c_hi = int(fp8.e4m3_encode(lo)), int(fp8.e4m3_encode(hi))
        c_mid = int(fp8.e4m3_encode(mid))
        assert c_mid == (c_lo if c_lo % 2 == 0 else c_hi)   # ties go to the even mantissa
        assert int(fp8.e4m3_encode(np.nextafter(mid, 0))) == c_lo
        assert int(fp8.e4m3_encode(np.nextafter(mid, 1e9))) == c_hi
    for x in (448.0, 449.0, 464.0, 1e6, np.float32(3e38)):
        assert float(fp8.e4m3_decode(fp8.e4m3_encode(x))) == 448.0
        assert float(fp8.e4m3_decode(fp8.e4m3_encode(-x))) == -448.0
    assert int(fp8.e4m3_encode(-0.0)) == 0x80 and int(fp8.e4m3_encode(2.0 ** -11)) == 0


def test_fp8_per_token_quant_invariants():
    from oracle import fp8
    r = np.random.default_rng(5)
    X = (r.standard_normal((6, 256)) * np.array([1e-3, 0.1, 1, 10, 300, 1e4])[:, None]).astype(np.float32)
    X[2, :] = 0.0
    q, s = fp8.quant_per_token_fp8(X)
    assert q.dtype == np.uint8 and s.dtype == np.float32
    v = fp8.e4m3_decode(q)
    assert np.all(np.abs(v) <= 448.0)
    for m in (0, 1, 3, 4, 5):
        assert np.max(np.abs(v[m])) == 448.0                 # the row absmax maps to the largest code
        # relative error of each element within half an E4M3 ulp (2**-4) or the subnormal step
        err = np.abs(v[m] * np.float64(s[m]) - X[m])
        bound = np.maximum(np.abs(X[m]) * 2.0 ** -4, 2.0 ** -10 * np.float64(s[m]))
        assert np.all(err <= bound * (1 + 1e-6))
    assert np.all(v[2] == 0.0)


def test_fp8_gemm_exact_against_fractions():
    from fractions import Fraction
    from oracle import fp8
    r = np.random.default_rng(9)
    A = r.integers(0, 256, (3, 40), dtype=np.uint8)
    B = r.integers(0, 256, (4, 40), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x38                             # no NaN codes
    B[(B & 0x7F) == 0x7F] = 0xB8
    D = fp8.fp8_gemm(A, B)
    va, vb = fp8.E4M3_VALUES[A], fp8.E4M3_VALUES[B]
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(va[m], vb[n]))
            assert Fraction(float(D[m, n])) == exact
    out = fp8.fp8_linear(A, B, np.float32([0.5, 2, 4]), np.float32([1, 0.25, 3, 8]), np.float64([1, 2, 3, 4]))
    assert np.allclose(out, np.float64([0.5, 2, 4])[:, None] * np.float64([1, 0.25, 3, 8])[None] * D + [1, 2, 3, 4],
                       rtol=0, atol=0)


# ---------------------------------------------------------------- RMSNorm + per-token quant

def _f16_rows(r, M, K, scale=1.0):
    return (r.standard_normal((M, K)) * scale).astype(np.float16).astype(np.float64)


def test_rmsnorm_constant_rows_closed_form():
    # row m = c_m everywhere: y[m, k] = gamma[k] * c_m / sqrt(c_m^2 + eps)
    from oracle import rmsnorm as rn
    c = np.array([0.5, -3.0, 7.25, 1e-3])
    gamma = np.linspace(-2.0, 3.0, 9)
    for eps in (0.0, 1e-6, 0.25):
        X = np.repeat(c[:, None], 9, axis=1)
        want = gamma[None, :] * (c / np.sqrt(c * c + eps))[:, None]
        np.testing.assert_allclose(rn.rms_norm64(X, gamma, eps), want, rtol=1e-14)
        y32, _ = rn.rms_norm_f32(X, gamma, eps)
        np.testing.assert_allclose(y32, want, rtol=4 * 2.0 ** -24, atol=1e-30)


def test_rmsnorm_f32_steps_against_exact_arithmetic():
    # mean square within one fp32 ulp of the exact rational value; y within a
    # few fp32 ulps of the exact real result
    from oracle import rmsnorm as rn
    r = np.random.default_rng(11)
    for K in (1, 3, 8, 33):
        X = _f16_rows(r, 4, K, 3.0)
        gamma = _f16_rows(r, 1, K)[0]
        eps = 1e-5
        ms = rn.mean_square_f32(X)
        y32, inv = rn.rms_norm_f32(X, gamma, eps)
        for m in range(4):
            ex = sum(Fraction(float(v)) ** 2 for v in X[m]) / K
            assert abs(Fraction(float(ms[m])) - ex) <= Fraction(float(np.spacing(np.float32(ms[m]))))
            exact_inv = 1.0 / np.sqrt(float(ex) + float(np.float32(eps)))
            assert abs(float(inv[m]) - exact_inv) <= 3 * 2.0 ** -24 * exact_inv
            want = X[m] * exact_inv * gamma
            assert np.all(np.abs(y32[m] - want) <= 5 * 2.0 ** -24 * np.abs(want) + 1e-40)


def test_rmsnorm_power_of_two_scale_invariance_is_exact():
    # with eps = 0, scaling a row by 2**j changes nothing, bit for bit
    from oracle import rmsnorm as rn
    r = np.random.default_rng(12)
    X = _f16_rows(r, 3, 64)
    gamma = _f16_rows(r, 1, 64)[0]
    y0, _ = rn.rms_norm_f32(X, gamma, 0.0)
    for j in (-6, 3):
        yj, _ = rn.rms_norm_f32(X * 2.0 ** j, gamma, 0.0)
        assert np.array_equal(y0, yj)


def test_rmsnorm_rows_are_independent_and_gamma_is_per_channel():
    from oracle import rmsnorm as rn
    r = np.random.default_rng(13)
    X = _f16_rows(r, 5, 16)
    gamma = _f16_rows(r, 1, 16)[0]
    y, _ = rn.rms_norm_f32(X, gamma, 1e-6)
    for m in range(5):
        ym, _ = rn.rms_norm_f32(X[m:m + 1], gamma, 1e-6)
        assert np.array_equal(ym[0], y[m])
    # permuting channels of x and gamma together permutes y
    p = r.permutation(16)
    yp, _ = rn.rms_norm_f32(X[:, p], gamma[p], 1e-6)
    assert np.array_equal(yp, y[:, p])


def test_rmsnorm_quant_is_the_per_token_quant_of_y():
    from oracle import rmsnorm as rn
    from oracle import w8a8 as w8
    r = np.random.default_rng(14)
    X = _f16_rows(r, 6, 128, 2.0)
    gamma = _f16_rows(r, 1, 128)[0]
    Aq, s_a, azp = rn.rmsnorm_quant_per_token(X, gamma, 1e-6)
    y, _ = rn.rms_norm_f32(X, gamma, 1e-6)
    Aq2, s2, z2 = w8.quant_per_token_asym(y)
    assert np.array_equal(Aq, Aq2) and np.array_equal(s_a, s2) and np.array_equal(azp, z2)
    # dequantized codes sit within half a step of y
    deq = s_a[:, None].astype(np.float64) * (Aq.astype(np.float64) - azp[:, None])
    assert np.all(np.abs(deq - y) <= 0.5 * s_a[:, None] * (1 + 1e-6))
    Aqs, ss = rn.rmsnorm_quant_per_token(X, gamma, 1e-6, asym=False)
    assert np.all(np.abs(Aqs.astype(np.int32)).max(axis=1) == 127)


# ---------------------------------------------------------------- act-order (g_idx)

def test_act_order_identity_order_is_the_plain_path():
    from oracle import w4a16 as w4
    r = np.random.default_rng(21)
    W = (r.standard_normal((24, 384)) * 0.02).astype(np.float32)
    X = r.standard_normal((3, 384))
    g = w4.g_idx_from_order(np.arange(384))
    assert np.array_equal(g, np.arange(384) // 128)
    qa, sa, za = w4.quantize_w4_act_order(W, g)
    q, s, z = w4.quantize_w4(W)
    assert np.array_equal(qa, q) and np.array_equal(sa.view(np.uint16), s.view(np.uint16)) and np.array_equal(za, z)
    np.testing.assert_array_equal(w4.w4a16_linear_gidx(X, qa, sa, za, g), w4.w4a16_linear(X, q, s, z))


def test_act_order_equals_plain_path_on_permuted_channels():
    # quantizing in order P == plain grouping of W[:, P]; the product is the
    # same with X[:, P]
    from oracle import w4a16 as w4
    r = np.random.default_rng(22)
    K = 512
    W = (r.standard_normal((16, K)) * 0.02).astype(np.float32)
    X = r.standard_normal((4, K))
    P = r.permutation(K)
    g = w4.g_idx_from_order(P)
    qa, sa, za = w4.quantize_w4_act_order(W, g)
    q, s, z = w4.quantize_w4(W[:, P])
    assert np.array_equal(qa[:, P], q) and np.array_equal(sa.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(za, z)
    np.testing.assert_allclose(w4.w4a16_linear_gidx(X, qa, sa, za, g), w4.w4a16_linear(X[:, P], q, s, z),
                               rtol=1e-12, atol=1e-12)
    # every group holds exactly `group` channels and g_idx inverts the order
    assert np.all(np.bincount(g) == 128)
    assert np.all(g[P] == np.arange(K) // 128)


def test_act_order_brute_force_tiny():
    # one output channel, K = 256: the product written out channel by channel
    from oracle import w4a16 as w4
    r = np.random.default_rng(23)
    K = 256
    W = (r.standard_normal((1, K)) * 0.05).astype(np.float32)
    x = r.standard_normal(K)
    P = r.permutation(K)
    g = w4.g_idx_from_order(P)
    q, s, z = w4.quantize_w4_act_order(W, g)
    want = sum(x[k] * float(s[g[k], 0]) * (int(q[0, k]) - int(z[g[k], 0])) for k in range(K))
    got = w4.w4a16_linear_gidx(x[None], q, s, z, g)[0, 0]
    assert abs(got - want) <= 1e-12 * max(1.0, abs(want))
    # a wrong channel-to-group map changes the result
    g_bad = np.roll(g, 1)
    assert abs(w4.w4a16_linear_gidx(x[None], q, s, z, g_bad)[0, 0] - want) > 1e-6


def test_rmsnorm_mean_square_on_and_next_to_an_fp32_boundary():
    """The mean-square reading (the correctly rounded fp64 sum of the exact
    squares, then fp32) on rows built with exact integers: a row whose mean
    square IS an fp32 midpoint rounds to the even neighbour; a row whose exact
    mean square lies just above the midpoint rounds up, although a plain fp64
    sum that adds the tiny squares last lands on the midpoint and rounds down
    (the order dependence the correctly rounded reading removes)."""
    from fractions import Fraction
    from oracle import rmsnorm as rn
    from tests import rmsnorm_rows as rr
    def neighbours(mid):
        f = np.float32(mid)
        below = f if float(f) < mid else np.nextafter(f, np.float32(0))
        up = np.nextafter(below, np.float32(8))
        assert float(below) < mid < float(up) and float(up) - mid == mid - float(below)
        assert int(below.view(np.uint32)) % 2 == 0               # the lower neighbour is the even one
        return below, up

    x, mid = rr.tie_row()
    assert sum(Fraction(v) ** 2 for v in x.tolist()) / rr.K == Fraction(mid)
    below, _ = neighbours(mid)
    assert rn.mean_square_f32(x[None, :])[0] == below
    for kw in ({}, {"tiny_start": 2048, "big_from": 0}):
        x, mid = rr.straddle_row(**kw)
        below, up = neighbours(mid)
        exact = sum(Fraction(v) ** 2 for v in x.tolist()) / rr.K
        assert exact > Fraction(mid) and float(exact - Fraction(mid)) < 1e-14
        assert rn.mean_square_f32(x[None, :])[0] == up
        seq = 0.0
        for v in np.concatenate([x[x != rr.TINY], x[x == rr.TINY]]):
            seq += v * v
        assert np.float32(seq / rr.K) == below
