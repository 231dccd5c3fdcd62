"""The oracle against values the pages print (tests/golden/*.json, each with
its source).  CPU only."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import numerics as nu
from oracle import quant as qu
from oracle import w4a16 as w4
from oracle import w8a8 as w8
from tests.conftest import golden


# ---------------------------------------------------------------- numerics

def test_float_encodings():
    g = golden("lq_float_encodings.json")
    c13, c70k = g["cases"]
    assert round(float(nu.to_f16(1.0 / 3.0)), 6) == c13["f16"]
    assert round(float(nu.to_bf16(1.0 / 3.0)), 6) == c13["bf16"]
    assert np.isinf(nu.to_f16(70000.0))
    assert float(nu.to_bf16(70000.0)) == c70k["bf16"]


def test_nibble_readings():
    for p in golden("lq_int4_nibbles.json")["patterns"]:
        n = int(p["bits"], 2)
        assert n == p["unsigned"]
        assert int(nu.signed_nibble(n)) == p["signed"]


def test_magic_constants_decode():
    g = golden("qk_magic_constants.json")
    for key in ("EX", "SUB", "MUL", "ADD"):
        bits = int(g["f16"][key], 16)
        assert float(nu.f16_from_bits(bits)) == g["f16"][key + "_value"]
    for key in ("EX", "MUL", "ADD"):
        bits = int(g["bf16"][key], 16)
        assert float(nu.bf16_from_bits(bits)) == g["bf16"][key + "_value"]


# ---------------------------------------------------------------- generic quantizers

def test_qk_int8_example():
    g = golden("qk_int8_example.json")
    lo, hi = g["range"]
    s_exact = (hi - lo) / g["levels"]
    assert round(s_exact, 4) == g["scale_printed"]
    for s in (s_exact, g["scale_printed"]):
        codes = qu.quantize(np.array(g["x"]), s, 0, -128, 127)
        assert codes.tolist() == g["codes"]
    d = qu.dequantize(96, g["scale_printed"], 0)
    assert round(d, 3) == g["dequant_of_96_printed"]
    assert round(d - 1.5, 3) == g["dequant_error_printed"]


def test_lq_ruler():
    g = golden("lq_ruler.json")
    s, z = qu.affine_params(*g["range"], g["qmin"], g["qmax"])
    assert s == pytest.approx(g["scale"], abs=1e-12)
    assert z == g["zero_point"]
    codes = qu.quantize(np.array(g["range"]), s, z, g["qmin"], g["qmax"])
    assert codes.tolist() == [g["code_of_xmin"], g["code_of_xmax"]]


def test_lq_asym_vs_sym_vector():
    g = golden("lq_asym_vs_sym.json")
    x = np.array(g["x"])
    # the product quantizer, one group of 8 values
    q, s16, z = w4.quantize_w4(x[None, :], group=8)
    s = float(s16[0, 0])
    zz = int(z[0, 0])
    deq = w4.dequantize_w4(q, s16, z, group=8)[0]
    i_min = int(np.argmin(x))
    assert round(float(deq[i_min]), 2) == g["asym_int4_dequant_of_min"]
    shift = zz - (-x.min() / s)
    assert round(shift, 2) == g["asym_grid_shift_in_scales"]
    # signed 4-bit form: same dequantized values with codes and zero point shifted by 8
    assert zz - 8 == g["signed_form_zero_point"]
    assert np.array_equal(s * ((q[0].astype(int) - 8) - (zz - 8)), deq)
    # symmetric INT4 / INT8 (fp64), against the printed ratios
    s4, q4max = qu.symmetric_params(x, 4)
    s8, q8max = qu.symmetric_params(x, 8)
    mse4 = qu.mse(qu.quantize_symmetric(x, s4, q4max) * s4, x)
    mse8 = qu.mse(qu.quantize_symmetric(x, s8, q8max) * s8, x)
    mse_asym = qu.mse(deq, x)
    assert round(s4 / s8) == g["sym_int4_to_int8_scale_ratio_approx"]
    assert round(mse4 / mse8, -1) == g["sym_int4_over_int8_mse_ratio_approx"]
    assert round(1 - mse_asym / mse4, 2) == g["asym_better_than_sym_int4_fraction_approx"]


def test_lq_gelu_row():
    g = golden("lq_asym_vs_sym.json")
    x = np.array(g["gelu_row"])
    s4, qmax = qu.symmetric_params(x, 4)
    assert s4 == pytest.approx(3.1 / 7)
    mse_sym = qu.mse(qu.quantize_symmetric(x, s4, qmax) * s4, x)
    assert float(f"{mse_sym:.3g}") == g["gelu_sym_int4_mse"]
    q, s16, z = w4.quantize_w4(x[None, :], group=8)
    assert int(z[0, 0]) == g["gelu_asym_int4_zero_point"]
    assert float(s16[0, 0]) == pytest.approx(3.1 / 15, rel=1e-3)   # fp16-rounded scale
    mse_asym = qu.mse(w4.dequantize_w4(q, s16, z, group=8)[0], x)
    assert float(f"{mse_asym:.3g}") == g["gelu_asym_int4_mse"]
    assert round(mse_sym / mse_asym, 1) == g["gelu_improvement_approx"]


def test_lq_granularity():
    g = golden("lq_granularity.json")
    W = np.array(g["W"])
    qmax = g["qmax"]
    s_t = np.abs(W).max() / qmax
    assert round(s_t, 4) == g["per_tensor_scale"]
    q_t = qu.quantize_symmetric(W, s_t, qmax)
    assert q_t[0].tolist() == g["per_tensor_row1_codes"]
    assert round(qu.mse(q_t[0] * s_t, W[0]), 4) == g["per_tensor_row1_mse"]
    s_c = np.abs(W[0]).max() / qmax
    q_c = qu.quantize_symmetric(W[0], s_c, qmax)
    assert q_c.tolist() == g["per_channel_row1_codes"]
    assert np.round(q_c * s_c, 3).tolist() == g["per_channel_row1_dequant"]
    assert round(qu.mse(q_c * s_c, W[0]), 4) == g["per_channel_row1_mse"]
    # effective bits per weight of per-group storage
    assert 4 + (16 + 16) / 128 == g["effective_bits_g128_fp16_scale_and_zero"]
    assert round(4 + (16 + 4) / 128, 2) == g["effective_bits_g128_fp16_scale_4bit_zero_approx"]
    assert 4 + (16 + 16) / 32 == g["effective_bits_g32_fp16_scale_and_zero"]


def test_lq_awq_rtn_example():
    g = golden("lq_awq_rtn_example.json")
    w = np.array(g["w"])
    x = np.array(g["x"])
    assert round(float(w @ x), 3) == g["exact"]
    step = np.abs(w).max() / 3
    wq = qu.quantize_symmetric(w, step, 3, qmin=-4) * step
    assert np.round(np.abs(wq - w), 2).tolist() == g["rtn_abs_errors"]
    assert round(float(wq @ x), 3) == g["rtn_output"]
    sc = np.ones_like(w)
    sc[g["awq_channel"]] = g["awq_scale"]
    ws = w * sc
    step = np.abs(ws).max() / 3
    wsq = qu.quantize_symmetric(ws, step, 3, qmin=-4) * step
    assert np.round(wsq, 2).tolist() == g["awq_quantized_scaled_w"]
    assert round(float(wsq @ (x / sc)), 3) == g["awq_output"]


# ---------------------------------------------------------------- W4A16 packing

def test_lq_pack_example():
    g = golden("lq_pack_example.json")
    codes = np.array(g["codes"], np.uint8)[None, :]          # one output channel, K = 8
    words = w4.pack_canonical(codes)
    assert words.shape == (1, 1)
    assert int(words[0, 0]) == int(g["packed_hex"], 16)
    assert w4.unpack_canonical(words).tolist() == codes.tolist()


def test_lq_magic_number_worked_example():
    """The nibble-into-mantissa example of the W4A16 section, done in numpy fp16."""
    m = golden("lq_pack_example.json")["magic"]
    bits = int(m["f16_bits_of_1024"], 16) | m["q"]
    assert bits == int(m["or_bits"], 16)
    v = nu.f16_from_bits(bits)
    assert float(v) == m["or_value"]
    c = np.float16(v) - np.float16(1024 + m["z"])
    assert float(c) == m["centered"]
    assert round(float(c) * m["s"], 2) == m["dequant"]


# ---------------------------------------------------------------- W8A8

def test_lq_w8a8_example():
    g = golden("lq_w8a8_example.json")
    Wq = np.array(g["Wq"], np.int8)
    Xq = np.array(g["Xq"], np.int8)
    Dq = w8.int_gemm(Xq, Wq)
    assert int(Dq[0, 0]) == g["Dq11"]
    s_w = np.array(g["w_absmax"]) / g["qmax"]
    s_x = np.array(g["x_absmax"]) / g["qmax"]
    assert np.round(s_w, 6).tolist() == g["s_w_printed"]
    assert np.round(s_x, 6).tolist() == g["s_x_printed"]
    C, out = w8.w8a8_linear(Xq, Wq, s_x, s_w)
    assert np.array_equal(C, Dq)
    assert np.round(out, 4).tolist() == g["Y_printed"]
    b = g["int32_bound"]
    assert 127 * 127 == b["max_product"]
    assert round(b["max_product"] * b["K"], -6) == b["approx_sum"]
    # the printed weight codes and scales are what the per-channel weight
    # quantizer gives.  The page prints each row's absmax and codes but not
    # the fp weights; both rows hold the extreme code 127, so the row on the
    # printed grid, Wq[n] * absmax[n] / 127, has exactly the printed absmax.
    Wf = (Wq.astype(np.float64) * (np.array(g["w_absmax"]) / g["qmax"])[:, None]).astype(np.float32)
    assert np.abs(Wf).max(axis=1).tolist() == pytest.approx(g["w_absmax"], rel=1e-7)
    Bq, s_b = w8.quant_weight_per_channel_sym(Wf)
    assert Bq.tolist() == g["Wq"]
    assert np.round(s_b.astype(np.float64), 6).tolist() == g["s_w_printed"]
    # the printed activation codes are what the symmetric per-token quantizer
    # gives for a row whose absmax is the printed one (the row's own max
    # element maps to the extreme code)
    for r in range(2):
        row = Xq[r].astype(np.float64) * s_x[r]
        Aq, s_a = w8.quant_per_token_sym(row[None, :].astype(np.float32))
        assert Aq[0].tolist() == Xq[r].tolist()
        assert float(s_a[0]) == pytest.approx(s_x[r], rel=1e-6)


def test_exact_fraction_w8a8_epilogue():
    """Example outputs recomputed with exact rationals agree with the fp64 epilogue."""
    g = golden("lq_w8a8_example.json")
    Wq, Xq = g["Wq"], g["Xq"]
    for m in range(2):
        for n in range(2):
            dq = sum(Xq[m][k] * Wq[n][k] for k in range(3))
            y = Fraction(dq) * Fraction(g["x_absmax"][m]).limit_denominator(100) / 127 \
                * Fraction(g["w_absmax"][n]).limit_denominator(100) / 127
            assert round(float(y), 4) == g["Y_printed"][m][n]


# ---------------------------------------------------------------- FP8 E4M3

def test_lq_fp8_e4m3_examples():
    from oracle import fp8
    g = golden("lq_fp8_e4m3.json")
    c03, c500, c04 = g["cases"]
    code = int(fp8.e4m3_encode(np.float32(c03["x"])))
    assert code == int(c03["bits"], 2)
    v = float(fp8.e4m3_decode(code))
    assert v == c03["value"]
    assert round(abs(v - c03["x"]) / c03["x"] * 100, 1) == c03["rel_err_percent"]
    assert float(fp8.e4m3_decode(fp8.e4m3_encode(c500["x"]))) == c500["value"]
    assert float(fp8.e4m3_decode(fp8.e4m3_encode(np.float32(c04["x"])))) == c04["value"]
    # format limits
    vals = fp8.E4M3_VALUES
    assert np.nanmax(vals) == g["max_finite"] == 1.75 * 2 ** 8
    nan_codes = [c for c in range(256) if np.isnan(vals[c])]
    assert nan_codes == [0x7F, 0xFF]                    # S.1111.111 only, no infinities
    assert np.nanmin(np.abs(vals[vals != 0])) == 2.0 ** -9


def test_lq_symmetric_int4_as_zero8_codes():
    """The symmetric W4 quantizer (codes + 8, z = 8) reproduces the page's
    symmetric INT4 codes on its vector and its GELU row (one group of 8); the
    MSE printed for the GELU row (with the exact scale 3.1/7) holds within the
    fp16 rounding of the stored scale."""
    g = golden("lq_asym_vs_sym.json")
    for key in ("x", "gelu_row"):
        x = np.array(g[key])
        q, s16, z = w4.quantize_w4_sym(x[None, :], group=8)
        s4, qmax = qu.symmetric_params(x, 4)
        assert np.array_equal(q[0].astype(int) - 8, qu.quantize_symmetric(x, s4, qmax).astype(int))
        assert np.all(z == 8) and q.min() >= 1
        deq = w4.dequantize_w4(q, s16, z, group=8)[0]
        assert np.array_equal(deq, float(s16[0, 0]) * (q[0].astype(np.float64) - 8))
    assert abs(qu.mse(deq, x) - g["gelu_sym_int4_mse"]) / g["gelu_sym_int4_mse"] < 0.01


# ---------------------------------------------------------------- RMSNorm + per-token quant

def test_lq_rmsnorm_is_x_over_norm_times_sqrt_d():
    from oracle import rmsnorm as rn
    assert golden("lq_rmsnorm_fold.json")["quarot_norm_of_output"] == "sqrt(d)"
    r = np.random.default_rng(5)
    for d in (4, 37, 4096):
        x = r.standard_normal((3, d))
        y = rn.rms_norm64(x, np.ones(d), 0.0)
        np.testing.assert_allclose(y, x / np.linalg.norm(x, axis=1, keepdims=True) * np.sqrt(d), rtol=1e-13)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.sqrt(d), rtol=1e-13)


def test_lq_awq_gamma_over_s_emits_x_over_s():
    # an RMSNorm whose output is the page's x (gamma = rms(row), eps = 0, row = x);
    # dividing gamma by the AWQ scale s must emit the page's x / s
    from oracle import rmsnorm as rn
    g = golden("lq_rmsnorm_fold.json")
    x = np.array(g["awq_x"], np.float64)
    s = np.array(g["awq_s"], np.float64)
    rms = np.sqrt(np.mean(x * x))
    np.testing.assert_allclose(rn.rms_norm64(x[None], np.full(4, rms), 0.0)[0], x, rtol=1e-14)
    np.testing.assert_allclose(rn.rms_norm64(x[None], rms / s, 0.0)[0], g["awq_x_over_s"], rtol=1e-14)
