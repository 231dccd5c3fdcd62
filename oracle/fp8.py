"""FP8 (E4M3) W8A8 reference (test infrastructure only).

The format ([LQ] "浮点：指数管范围，尾数管精度" (floating point: exponent for
range, mantissa for precision)): E4M3 is the "FN" variant, sign, 4 exponent
bits with bias 7, 3 mantissa bits; there is no infinity, only S.1111.111 is
NaN, so the largest finite value is 1.75 * 2**8 = 448; exponent field 0 holds
the subnormals m * 2**-9.  Conversion rounds to nearest even and saturates
(the page converts 500 to 448).

The W8A8 route ([LQ] "W4A4、FP8 与块缩放格式", its FP8 W8A8 item): instead of
rounding x / s to an int8 code, x / s is converted to E4M3; the FP8 products
are accumulated in FP32 and the epilogue multiplies the two scales; the
scales are per token for activations and per channel for weights ([LQ]
"哪些 scale 能提到求和号外面": scales along T and N only).  The plainest reading
of the scale: the absmax maps to the largest code, s = absmax / 448 (the page
notes FP8 needs a scale to avoid overflow, [QK] §9.8), with the same 1e-5
floor on the range as the int8 paths.

All decisions that produce a code are taken in IEEE fp32 (x / s with true
division), then the fp32 value is rounded once to E4M3.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def _e4m3_value_table():
    """The 256 code values (NaN for S.1111.111)."""
    v = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            v[c] = np.nan
        elif e == 0:
            v[c] = s * m * 2.0 ** -9
        else:
            v[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


E4M3_VALUES = _e4m3_value_table()


def e4m3_decode(codes):
    """Code bytes -> float64 values."""
    return E4M3_VALUES[np.asarray(codes, np.uint8)]


def e4m3_encode(x):
    """Round float values to E4M3 codes: nearest, ties to the even mantissa,
    magnitudes from 448 up saturate to +-448, NaN gives the NaN code.

    Works from the exact input value (float32 or float64): the quantum of a
    magnitude a is 2**(E - 4) for a in [2**(E-1), 2**E) at or above the
    smallest normal 2**-6, and 2**-9 below it.
    """
    x = np.asarray(x, np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    _, E = np.frexp(a)                       # a = f * 2**E, 0.5 <= f < 1 (E = 0 for a = 0)
    q_exp = np.where(a >= 2.0 ** -6, E - 4, -9)
    r = np.rint(np.ldexp(a, -q_exp))         # ties to even on the integer significand grid
    val = np.ldexp(r, q_exp)
    val = np.minimum(val, E4M3_MAX)
    val = np.where(a >= E4M3_MAX, E4M3_MAX, val)
    # encode the (representable) value
    _, E2 = np.frexp(val)
    normal = val >= 2.0 ** -6
    e_field = np.where(normal, E2 - 1 + 7, 0)
    m_field = np.where(normal, np.rint(np.ldexp(val, -(E2 - 1)) * 8 - 8), np.rint(val * 2.0 ** 9))
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = code.astype(np.uint8) | sign
    return np.where(nan, np.uint8(E4M3_NAN) | sign, code).astype(np.uint8)


def quant_per_token_fp8(X):
    """Dynamic per-token FP8 activations, fp32 arithmetic:
    s_a = max(max_k |x|, 1e-5) / 448,  A_hat = e4m3(x / s_a).
    X: float values [M, K].  Returns (A_hat uint8 codes [M, K], s_a float32 [M])."""
    X = np.asarray(X, np.float32)
    amax = np.maximum(np.abs(X).max(axis=1), np.float32(1e-5))
    s_a = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode((X / s_a[:, None]).astype(np.float32)), s_a


def quant_weight_per_channel_fp8(W):
    """Per-output-channel FP8 weights, fp32 arithmetic:
    s_b[n] = max(max_k |W[n, k]|, 1e-5) / 448,  B_hat = e4m3(W / s_b).
    W: [N, K].  Returns (B_hat uint8 codes [N, K], s_b float32 [N])."""
    return quant_per_token_fp8(W)


def fp8_gemm(Aq, Bq):
    """D[m, n] = sum_k e4m3(A_hat[m, k]) * e4m3(B_hat[n, k]) in fp64.

    Exact: every product is a multiple of 2**-18 below 2**18, so the sum of K
    such terms needs fewer than 36 + log2(K) bits, within fp64's 53 for
    K < 2**17."""
    A = e4m3_decode(Aq)
    B = e4m3_decode(Bq)
    if A.shape[1] >= 2 ** 17:
        raise OverflowError("K too large for an exact fp64 sum")
    return A @ B.T


def fp8_linear(Aq, Bq, s_a, s_b, bias=None):
    """out64[m, n] = s_a[m] * s_b[n] * D[m, n] + bias[n] (fp64)."""
    D = fp8_gemm(Aq, Bq)
    M, N = D.shape
    sa = np.broadcast_to(np.asarray(s_a, np.float64).reshape(-1, 1), (M, 1))
    sb = np.broadcast_to(np.asarray(s_b, np.float64).reshape(1, -1), (1, N))
    out = sa * sb * D
    if bias is not None:
        out = out + np.asarray(bias, np.float64)[None, :]
    return out
