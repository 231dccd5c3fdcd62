"""Rounding primitives of the oracle (test infrastructure only).

[LQ] states in its notation paragraph (the opening section, where Y = X·Wᵀ is
fixed) that its worked examples use round-half-to-even; [LQ] "浮点：指数管范围，
尾数管精度" (floating point: exponent for range, mantissa for precision) works
1/3 and 70000 through fp16 and bf16 with round-to-nearest-even.  Those are
the only rounding rules used here.
"""

import numpy as np


def rne(x):
    """Round half to even, elementwise (``np.rint`` is IEEE round-to-nearest-even)."""
    return np.rint(x)


def to_f16(x):
    """Round to IEEE binary16, nearest-even, straight from the input precision.

    NumPy converts float64 and float32 to float16 with one correct rounding;
    values beyond the fp16 range become +-inf ([LQ] floating-point section:
    70000 overflows fp16).
    """
    with np.errstate(over="ignore"):
        return np.asarray(x).astype(np.float16)


def f16_bits(x_f16):
    return np.asarray(x_f16, np.float16).view(np.uint16)


def f16_from_bits(bits):
    return np.asarray(bits, np.uint16).view(np.float16)


def to_bf16(x):
    """Round to bfloat16 (8 significant bits, fp32 exponent range), nearest-even.

    Returned as float64 values that are exactly representable in bf16.  The
    rounding is done once, from the input's own precision (no detour through
    fp32, which could round twice): the significand from ``frexp`` lies in
    [0.5, 1), so scaling it by 2**8 and rounding half-to-even keeps exactly 8
    significant bits.  Magnitudes that round above the largest finite bf16
    become inf; bf16 subnormals (below 2**-126) are rounded on the subnormal
    grid of spacing 2**-133.
    """
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    m, e = np.frexp(xf)               # xf = m * 2**e, 0.5 <= |m| < 1
    # the smallest normal bf16 is 2**-126 = 0.5 * 2**-125: below it the grid is fixed
    e = np.maximum(e, -125)
    r = rne(np.ldexp(xf, 8 - e))      # integer number of ulps, |r| <= 2**8
    y = np.ldexp(r, e - 8)
    max_bf16 = float(np.ldexp(255.0, 127 - 7))   # (2 - 2**-7) * 2**127
    y = np.where(np.abs(y) > max_bf16, np.copysign(np.inf, y), y)
    out[finite] = y
    return out


def bf16_bits(x_bf16_values):
    """Bit pattern of values that are already exact bf16 numbers."""
    f = np.asarray(x_bf16_values, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to(dtype, x):
    """Round fp64 values to the named 16-bit float type ('f16' or 'bf16');
    returns float64 values on that type's grid."""
    if dtype == "f16":
        return to_f16(x).astype(np.float64)
    if dtype == "bf16":
        return to_bf16(x)
    raise ValueError(dtype)


def signed_nibble(n):
    """Two's-complement reading of a 4-bit code ([LQ] "整数：等间隔的码点"
    (integers: evenly spaced code points): 1101 is -3 signed, 13 unsigned)."""
    n = np.asarray(n, np.int64) & 0xF
    return np.where(n >= 8, n - 16, n)
