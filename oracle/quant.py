"""Generic uniform (affine) quantizers of the oracle (test infrastructure only).

These are the textbook forms the pages build everything else from; the
W4A16 and W8A8 modules specialise them.  Arithmetic is fp64 unless a caller
passes fp32 arrays (NumPy keeps the input precision).

Sign convention ([QK] §9.2 "量化基础"; [LQ] "线性量化：一把刻度尺" (linear
quantization: a ruler)): quantize ADDS the zero point, dequantize SUBTRACTS it:

    q = clamp(round(x / s) + z, qmin, qmax)          x_hat = s * (q - z)
"""

import numpy as np

from .numerics import rne


def affine_params(xmin, xmax, qmin, qmax):
    """Scale and zero point of the ruler that maps [xmin, xmax] onto the
    integer range [qmin, qmax] ([LQ] linear-quantization section: the range is
    cut into (qmax - qmin) equal steps, and z is the integer code that real 0
    lands on, so 0 is exact)."""
    s = (xmax - xmin) / (qmax - qmin)
    z = qmin - rne(xmin / s)
    return s, z


def quantize(x, s, z, qmin, qmax):
    """Round to the nearest tick, shift by z, clip to the code range."""
    return np.clip(rne(x / s) + z, qmin, qmax)


def dequantize(q, s, z):
    return s * (q - z)


def symmetric_params(x, bits):
    """Symmetric (z = 0) scale: s = max|x| / qmax with qmax = 2**(bits-1) - 1
    ([LQ] "对称与非对称" (symmetric vs asymmetric))."""
    qmax = 2 ** (bits - 1) - 1
    return np.max(np.abs(x)) / qmax, qmax


def quantize_symmetric(x, s, qmax, qmin=None):
    """Codes in [-qmax, qmax] by default (the most negative code stays unused,
    [LQ] symmetric section); a caller may widen the low end (``qmin``), as the
    3-bit example of [LQ]'s AWQ section does with [-4, 3]."""
    lo = -qmax if qmin is None else qmin
    return np.clip(rne(x / s), lo, qmax)


def mse(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.mean((a - b) ** 2))
