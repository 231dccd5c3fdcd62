"""RMSNorm followed by dynamic per-token int8 quantization, as one step
(test infrastructure only).

What is computed.  [LQ] "QuaRot：把整个残差流旋转掉" (QuaRot: rotate the whole
residual stream) gives RMSNorm with its gain folded away as x / ||x|| * sqrt(d),
i.e. x divided by the root mean square of the row; the gain gamma multiplies
channel by channel ([LQ] "缩放融合到哪里" (where the scaling is fused): AWQ
divides RMSNorm's gamma by s so the layer norm already emits X / s).  [QK]
§9.9 (engineering points of quantization kernels) and [LQ] "校准：静态与动态"
(static vs dynamic calibration) put the per-token range reduction of W8A8
activations into the RMSNorm kernel.  So, per row m:

    y[k] = x[k] / sqrt(mean_k(x^2) + eps) * gamma[k]
    (A_hat, s_a, azp) = per-token int8 quantization of y      (oracle.w8a8)

Readings where the pages are silent (each listed in the design notes):
  * eps sits inside the square root (the usual RMSNorm), as a caller-given
    fp32 constant;
  * y is not rounded to the 16-bit activation type before it is quantized
    (the fused step has no intermediate tensor);
  * precision: the mean square is the correctly rounded fp64 sum of the
    (exact) squares, divided by K in fp64 and rounded once to fp32;
    everything after it is IEEE fp32 in this order: v = ms + eps,
    r = sqrt(v), inv = 1 / r, y = (x * inv) * gamma.  Both sides take every
    step that decides a code in the same precision, so codes, scales and zero
    points are compared bit for bit.  "Correctly rounded" makes the sum
    independent of the order of the additions: a plain fp64 sum is not, and
    for a row whose mean square sits next to an fp32 rounding boundary two
    orders can give two different fp32 mean squares.

rms_norm64 is the plain definition in fp64, for the pins.
"""

import math

import numpy as np

from . import w8a8


def rms_norm64(X, gamma, eps):
    """y = x / sqrt(mean(x^2) + eps) * gamma per row, all in fp64."""
    X = np.asarray(X, np.float64)
    g = np.asarray(gamma, np.float64)
    ms = np.mean(X * X, axis=1, keepdims=True)
    return X / np.sqrt(ms + float(eps)) * g[None, :]


def mean_square_f32(X):
    """Per row: fp32(fp64(sum_k x^2) / K), the sum taken with math.fsum over
    the squares (each exact in fp64 for 16-bit inputs), so it is the
    correctly rounded fp64 value of the exact sum."""
    X = np.asarray(X, np.float64)
    K = X.shape[1]
    with np.errstate(over="ignore"):         # a mean square beyond the fp32 range becomes inf
        return np.array([math.fsum(r * r) / K for r in X], np.float64).astype(np.float32)


def rms_norm_f32(X, gamma, eps):
    """The fp32 steps above.  X: 16-bit values [M, K] (any float array holding
    them exactly), gamma [K] likewise, eps a float (rounded to fp32).
    Returns y float32 [M, K] and inv float32 [M]."""
    X32 = np.asarray(X, np.float32)
    g32 = np.asarray(gamma, np.float32)
    ms = mean_square_f32(X32)
    v = ms + np.float32(eps)
    inv = np.float32(1) / np.sqrt(v)
    y = (X32 * inv[:, None]) * g32[None, :]
    return y.astype(np.float32), inv.astype(np.float32)


def rmsnorm_quant_per_token(X, gamma, eps, asym=True):
    """RMSNorm then per-token int8 quantization of the fp32 result.
    asym: returns (A_hat int8, s_a fp32, azp int32); else (A_hat, s_a)."""
    y, _ = rms_norm_f32(X, gamma, eps)
    return w8a8.quant_per_token_asym(y) if asym else w8a8.quant_per_token_sym(y)
