"""Element-wise bounds on the float error of a device W4A16 result, derived
from the arithmetic the kernels perform (test infrastructure, beside the
oracle: it reads the oracle's dequantization inputs and models the rounding
steps of the device's evaluation order, not the method).

Rounding model: [LQ] "误差从哪来：舍入与截断" takes a rounding error to be
uniform on [-step/2, step/2] when the data are spread over many steps; with
independent errors the variance of a sum of roundings is the sum of
step^2 / 12.  Each rounding's step is bounded by the fp32 (or 16-bit) step at
a bound of the value being rounded, so the variance below is an upper bound
on the model's variance.  The element-wise bound is

    |Y_dev - Y64| <= u_out * |Y64| + (1 + u_out) * C_SIGMA * sigma + tiny

where u_out is the unit roundoff of the output type (the single rounding at
the store), sigma the model's standard deviation of the fp32 result before
that store, and C_SIGMA = 8 (a Gaussian leaves 8 sigma with probability
1.2e-15).  `tiny` is half the smallest subnormal of the output type.

Evaluation forms (one per kernel family):

  offset    the decode kernel: per group g of 128 input channels and per
            32-channel step j, one MFMA adds the 32 exact products
            x * (off + q) to the group's running sum, then one MFMA adds the
            32 exact products x * -(off + z) (off = 1024 for fp16 activations,
            128 for bf16, so (off + q) is an exact 16-bit value); the running
            sum starts at 0 for each group; then acc += s_g * t_g (at most two
            roundings) and the partial sums of up to 8 waves are added.  Each
            MFMA is charged 33 roundings, each at the fp32 step of a bound on
            every partial sum inside it: |sum before| + sum of |terms|.
  dequant16 the GEMM: each weight s * (q - z) is rounded once to the 16-bit
            type (a deterministic shift of the result, computed exactly from
            the oracle's weights), products are exact in fp32, each MFMA adds
            16 products (17 roundings), and the partials of up to 8 K-groups
            in a workgroup and of up to 8 K splits across workgroups are
            added at the end.
"""

import numpy as np

U32 = 2.0 ** -24
C_SIGMA = 8.0
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
MANT_BITS = {"f16": 10, "bf16": 7, "f32": 23}
TINY = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}
OFFSET = {"f16": 1024.0, "bf16": 128.0}


def step_of(v, kind):
    """Spacing of the floating-point grid of `kind` at |v| (0 where v == 0;
    normal range only, which the bounds here never leave)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - MANT_BITS[kind]), 0.0)


def _group_abs_sums(X, K, width):
    """S[m, c] = sum of |x| over the c-th run of `width` channels."""
    return np.abs(np.asarray(X, np.float64)).reshape(X.shape[0], K // width, width).sum(axis=2)


def sigma_offset(X, q, s16, z, dtype, group=128, step=32):
    """Model standard deviation [M, N] of the decode kernel's fp32 result."""
    X = np.asarray(X, np.float64)
    M, K = X.shape
    G, J = K // group, group // step
    off = OFFSET[dtype]
    S = _group_abs_sums(X, K, step).reshape(M, G, J)                # sum |x| per step
    # partial-sum bounds of the two MFMAs of step j (|q - z| <= 15, off + q <= off + 15)
    before = 15.0 * np.concatenate([np.zeros((M, G, 1)), np.cumsum(S, axis=2)[:, :, :-1]], axis=2)
    pc = before + (off + 15.0) * S
    pz = before + 2.0 * (off + 15.0) * S
    V = (33.0 / 12.0) * (step_of(pc, "f32") ** 2 + step_of(pz, "f32") ** 2).sum(axis=2)    # [M, G]
    s = np.asarray(s16, np.float64)                                   # [G, N]
    var = V @ (s * s)
    # acc += s_g * t_g over the groups, then the waves' partials: bounded by
    # sum_g s_g * 15 * sum_{k in g} |x_k|
    A = _group_abs_sums(X, K, group) @ (15.0 * s)
    var += (2 * G + 8) * step_of(A, "f32") ** 2 / 12.0
    return np.sqrt(var)


def dequant16_terms(X, Wd, dtype, mfma_k=16):
    """The GEMM's error before the store, as (shift [M, N], sigma [M, N]).

    Wd [N, K] holds the exact dequantized weights s * (q - z).  The kernel
    rounds each of them once to the 16-bit type, which moves the result by
    exactly shift = X . (rne16(Wd) - Wd)^T: a deterministic term (the 31
    values of a group round the same way wherever they occur, so the uniform
    model does not apply to it), computed here exactly.  sigma is the model's
    standard deviation of the fp32 accumulation of the exact products."""
    from oracle import numerics as nu
    X = np.asarray(X, np.float64)
    Wd = np.asarray(Wd, np.float64)
    K = X.shape[1]
    W16 = nu.to_bf16(Wd) if dtype == "bf16" else nu.to_f16(Wd).astype(np.float64)
    shift = X @ (np.asarray(W16, np.float64) - Wd).T
    A = np.abs(X) @ np.abs(np.asarray(W16, np.float64)).T             # bound of every partial sum
    # one rounding per product and per MFMA, then the partial tiles of up to 8
    # K-groups in a workgroup times up to 8 K splits across workgroups
    var = ((K // mfma_k) * (mfma_k + 1) + 64) * step_of(A, "f32") ** 2 / 12.0
    return shift, np.sqrt(var)


def bound(Y64, sigma, dtype, shift=None):
    """Element-wise bound on |Y_dev - Y64| (see the module docstring); shift
    is a deterministic displacement of the fp32 result (the GEMM's weight
    rounding), or None."""
    u = UNIT_ROUNDOFF[dtype]
    if shift is None:
        return u * np.abs(Y64) + (1.0 + u) * C_SIGMA * sigma + TINY[dtype]
    return u * np.abs(Y64 + shift) + (1.0 + u) * (np.abs(shift) + C_SIGMA * sigma) + TINY[dtype]


def w4a16_bound(X, q, s16, z, Y64, dtype, M_total, group=128):
    """Element-wise bound for the kernel q4_gemm runs at M_total tokens: the
    decode kernel for M <= 16, the GEMM above."""
    if M_total <= 16:
        return bound(Y64, sigma_offset(X, q, s16, z, dtype, group), dtype)
    from oracle import w4a16 as ow4
    shift, sig = dequant16_terms(X, ow4.dequantize_w4(q, s16, z, group), dtype)
    return bound(Y64, sig, dtype, shift)
