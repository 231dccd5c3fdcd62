"""W8A8 reference: int8 x int8 -> exact integer product, then the scaled
epilogue (test infrastructure only).

Algebra ([VE] "二、底层线性代数推导" (the underlying linear algebra) and
"2.4 ScaledEpilogueAzpPerToken"; [LQ] "W8A8：整数矩阵乘 + 反量化 epilogue"):

    A = s_a * (A_hat - z_a)   (per token: one s_a and one z_a per row m)
    B = s_b * B_hat           (symmetric, per output channel n)
    out[m, n] = s_a[m] * s_b[n] * (Dq[m, n] - z_a[m] * azp_adj[n]) + bias[n]
    Dq = A_hat · B_hatᵀ (int32 in the kernel),  azp_adj[n] = sum_k B_hat[n, k]

Here Dq is computed as an fp64 product of integer values, which is exact:
every partial sum is bounded by 128 * 127 * K < 2**53 for any K below 5e11.
The zero-point correction is done in exact int64.
"""

import numpy as np

from .numerics import rne


def quant_weight_per_channel_sym(W):
    """Symmetric per-output-channel int8 weights, fp32 arithmetic ([LQ]
    "对称与非对称": s = max|w| / 127, codes in [-127, 127]; [LQ] W8A8 section:
    per-channel weights, its worked example s_w1 = 1.1/127; [VE] "一、背景":
    weights are symmetric only).

    s_b[n] = max(max_k |W[n, k]|, 1e-5) / 127;   B_hat = clamp(round(W / s_b), -127, 127)
    (the 1e-5 floor only keeps an all-zero row from dividing by zero).
    W: [N, K].  Returns (B_hat int8 [N, K], s_b float32 [N]).
    """
    W = np.asarray(W, np.float32)
    amax = np.maximum(np.abs(W).max(axis=1), np.float32(1e-5))
    s_b = amax / np.float32(127)
    Bq = np.clip(rne(W / s_b[:, None]), -127, 127)
    return Bq.astype(np.int8), s_b.astype(np.float32)


def azp_adj(Bq):
    """azp_adj[n] = sum_k B_hat[n, k] ([VE] "二": every row of J_a·B_hat is the
    row vector 1·B_hat, the column sums of B_hat when B_hat is laid out
    [K, N]; [VE] "五、azp_adj 的离线预计算": computed once at weight load).

    Bq: int8 [N, K] (the [N][K] rows are B_hat's columns).  Returns int32 [N];
    raises if a sum does not fit int32.
    """
    s = np.asarray(Bq, np.int64).sum(axis=1)
    if np.any(np.abs(s) >= 2 ** 31):
        raise OverflowError("azp_adj does not fit int32")
    return s.astype(np.int32)


def quant_per_token_asym(X):
    """Dynamic per-token asymmetric int8 activations, fp32 arithmetic.

    Per row m ([LQ] "线性量化" for (s, z) from a range; [LQ] "校准：静态与动态"
    (static vs dynamic calibration): dynamic per-token ranges at run time; int8
    range [-128, 127] from [QK] §9.2; [VE] "4.1": azp is int32, one per row):

        mn = min(min_k x, 0)     mx = max(max_k x, 0)
        s_a = max(mx - mn, 1e-5) / 255
        azp = -128 - round(mn / s_a)                       (int32, in [-128, 127])
        A_hat = clamp(round(x / s_a) + azp, -128, 127)

    so the row minimum maps to code -128 and real 0 is exact.
    X: float values [M, K] (fp16 or bf16 values).  Returns
    (A_hat int8 [M, K], s_a float32 [M], azp int32 [M]).
    """
    X = np.asarray(X, np.float32)
    mn = np.minimum(X.min(axis=1), np.float32(0))
    mx = np.maximum(X.max(axis=1), np.float32(0))
    s_a = np.maximum(mx - mn, np.float32(1e-5)) / np.float32(255)
    azp = np.float32(-128) - rne(mn / s_a)
    Aq = np.clip(rne(X / s_a[:, None]) + azp[:, None], -128, 127)
    return Aq.astype(np.int8), s_a.astype(np.float32), azp.astype(np.int32)


def quant_per_token_sym(X):
    """Dynamic per-token symmetric int8 activations (z = 0), fp32 arithmetic:
    s_a = max(max_k |x|, 1e-5) / 127, A_hat = clamp(round(x / s_a), -127, 127)
    ([LQ] "对称与非对称"; [LQ] W8A8 worked example: s_x1 = 1.2/127)."""
    X = np.asarray(X, np.float32)
    amax = np.maximum(np.abs(X).max(axis=1), np.float32(1e-5))
    s_a = amax / np.float32(127)
    Aq = np.clip(rne(X / s_a[:, None]), -127, 127)
    return Aq.astype(np.int8), s_a.astype(np.float32)


def int_gemm(Aq, Bq):
    """Dq[m, n] = sum_k A_hat[m, k] * B_hat[n, k], exact (int64 result).

    [LQ] W8A8 section: int8 multiply with int32 accumulation (127**2 * 4096 is
    about 6.6e7, past int16).  The product is an fp64 BLAS call on integer
    values; it is exact because all partial sums stay below 2**53.
    """
    A = np.asarray(Aq, np.float64)
    B = np.asarray(Bq, np.float64)
    if A.shape[1] and 128.0 * 128.0 * A.shape[1] >= 2.0 ** 53:
        raise OverflowError("K too large for an exact fp64 integer product")
    return (A @ B.T).astype(np.int64)


def corrected_accumulator(Dq, azp=None, azp_adj_v=None):
    """C = Dq - azp[m] * azp_adj[n] in exact int64 ([VE] "2.4": the rank-1
    zero-point correction).  Per-tensor form ([VE] "2.3"): azp None and
    azp_adj_v already holding z_a * (1·B_hat), so C = Dq - azp_adj[n].
    Symmetric ([VE] "2.1"/"2.2"): both None, C = Dq."""
    C = np.asarray(Dq, np.int64).copy()
    if azp is not None:
        if azp_adj_v is None:
            raise ValueError("per-token azp needs azp_adj")
        C -= np.asarray(azp, np.int64)[:, None] * np.asarray(azp_adj_v, np.int64)[None, :]
    elif azp_adj_v is not None:
        C -= np.asarray(azp_adj_v, np.int64)[None, :]
    return C


def epilogue(C, s_a, s_b, bias=None):
    """out64[m, n] = s_a[m] * s_b[n] * C[m, n] + bias[n] in fp64 ([VE] "2.4").

    s_a may hold 1 value (per tensor) or M (per token); s_b 1 or N; bias None
    means 0 ([VE] "一": without a bias the kernel adds 0).
    """
    C = np.asarray(C, np.float64)
    M, N = C.shape
    sa = np.broadcast_to(np.asarray(s_a, np.float64).reshape(-1, 1), (M, 1)) \
        if np.size(s_a) in (1, M) else None
    sb = np.broadcast_to(np.asarray(s_b, np.float64).reshape(1, -1), (1, N)) \
        if np.size(s_b) in (1, N) else None
    if sa is None or sb is None:
        raise ValueError("s_a must hold 1 or M values, s_b 1 or N values")
    out = sa * sb * C
    if bias is not None:
        out = out + np.asarray(bias, np.float64)[None, :]
    return out


def w8a8_linear(Aq, Bq, s_a, s_b, azp=None, azp_adj_v=None, bias=None):
    """Whole W8A8 forward on already-quantized operands: returns (C int64, out64 float64)."""
    Dq = int_gemm(Aq, Bq)
    C = corrected_accumulator(Dq, azp, azp_adj_v)
    if np.any(np.abs(C) >= 2 ** 31):
        raise OverflowError("corrected accumulator does not fit int32")
    return C, epilogue(C, s_a, s_b, bias)
