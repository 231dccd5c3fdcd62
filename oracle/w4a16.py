"""W4A16 reference: per-group asymmetric uint4 weights, 16-bit activations
(test infrastructure only).

What the path computes ([QK] §9.5 "关键 Kernel: Dequant + GEMM"; [LQ] "W4A16：
权重在寄存器里'现场解压'" (W4A16: weights decompressed in registers)):

    Y[m, n] = sum_k X[m, k] * s[g(k), n] * (q[n, k] - z[g(k), n]),   g(k) = k // group

The fused kernel must equal "dequantize W explicitly, then multiply"; this
module is that plain definition: explicit dequant to fp64 (exact, since
s * (q - z) with an fp16 s and |q - z| <= 15 has at most 15 significant bits)
and an fp64 BLAS product.

Shapes follow [LQ]'s notation paragraph: X is [T, K] (tokens x input
channels), W is [N, K] (nn.Linear.weight), Y = X·Wᵀ is [T, N].
"""

import numpy as np

from .numerics import rne, to_f16

GROUP = 128


def quantize_w4(W, group=GROUP):
    """Per-group asymmetric round-to-nearest quantization to uint4.

    For each output channel n and each run of ``group`` consecutive input
    channels (one group g), in IEEE fp32 ([QK] §9.3 "量化方案的粒度" and [LQ]
    "粒度" (granularity): per-group along K, g = 128; [LQ] "对称与非对称":
    asymmetric uint4 codes 0..15; the range-to-(s, z) rule of [LQ]
    "线性量化：一把刻度尺"; the degenerate-range clamp at 1e-5 of the
    ``pseudo_quant`` routine in [LQ]'s AWQ section):

        mn = min(min_k w, 0)        mx = max(max_k w, 0)
        s16 = fp16(max(mx - mn, 1e-5) / 15)           (stored scale, RNE)
        z = clamp(round(-mn / s16), 0, 15)            (stored zero point)
        q = clamp(round(w / s16) + z, 0, 15)

    Readings where the pages are silent: the range is widened to contain 0 so
    that the integer z keeps real 0 on a tick ([LQ] linear-quantization
    section says z is an integer for exactly that reason); the codes are
    computed with the fp16-ROUNDED scale, so that the stored (s, z, q) are
    self-consistent.

    W: float array [N, K] (converted to fp32).  Returns
    q uint8 [N, K], s16 float16 [K/group, N], z uint8 [K/group, N].
    """
    W = np.asarray(W, np.float32)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    Wg = W.reshape(N, G, group)
    mn = np.minimum(Wg.min(axis=2), np.float32(0))         # [N, G]
    mx = np.maximum(Wg.max(axis=2), np.float32(0))
    rng = np.maximum(mx - mn, np.float32(1e-5))
    s16 = to_f16(rng / np.float32(15))                      # fp32 divide, then RNE to fp16
    sf = s16.astype(np.float32)
    z = np.clip(rne(-mn / sf), 0, 15).astype(np.float32)
    q = np.clip(rne(Wg / sf[:, :, None]) + z[:, :, None], 0, 15)
    return (q.reshape(N, K).astype(np.uint8),
            np.ascontiguousarray(s16.T),
            np.ascontiguousarray(z.T.astype(np.uint8)))


def quantize_w4_sym(W, group=GROUP):
    """Per-group symmetric round-to-nearest quantization to 4 bits, stored as
    unsigned codes with the zero point fixed at 8.

    [LQ] "对称与非对称" (symmetric vs asymmetric): z = 0, s = max|x| / q_max with
    q_max = 2**(b-1) - 1 = 7, signed codes -7..7 (the code -8 stays unused);
    [LQ] "整数" and [QK] §9.5's plain decode (code - 8): the signed code is
    stored as the unsigned nibble code + 8, which dequantizes exactly like an
    asymmetric code with z = 8.  Same readings as quantize_w4: fp32
    arithmetic, the codes use the fp16-rounded scale, the range is floored at
    1e-5.

        s16 = fp16(max(max_k |w|, 1e-5) / 7)
        q = clamp(round(w / s16), -7, 7) + 8

    Returns q uint8 [N, K] (1..15), s16 float16 [K/group, N], z uint8
    [K/group, N] (all 8).
    """
    W = np.asarray(W, np.float32)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    G = K // group
    Wg = W.reshape(N, G, group)
    amax = np.maximum(np.abs(Wg).max(axis=2), np.float32(1e-5))
    s16 = to_f16(amax / np.float32(7))
    sf = s16.astype(np.float32)
    q = np.clip(rne(Wg / sf[:, :, None]), -7, 7) + 8
    return (q.reshape(N, K).astype(np.uint8),
            np.ascontiguousarray(s16.T),
            np.full((G, N), 8, np.uint8))


def pack_canonical(q):
    """Canonical int32 packing: 8 codes along K per 32-bit word, code i of a
    word at bits 4i..4i+3, words indexed [k // 8, n] ([LQ] W4A16 section: the
    packed word is sum_i q_i << 4i, [11, 6, 15, 0, 3, 9, 12, 7] -> 0x7C930F6B;
    its tiled pseudocode indexes ``Wpacked[k0//8 ..., n0 ...]``).

    q: uint [N, K] with K % 8 == 0.  Returns uint32 [K/8, N].
    """
    q = np.asarray(q).astype(np.uint32)
    N, K = q.shape
    words = np.zeros((K // 8, N), np.uint32)
    for i in range(8):
        words |= (q[:, i::8].T & np.uint32(0xF)) << np.uint32(4 * i)
    return words


def unpack_canonical(words):
    """Inverse of ``pack_canonical``: shift right by 4i and mask with 0xF."""
    words = np.asarray(words, np.uint32)
    K8, N = words.shape
    q = np.zeros((N, K8 * 8), np.uint8)
    for i in range(8):
        q[:, i::8] = ((words >> np.uint32(4 * i)) & np.uint32(0xF)).T
    return q


def dequantize_w4(q, s16, z, group=GROUP):
    """Explicit dequantization x_hat = s * (q - z) in fp64 ([QK] §9.2;
    [LQ] linear-quantization section).  Returns float64 [N, K]."""
    q = np.asarray(q, np.float64)
    N, K = q.shape
    g_of_k = np.arange(K) // group
    s = np.asarray(s16, np.float64)[g_of_k, :].T           # [N, K]
    zz = np.asarray(z, np.float64)[g_of_k, :].T
    return s * (q - zz)


def w4a16_linear(X, q, s16, z, group=GROUP):
    """Y64 = X · dequant(W)ᵀ in fp64 (the un-fused "dequantize, then GEMM" of
    [QK] §9.5, which the fused kernel must reproduce).

    X: float values [M, K] (already on the fp16/bf16 grid).  Returns float64 [M, N].
    """
    Wd = dequantize_w4(q, s16, z, group)
    return np.asarray(X, np.float64) @ Wd.T


# ---------------------------------------------------------------- act-order (g_idx)

def g_idx_from_order(order, group=GROUP):
    """Group index of every input channel when channels are quantized in the
    given order ([LQ] GPTQ section, "工程细节" (engineering details), its
    act-order item: channels are processed in decreasing activation energy,
    groups are formed along that processing order, and g_idx records the group
    of each input channel).  order: a permutation of range(K); channel
    order[j] lands in group j // group.  Returns int64 [K]."""
    order = np.asarray(order, np.int64)
    K = order.size
    if sorted(order.tolist()) != list(range(K)):
        raise ValueError("order must be a permutation of range(K)")
    g = np.empty(K, np.int64)
    g[order] = np.arange(K) // group
    return g


def quantize_w4_act_order(W, g_idx, group=GROUP):
    """quantize_w4 with the groups given by g_idx instead of consecutive runs
    of K: group j holds the input channels k with g_idx[k] == j, and its
    (s16, z) come from those channels' weights by the same fp32 formulas.

    W: [N, K]; g_idx: int [K] with values 0..K/group-1.  Returns q uint8
    [N, K] (original channel order), s16 float16 [K/group, N], z uint8
    [K/group, N]."""
    W = np.asarray(W, np.float32)
    N, K = W.shape
    g_idx = np.asarray(g_idx, np.int64)
    G = K // group
    q = np.zeros((N, K), np.uint8)
    s16 = np.zeros((G, N), np.float16)
    z = np.zeros((G, N), np.uint8)
    for j in range(G):
        ch = np.nonzero(g_idx == j)[0]
        qj, sj, zj = quantize_w4(W[:, ch], group=len(ch))
        q[:, ch] = qj
        s16[j], z[j] = sj[0], zj[0]
    return q, s16, z


def dequantize_w4_gidx(q, s16, z, g_idx):
    """x_hat[n, k] = s[g_idx[k], n] * (q[n, k] - z[g_idx[k], n]) in fp64 (the
    non-contiguous scale reads the act-order item describes)."""
    g_idx = np.asarray(g_idx, np.int64)
    s = np.asarray(s16, np.float64)[g_idx, :].T
    zz = np.asarray(z, np.float64)[g_idx, :].T
    return s * (np.asarray(q, np.float64) - zz)


def w4a16_linear_gidx(X, q, s16, z, g_idx):
    """Y64 = X · dequant_gidx(W)ᵀ in fp64."""
    return np.asarray(X, np.float64) @ dequantize_w4_gidx(q, s16, z, g_idx).T
