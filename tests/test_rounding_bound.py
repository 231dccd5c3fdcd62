"""The element-wise rounding bound of the W4A16 parity tests, on the CPU.

It must (a) hold for a result computed in the kernels' own arithmetic (a
NumPy emulation of each evaluation order in fp32, rounded once to the output
type), and (b) reject results the 1e-2 gate accepts: one missing product, or
one missing 32-channel step, in a single output element."""

import numpy as np
import pytest

import workloads as wl
from oracle import numerics as nu
from oracle import w4a16 as ow4
from tests import rounding_bound as rb

GATE = 1e-2


def _layer(wname, M, K, N, ncols=256):
    w = wl.WORKLOADS[wname]
    W = wl.weight(w, K, N)[:ncols]
    X = wl.as_f64(wl.activations(w, M, K, N))
    q, s, z = ow4.quantize_w4(W)
    return X, q, s, z, ow4.w4a16_linear(X, q, s, z)


def _round_out(v, dtype):
    return np.asarray(nu.to_bf16(v) if dtype == "bf16" else nu.to_f16(v), np.float64)


def emulate_offset(X, q, s, z, dtype):
    """The decode kernel's order in fp32: per group and 32-channel step, the
    code products, then the zero-point products; the group sum scaled into
    the accumulator."""
    off = np.float32(rb.OFFSET[dtype])
    x = X.astype(np.float32)
    M, K = x.shape
    N = q.shape[0]
    acc = np.zeros((M, N), np.float32)
    for g in range(K // 128):
        t = np.zeros((M, N), np.float32)
        for j in range(4):
            ks = slice(128 * g + 32 * j, 128 * g + 32 * j + 32)
            t = t + x[:, ks] @ (off + q[:, ks].astype(np.float32)).T
            t = t - np.outer(x[:, ks].sum(axis=1, dtype=np.float32), off + z[g].astype(np.float32))
        acc = acc + s[g].astype(np.float32)[None, :] * t
    return _round_out(acc.astype(np.float64), dtype)


def emulate_dequant16(X, q, s, z, dtype):
    """The GEMM's order: each weight rounded to the 16-bit type, exact
    products summed in fp32."""
    Wd = ow4.dequantize_w4(q, s, z)
    W16 = _round_out(Wd, dtype).astype(np.float32)
    return _round_out((X.astype(np.float32) @ W16.T).astype(np.float64), dtype)


def gate_err(Yd, Y64):
    return np.abs(Yd - Y64).max() / np.abs(Y64).max()


CASES = [("decode_7b", 1, 4096, 4096, "f16", 1), ("decode_7b", 16, 11008, 4096, "f16", 16),
         ("decode_70b", 8, 8192, 8192, "bf16", 8), ("w4a16_prefill", 48, 4096, 14336, "bf16", 4096)]


@pytest.mark.parametrize("wname,M,K,N,dtype,M_total", CASES)
def test_bound_holds_for_the_kernels_arithmetic(wname, M, K, N, dtype, M_total):
    X, q, s, z, Y64 = _layer(wname, M, K, N)
    b = rb.w4a16_bound(X, q, s, z, Y64, dtype, M_total)
    Yd = emulate_offset(X, q, s, z, dtype) if M_total <= 16 else emulate_dequant16(X, q, s, z, dtype)
    assert np.all(np.abs(Yd - Y64) <= b)
    assert np.all(np.abs(_round_out(Y64, dtype) - Y64) <= b)     # the correctly rounded result
    # and the bound is much tighter than the gate
    assert np.median(b) < 0.2 * GATE * np.abs(Y64).max()


@pytest.mark.parametrize("wname,M,K,N,dtype,M_total", CASES)
def test_bound_rejects_a_missing_product_the_gate_accepts(wname, M, K, N, dtype, M_total):
    X, q, s, z, Y64 = _layer(wname, M, K, N)
    b = rb.w4a16_bound(X, q, s, z, Y64, dtype, M_total)
    Yd = _round_out(Y64, dtype)
    Wd = ow4.dequantize_w4(q, s, z)
    terms = np.abs(X[0][None, :] * Wd)                          # products of row 0, [N, K]
    lim = GATE * np.abs(Y64).max()
    caught = (terms > b[0][:, None]) & (terms < lim)
    # a large share of single products: the gate passes them all, the bound none
    assert caught.mean() > 0.2
    n, k = np.argwhere(caught)[len(np.argwhere(caught)) // 2]
    bad = Yd.copy()
    bad[0, n] = _round_out(Y64[0, n] - X[0, k] * Wd[n, k], dtype)
    assert gate_err(bad, Y64) <= GATE
    assert np.abs(bad[0, n] - Y64[0, n]) > b[0, n]


@pytest.mark.parametrize("wname,M,K,N,dtype,M_total", CASES)
def test_bound_rejects_a_missing_step(wname, M, K, N, dtype, M_total):
    X, q, s, z, Y64 = _layer(wname, M, K, N)
    b = rb.w4a16_bound(X, q, s, z, Y64, dtype, M_total)
    Wd = ow4.dequantize_w4(q, s, z)
    j = (K // 32) // 2                                           # one 32-channel step in the middle
    part = X[:, 32 * j:32 * j + 32] @ Wd[:, 32 * j:32 * j + 32].T
    bad = _round_out(Y64 - part, dtype)
    assert np.mean(np.abs(bad - Y64) > b) > 0.5                 # most elements fail the bound
