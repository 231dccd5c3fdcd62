"""W4A16 parity on the GPU: q4_gemm (decode kernel for M <= 16, MFMA GEMM
above) against the oracle's explicit-dequant fp64 product.

Two bars on every checked element.  The task's gate:
max|Y_dev - Y64| / max|Y64| <= 1e-2 (Y64 = the oracle's fp64 result before
rounding to the 16-bit output type).  And an element-wise bound from the
arithmetic of the kernel that ran (tests/rounding_bound.py: one rounding at
the store plus the rounding-error model of the fp32 accumulation), about ten
times tighter than the gate, so that a result missing a k-chunk or a single
large product fails.  The achieved errors are appended to the JSON-lines
file named by QL_PARITY_LOG when it is set.  Expected values are always the
oracle's own (its own quantization of the same seeded fp32 weights); the
device side quantizes with the library's host function, which is bit-exact
with the oracle (tests/test_abi.py).  Layers too big for a full fp64 product
are checked on sampled output channels and rows, which the oracle computes
one by one.
"""

import json
import os

import numpy as np
import pytest
import torch

import quantized_linear_layers_amd as ql
import workloads as wl
from oracle import w4a16 as ow4
from tests import rounding_bound as rb

pytestmark = pytest.mark.gpu
TOL = 1e-2

_layers = {}


def device_layer(W):
    key = (W.shape, float(W[0, 0]), float(W[-1, -1]))
    if key not in _layers:
        N, K = W.shape
        wq, s, z = ql.q4_quantize_host(torch.from_numpy(W))
        _layers[key] = ql.q4_pack(wq, s, z, N, K, device="cuda")
    return _layers[key]


def rel_err(Yd, Y64):
    return float(np.abs(Yd - Y64).max() / max(np.abs(Y64).max(), 1e-30))


def dtype_name(t):
    return "bf16" if t == torch.bfloat16 else "f16"


def log_parity(**rec):
    path = os.environ.get("QL_PARITY_LOG")
    if path:
        rec["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def assert_parity(Yd, Y64, X64, q, s, z, dtype, M_total, tol=TOL):
    """The gate and the element-wise bound on one block of outputs; returns the
    gate's relative error."""
    assert np.all(np.isfinite(Yd))
    e = rel_err(Yd, Y64)
    b = rb.w4a16_bound(X64, q, s, z, Y64, dtype, M_total)
    ratio = np.abs(Yd - Y64) / b
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    log_parity(M=int(M_total), K=int(X64.shape[1]), dtype=dtype, kernel="gemv" if M_total <= 16 else "gemm",
               elements=int(Yd.size), rel_err=e, max_abs_err=float(np.abs(Yd - Y64).max()),
               max_err_over_bound=float(ratio.max()), median_bound_over_maxabs=float(np.median(b) / np.abs(Y64).max()))
    assert e <= tol, f"relative error {e:.3e}"
    assert ratio.max() <= 1.0, (f"element {worst}: |err| {abs(Yd[worst] - Y64[worst]):.3e} exceeds the rounding bound "
                                f"{b[worst]:.3e} (Y64 {Y64[worst]:.4e})")
    return e


def run_unsplit(X, blob, N):
    """q4_gemm without a workspace (the plan that does not split K)."""
    Xd = X.cuda()
    M, K = X.shape
    Y = torch.full((M, N), float("nan"), dtype=X.dtype, device="cuda")
    ql.launcher("q4_gemm", Xd, X.dtype, M, K, N, blob, blob.numel(), 128, Y, None, 0)()
    return Y


def check(W, X, rows=None, cols=None, tol=TOL, workspace=True):
    """Run the device layer on X (with a workspace when its plan needs one, or
    without) and compare the (rows, cols) block with the oracle."""
    N, K = W.shape
    blob = device_layer(W)
    Y = ql.q4_gemm(X.cuda(), blob, N) if workspace else run_unsplit(X, blob, N)
    torch.cuda.synchronize()
    Yd = wl.as_f64(Y.cpu())
    rows = np.arange(X.shape[0]) if rows is None else rows
    cols = np.arange(N) if cols is None else cols
    q, s, z = ow4.quantize_w4(W[cols])
    X64 = wl.as_f64(X)[rows]
    Y64 = ow4.w4a16_linear(X64, q, s, z)
    return assert_parity(Yd[np.ix_(rows, cols)], Y64, X64, q, s, z, dtype_name(X.dtype), X.shape[0], tol)


# ---------------------------------------------------------------- the workloads

def test_tiny_gemv():
    w = wl.WORKLOADS["tiny_gemv"]
    W = wl.weight(w, 256, 256)
    X = wl.activations(w, 1, 256, 256)
    check(W, X)


@pytest.mark.parametrize("K,N", wl.WORKLOADS["decode_7b"].shapes)
@pytest.mark.parametrize("M", wl.WORKLOADS["decode_7b"].Ms)
def test_decode_7b(M, K, N):
    w = wl.WORKLOADS["decode_7b"]
    check(wl.weight(w, K, N), wl.activations(w, M, K, N))


@pytest.mark.parametrize("K,N", wl.WORKLOADS["decode_70b"].shapes)
@pytest.mark.parametrize("M", wl.WORKLOADS["decode_70b"].Ms)
def test_decode_70b_sampled(M, K, N):
    w = wl.WORKLOADS["decode_70b"]
    W = wl.weight(w, K, N)
    cols = np.sort(np.random.default_rng(K + N + M).choice(N, 384, replace=False))
    check(W, wl.activations(w, M, K, N), cols=cols)


@pytest.mark.parametrize("M,K,N", [(8, 8192, 8192), (1, 28672, 8192)])
def test_decode_70b_full(M, K, N):
    """Two 70B cases on every output channel."""
    w = wl.WORKLOADS["decode_70b"]
    check(wl.weight(w, K, N), wl.activations(w, M, K, N))


@pytest.mark.parametrize("K,N", wl.WORKLOADS["mid_m_7b"].shapes)
@pytest.mark.parametrize("M", wl.WORKLOADS["mid_m_7b"].Ms)
def test_mid_m_7b(M, K, N):
    w = wl.WORKLOADS["mid_m_7b"]
    check(wl.weight(w, K, N), wl.activations(w, M, K, N))


# shapes whose token and channel counts select the tiles of the large-M kernel
# (32 x 32, 32 x 64, 64 x 64, 64 x 128, 128 x 128: the K range split among
# 8, 4, 4, 2, 2 K-groups of waves, with uneven and empty runs for K = 1152
# and 384); 256 x 256 is the prefill test
@pytest.mark.parametrize("M,K,N,dtype", [(200, 1152, 1000, torch.float16), (77, 384, 4160, torch.bfloat16),
                                         (256, 1152, 4096, torch.float16), (300, 2560, 4000, torch.bfloat16),
                                         (512, 1152, 8192, torch.bfloat16), (400, 384, 8000, torch.float16)])
def test_gemm_tiles(M, K, N, dtype):
    r = np.random.default_rng(M + K + N)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    cols = np.sort(r.choice(N, min(N, 512), replace=False))
    check(W, X, cols=cols, workspace=False)
    check(W, X, cols=cols)


# shapes that select the two non-square tiles (32 x 64 with the K range split
# among 4 K-groups, 64 x 128 among 2): ragged M, N and K, uneven K-group runs;
# every column of the last (partial) column tile is checked, plus a sample
@pytest.mark.parametrize("M,K,N,dtype,tile", [
    (17, 128, 72, torch.float16, (32, 64)), (33, 1152, 4160, torch.bfloat16, (32, 64)),
    (40, 128, 1000, torch.float16, (32, 64)), (17, 4224, 11000, torch.bfloat16, (32, 64)),
    (70, 2560, 11000, torch.float16, (64, 128)), (100, 6016, 8200, torch.bfloat16, (64, 128)),
    (127, 128, 4160, torch.float16, (64, 128)), (33, 128, 8200, torch.bfloat16, (64, 128))])
def test_nonsquare_tiles(M, K, N, dtype, tile):
    assert ql.q4_gemm_tile_shape(M, N, K, with_workspace=False) == tile
    r = np.random.default_rng(M * 7 + K + N)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    tail = np.arange(max(0, N - 200), N)
    cols = np.union1d(np.sort(r.choice(N, min(N, 384), replace=False)), tail)
    check(W, X, cols=cols, workspace=False)
    check(W, X, cols=cols)


# shapes that select the 128 x 256 tile (8 waves of 128 rows x 32 columns,
# planned for 129 to 512 tokens): with and without a K split, ragged M, N
# and K, uneven splits; every column of the last column tile is checked
@pytest.mark.parametrize("M,K,N,dtype,plan_ws,plan_nows", [
    (300, 1152, 11000, torch.bfloat16, (128, 256, 1), (128, 256, 1)),
    (130, 9088, 6000, torch.float16, (128, 256, 4), (32, 64, 1)),
    (193, 9088, 16400, torch.bfloat16, (128, 256, 3), (128, 256, 1))])
def test_tile_128x256(M, K, N, dtype, plan_ws, plan_nows):
    assert ql.q4_gemm_plan(M, N, K) == plan_ws
    assert ql.q4_gemm_plan(M, N, K, False) == plan_nows
    r = np.random.default_rng(M * 3 + K + N)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    cols = np.union1d(np.sort(r.choice(N, 384, replace=False)), np.arange(N - (N % 256 or 256), N))
    check(W, X, cols=cols)
    check(W, X, cols=cols, workspace=False)


# shapes whose plan splits K across workgroups (fp32 partials in the
# workspace, then the reduce pass): the 7B/70B mid-M layers the plan splits,
# and ragged M, N and K with uneven splits and empty K-group runs; each also
# runs without a workspace (the unsplit plan) and both are checked
@pytest.mark.parametrize("M,K,N,dtype", [(32, 11008, 4096, torch.float16), (128, 11008, 4096, torch.float16),
                                         (64, 28672, 8192, torch.bfloat16), (17, 11008, 4096, torch.bfloat16),
                                         (40, 11008, 1000, torch.float16), (77, 5248, 700, torch.bfloat16),
                                         (100, 5248, 500, torch.float16), (130, 6016, 1000, torch.bfloat16),
                                         (130, 9088, 3000, torch.float16), (200, 9088, 2000, torch.bfloat16)])
def test_split_k(M, K, N, dtype):
    rows, cols, S = ql.q4_gemm_plan(M, N, K)
    assert S > 1, (M, K, N, rows, cols)
    r = np.random.default_rng(M + K + N)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    cols_ = np.union1d(np.sort(r.choice(N, min(N, 384), replace=False)), np.arange(max(0, N - 100), N))
    check(W, X, cols=cols_)
    check(W, X, cols=cols_, workspace=False)      # the unsplit plan of the same layer


def test_split_k_workspace_contents_do_not_matter():
    """A workspace full of garbage (NaN bit patterns) gives the same result as
    a fresh one: every partial is written before the reduce pass reads it."""
    M, K, N = 32, 11008, 4096
    w = wl.WORKLOADS["mid_m_7b"]
    W = wl.weight(w, K, N)
    X = wl.activations(w, M, K, N).cuda()
    blob = device_layer(W)
    need = ql.q4_gemm_workspace_bytes(M, N, K)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Y1 = ql.q4_gemm(X, blob, N, workspace=ws)
    ws.fill_(0xFF)
    Y2 = ql.q4_gemm(X, blob, N, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_prefill_sampled():
    w = wl.WORKLOADS["w4a16_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    W = wl.weight(w, K, N)
    r = np.random.default_rng(3)
    rows = np.sort(r.choice(M, 96, replace=False))
    cols = np.sort(r.choice(N, 256, replace=False))
    check(W, wl.activations(w, M, K, N), rows=rows, cols=cols)


@pytest.mark.parametrize("M,K,N,dtype", [(1100, 256, 13400, torch.float16), (700, 384, 26000, torch.bfloat16)])
def test_prefill_split_round(M, K, N, dtype):
    """Grids of 256 x 256 tiles whose last round is at most half full: the
    columns of that round run as 128 x 256 tiles in a second launch (ragged
    rows and columns on both sides).  Every column past the split, the 64
    before it and a sample of the rest are checked on every row."""
    tm, tn = (M + 255) // 256, (N + 255) // 256
    rounds = (tm * tn + 255) // 256
    n_off = ((rounds - 1) * 256 // tm) * 256
    assert rounds >= 2 and 2 * (tm * tn - (rounds - 1) * 256) <= 256 and n_off < N
    r = np.random.default_rng(M + N)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    cols = np.union1d(np.arange(n_off - 64, N), r.choice(n_off, 192, replace=False))
    check(W, X, cols=cols)


# ---------------------------------------------------------------- ragged shapes and edges

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13, 16, 17, 24, 32, 33, 40, 48, 49, 64, 65, 130])
@pytest.mark.parametrize("K,N", [(128, 72), (384, 200), (1152, 1000), (2560, 64)])
def test_ragged(M, K, N, dtype):
    r = np.random.default_rng(M * 1000 + K + N)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    check(W, X)


def test_repeat_call_and_zero_input():
    """Two calls in a row give identical results, and an all-zero activation
    gives exactly zero."""
    w = wl.WORKLOADS["decode_7b"]
    W = wl.weight(w, 4096, 11008)
    X = wl.activations(w, 4, 4096, 11008)
    e1 = check(W, X)
    e2 = check(W, X)
    assert e1 == e2
    blob = device_layer(W)
    Y = ql.q4_gemm(torch.zeros((3, 4096), dtype=torch.float16, device="cuda"), blob, 11008)
    assert torch.count_nonzero(Y).item() == 0


def test_large_activation_values():
    """Outlier-heavy bf16 activations (values up to ~1e4) stay within the bar."""
    r = np.random.default_rng(99)
    W = (r.standard_normal((512, 1024)) * 0.02).astype(np.float32)
    Xf = r.standard_normal((4, 1024)).astype(np.float32)
    Xf[:, ::97] *= 5000.0
    check(W, torch.from_numpy(Xf).to(torch.bfloat16))


def test_alternating_shapes_are_deterministic():
    """Layers of different tile counts called alternately give bit-identical
    results on every repetition (no state carried between calls)."""
    r = np.random.default_rng(17)
    shapes = [(4096, 11008), (8192, 4096), (2048, 640)]
    Ws = [(r.standard_normal((N, K)) * 0.02).astype(np.float32) for (K, N) in shapes]
    Xs = [torch.from_numpy(r.standard_normal((2, K)).astype(np.float32)).half() for (K, _) in shapes]
    first = []
    for rep in range(3):
        for i, (W, X) in enumerate(zip(Ws, Xs)):
            e = check(W, X)
            if rep == 0:
                first.append(e)
            else:
                assert e == first[i]


# ---------------------------------------------------------------- symmetric codes (zero point 8)

@pytest.mark.parametrize("M,K,N,dtype", [(1, 4096, 4096, torch.float16), (16, 11008, 4096, torch.float16),
                                         (8, 8192, 1024, torch.bfloat16), (300, 1024, 520, torch.bfloat16)])
def test_symmetric_codes(M, K, N, dtype):
    """Blobs from q4_quantize_sym_host + q4_pack(zeros=None) through both
    kernels (decode for M <= 16, GEMM above) against the oracle's symmetric
    quantizer and explicit-dequant product."""
    w = wl.WORKLOADS["decode_7b"]
    W = wl.weight(w, K, N)
    wq, s = ql.q4_quantize_sym_host(torch.from_numpy(W))
    blob = ql.q4_pack(wq, s, None, N, K, device="cuda")
    r = np.random.default_rng(M + K)
    X = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).to(dtype)
    Y = ql.q4_gemm(X.cuda(), blob, N)
    torch.cuda.synchronize()
    q, s_o, z = ow4.quantize_w4_sym(W)
    Y64 = ow4.w4a16_linear(wl.as_f64(X), q, s_o, z)
    assert_parity(wl.as_f64(Y.cpu()), Y64, wl.as_f64(X), q, s_o, z, dtype_name(dtype), M)


# ---------------------------------------------------------------- act-order (g_idx)

def _act_order_layer(K, N, seed):
    r = np.random.default_rng(seed)
    W = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
    order = np.argsort(-(r.standard_normal(K) ** 2), kind="stable")   # decreasing stand-in energy
    return W, ow4.g_idx_from_order(order).astype(np.int32)


@pytest.mark.parametrize("M,K,N,dtype", [(1, 4096, 4096, torch.float16), (5, 1152, 1000, torch.bfloat16),
                                         (16, 4096, 11008, torch.float16), (64, 2560, 640, torch.bfloat16),
                                         (300, 1024, 768, torch.float16)])
def test_act_order(M, K, N, dtype):
    W, g = _act_order_layer(K, N, M + K + N)
    wq, s, z = ql.q4_quantize_act_order_host(torch.from_numpy(W), torch.from_numpy(g))
    blob, perm = ql.q4_pack_act_order(wq, s, z, torch.from_numpy(g), N, K, device="cuda")
    X = torch.from_numpy(np.random.default_rng(M).standard_normal((M, K)).astype(np.float32)).to(dtype)
    Xd = X.cuda()
    Xp = ql.q4_permute_columns(Xd, perm)
    Y = ql.q4_gemm_act_order(Xd, blob, perm, N)
    torch.cuda.synchronize()
    # the permutation is a pure gather: bit-exact
    assert torch.equal(Xp.cpu(), X[:, torch.from_numpy(perm.cpu().numpy().astype(np.int64))])
    q, s_o, z_o = ow4.quantize_w4_act_order(W, g)
    Y64 = ow4.w4a16_linear_gidx(wl.as_f64(X), q, s_o, z_o, g)
    # the device multiplies in processing order (group by group, ascending
    # channels inside a group): the bound is that of the permuted layer
    order = np.argsort(g, kind="stable")
    assert_parity(wl.as_f64(Y.cpu()), Y64, wl.as_f64(X)[:, order], q[:, order], s_o, z_o, dtype_name(dtype), M)
