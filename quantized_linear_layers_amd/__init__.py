"""Python binding of libqlinear.so (the MI355X quantized linear layer).

Argument marshalling only: every function here checks tensor dtypes, devices
and shapes, allocates outputs with torch (device memory is torch's), and calls
the C ABI function of the same name in ``include/qlinear.h``.  All arithmetic
happens in the library (host C++ for the offline steps, HIP kernels for the
forward).  There is no fallback: if the library is not built, importing works
but every call raises.
"""

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlinear.so")

QL_F16, QL_BF16 = 0, 1
GROUP = 128
ABI_VERSION = 2

_lib = None


class QLError(RuntimeError):
    pass


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QLError(f"{LIB_PATH} is missing: build it with `python -m quantized_linear_layers_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I, Z = C.c_void_p, C.c_int, C.c_size_t
        sig = {
            "ql_last_error": (C.c_char_p, []),
            "ql_abi_version": (I, []),
            "q4_quantize_host": (I, [P, I, I, I, P, P, P]),
            "q4_quantize_sym_host": (I, [P, I, I, I, P, P]),
            "q4_packed_bytes": (Z, [I, I, I]),
            "q4_pack": (I, [P, P, P, I, I, I, P, Z]),
            "q4_unpack": (I, [P, Z, I, I, I, P, P, P]),
            "q4_gemm": (I, [P, I, I, I, I, P, Z, I, P, P, Z, P]),
            "q4_gemm_workspace_bytes": (Z, [I, I, I, I]),
            "q4_gemm_no_alloc": (I, [P, I, I, I, I, P, Z, I, P, P]),
            "q4_gemm_tile_shape": (I, [I, I, I, I, P, P, P]),
            "q4_quantize_act_order_host": (I, [P, I, I, I, P, P, P, P]),
            "q4_pack_act_order": (I, [P, P, P, P, I, I, I, P, Z, P]),
            "q4_permute_columns": (I, [P, I, I, I, P, P, P]),
            "i8_quant_weight_host": (I, [P, I, I, P, P]),
            "i8_azp_adj": (I, [P, I, I, P]),
            "i8_quant_per_token": (I, [P, I, I, I, P, P, P, P]),
            "i8_rmsnorm_quant_per_token": (I, [P, I, I, I, P, C.c_float, P, P, P, P]),
            "i8_gemm_scaled": (I, [P, P, I, I, I, P, I, P, I, P, P, P, P, I, P, P]),
            "f8_quant_weight_host": (I, [P, I, I, P, P]),
            "f8_quant_per_token": (I, [P, I, I, I, P, P, P]),
            "f8_gemm_scaled": (I, [P, P, I, I, I, P, I, P, I, P, P, I, P]),
            "ql_read_probe": (I, [P, Z, P, I, I, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.ql_abi_version() != ABI_VERSION:
            raise QLError(f"libqlinear ABI {L.ql_abi_version()} != {ABI_VERSION}")
        _lib = L
    return _lib


def _check(rc, fn):
    if rc != 0:
        raise QLError(f"{fn} returned {rc}: {lib().ql_last_error().decode()}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(t, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return C.c_void_p(s.cuda_stream)


def _dtype_code(dt):
    if dt == torch.float16:
        return QL_F16
    if dt == torch.bfloat16:
        return QL_BF16
    raise QLError(f"unsupported activation dtype {dt}")


def _host(t, dtype):
    if t.device.type != "cpu" or t.dtype != dtype or not t.is_contiguous():
        raise QLError(f"expected a contiguous CPU {dtype} tensor, got {t.dtype} on {t.device}")
    return t


def _dev(t, dtype=None, name="tensor"):
    if t.device.type != "cuda" or not t.is_contiguous():
        raise QLError(f"{name}: expected a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise QLError(f"{name}: expected {dtype}, got {t.dtype}")
    return t


def _shape(t, shape, name):
    """The C entry points see only pointers: every buffer's extent is checked here."""
    if tuple(t.shape) != tuple(shape):
        raise QLError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _same_device(name, *ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise QLError(f"{name}: operands on different devices {sorted(map(str, devs))}")


def _epilogue_operands(name, M, N, s_a, s_b, azp, azp_adj, bias, out_dtype, out):
    """Checks the epilogue vectors and the output of a scaled GEMM against (M, N)."""
    _dev(s_a, torch.float32, "s_a")
    _dev(s_b, torch.float32, "s_b")
    if s_a.numel() not in (1, M):
        raise QLError(f"{name}: s_a has {s_a.numel()} entries, expected 1 or M={M}")
    if s_b.numel() not in (1, N):
        raise QLError(f"{name}: s_b has {s_b.numel()} entries, expected 1 or N={N}")
    if azp is not None:
        _dev(azp, torch.int32, "azp")
        if azp.numel() != M:
            raise QLError(f"{name}: azp has {azp.numel()} entries, expected M={M}")
    if azp_adj is not None:
        _dev(azp_adj, torch.int32, "azp_adj")
        if azp_adj.numel() != N:
            raise QLError(f"{name}: azp_adj has {azp_adj.numel()} entries, expected N={N}")
    if bias is not None:
        _dev(bias, out_dtype, "bias")
        if bias.numel() != N:
            raise QLError(f"{name}: bias has {bias.numel()} entries, expected N={N}")
    if out is not None:
        _dev(out, out_dtype, "out")
        _shape(out, (M, N), f"{name}: out")


# ---------------------------------------------------------------- W4A16 offline (host)

def q4_quantize_host(W, group=GROUP):
    """W: CPU fp32 [N, K] -> (wq uint32 [K/8, N] as int32, scales fp16 [K/g, N], zeros uint8 [K/g, N])."""
    W = _host(W, torch.float32)
    N, K = W.shape
    wq = torch.empty((K // 8, N), dtype=torch.int32)
    scales = torch.empty((K // group, N), dtype=torch.float16)
    zeros = torch.empty((K // group, N), dtype=torch.uint8)
    _check(lib().q4_quantize_host(_ptr(W), N, K, group, _ptr(wq), _ptr(scales), _ptr(zeros)), "q4_quantize_host")
    return wq, scales, zeros


def q4_quantize_sym_host(W, group=GROUP):
    """W: CPU fp32 [N, K] -> (wq uint32 [K/8, N] as int32, scales fp16 [K/g, N]); symmetric codes with
    the zero point fixed at 8 (pack with zeros=None)."""
    W = _host(W, torch.float32)
    N, K = W.shape
    wq = torch.empty((K // 8, N), dtype=torch.int32)
    scales = torch.empty((K // group, N), dtype=torch.float16)
    _check(lib().q4_quantize_sym_host(_ptr(W), N, K, group, _ptr(wq), _ptr(scales)), "q4_quantize_sym_host")
    return wq, scales


def q4_packed_bytes(N, K, group=GROUP):
    return int(lib().q4_packed_bytes(N, K, group))


def q4_pack(wq, scales, zeros, N, K, group=GROUP, device=None):
    """Canonical host triple -> device blob (uint8 tensor on `device`, CPU if None).
    zeros=None stores the zero point 8 for every group (symmetric codes)."""
    wq = _host(wq, torch.int32)
    scales = _host(scales, torch.float16)
    if zeros is not None:
        zeros = _host(zeros, torch.uint8)
    nb = q4_packed_bytes(N, K, group)
    if nb == 0:
        raise QLError(f"q4_pack: invalid shape N={N} K={K} group={group}")
    blob = torch.empty(nb, dtype=torch.uint8)
    _check(lib().q4_pack(_ptr(wq), _ptr(scales), _ptr(zeros), N, K, group, _ptr(blob), nb), "q4_pack")
    return blob if device is None else blob.to(device)


def q4_unpack(blob, N, K, group=GROUP):
    blob = blob.cpu().contiguous()
    wq = torch.empty((K // 8, N), dtype=torch.int32)
    scales = torch.empty((K // group, N), dtype=torch.float16)
    zeros = torch.empty((K // group, N), dtype=torch.uint8)
    _check(lib().q4_unpack(_ptr(blob), blob.numel(), N, K, group, _ptr(wq), _ptr(scales), _ptr(zeros)), "q4_unpack")
    return wq, scales, zeros


# ---------------------------------------------------------------- W4A16 forward (device)

def q4_gemm_workspace_bytes(M, N, K, group=GROUP):
    """Bytes of device workspace q4_gemm uses for an M x N x K layer (0: none)."""
    return int(lib().q4_gemm_workspace_bytes(M, N, K, group))


def _workspace(M, N, K, group, device, workspace):
    need = q4_gemm_workspace_bytes(M, N, K, group)
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace")
        if workspace.numel() < need:
            raise QLError(f"q4_gemm: workspace has {workspace.numel()} bytes, needs {need}")
        return workspace
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def q4_gemm(X, packed, N, group=GROUP, Y=None, workspace=None, stream=None):
    """Y[M, N] = X[M, K] · dequant(W)ᵀ; X fp16/bf16 on the device, packed from q4_pack.
    workspace: a uint8 device buffer of at least q4_gemm_workspace_bytes(M, N, K)
    bytes, or None (then one is allocated when the plan splits K)."""
    X = _dev(X, name="X")
    _dev(packed, torch.uint8, "packed")
    if X.dim() != 2:
        raise QLError(f"q4_gemm: X must be 2-D, got shape {tuple(X.shape)}")
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=X.dtype, device=X.device)
    else:
        _dev(Y, X.dtype, "Y")
        _shape(Y, (M, N), "q4_gemm: Y")
    ws = _workspace(M, N, K, group, X.device, workspace)
    _same_device("q4_gemm", X, packed, Y, ws)
    _check(lib().q4_gemm(_ptr(X), _dtype_code(X.dtype), M, K, N, _ptr(packed), packed.numel(), group, _ptr(Y),
                         _ptr(ws), 0 if ws is None else ws.numel(), _stream(X, stream)), "q4_gemm")
    return Y


def q4_gemm_no_alloc(X, packed, N, Y, group=GROUP, stream=None):
    """q4_gemm into a caller-given Y with the library's static scratch: the C
    call allocates nothing (neither does this wrapper)."""
    X = _dev(X, name="X")
    _dev(packed, torch.uint8, "packed")
    _dev(Y, X.dtype, "Y")
    if X.dim() != 2:
        raise QLError(f"q4_gemm_no_alloc: X must be 2-D, got shape {tuple(X.shape)}")
    M, K = X.shape
    _shape(Y, (M, N), "q4_gemm_no_alloc: Y")
    _same_device("q4_gemm_no_alloc", X, packed, Y)
    _check(lib().q4_gemm_no_alloc(_ptr(X), _dtype_code(X.dtype), M, K, N, _ptr(packed), packed.numel(), group,
                                  _ptr(Y), _stream(X, stream)), "q4_gemm_no_alloc")
    return Y


# ---------------------------------------------------------------- act-order (g_idx)

def q4_quantize_act_order_host(W, g_idx, group=GROUP):
    """W: CPU fp32 [N, K], g_idx: CPU int32 [K] -> (wq, scales, zeros) as q4_quantize_host, with the
    groups given by g_idx."""
    W = _host(W, torch.float32)
    g_idx = _host(g_idx, torch.int32)
    N, K = W.shape
    wq = torch.empty((K // 8, N), dtype=torch.int32)
    scales = torch.empty((K // group, N), dtype=torch.float16)
    zeros = torch.empty((K // group, N), dtype=torch.uint8)
    _check(lib().q4_quantize_act_order_host(_ptr(W), N, K, group, _ptr(g_idx), _ptr(wq), _ptr(scales), _ptr(zeros)),
           "q4_quantize_act_order_host")
    return wq, scales, zeros


def q4_pack_act_order(wq, scales, zeros, g_idx, N, K, group=GROUP, device=None):
    """Canonical triple + g_idx -> (blob in processing order, perm int32 [K]), both on `device`."""
    wq = _host(wq, torch.int32)
    scales = _host(scales, torch.float16)
    if zeros is not None:
        zeros = _host(zeros, torch.uint8)
    g_idx = _host(g_idx, torch.int32)
    nb = q4_packed_bytes(N, K, group)
    if nb == 0:
        raise QLError(f"q4_pack_act_order: invalid shape N={N} K={K} group={group}")
    blob = torch.empty(nb, dtype=torch.uint8)
    perm = torch.empty(K, dtype=torch.int32)
    _check(lib().q4_pack_act_order(_ptr(wq), _ptr(scales), _ptr(zeros), _ptr(g_idx), N, K, group, _ptr(blob), nb,
                                   _ptr(perm)), "q4_pack_act_order")
    return (blob, perm) if device is None else (blob.to(device), perm.to(device))


def q4_permute_columns(X, perm, Xp=None, stream=None):
    """Xp[m, j] = X[m, perm[j]] on the device (the activations in the blob's channel order)."""
    X = _dev(X, name="X")
    _dev(perm, torch.int32, "perm")
    M, K = X.shape
    if perm.numel() != K:
        raise QLError(f"q4_permute_columns: perm has {perm.numel()} entries, expected {K}")
    if Xp is None:
        Xp = torch.empty_like(X)
    else:
        _dev(Xp, X.dtype, "Xp")
        _shape(Xp, (M, K), "q4_permute_columns: Xp")
    _check(lib().q4_permute_columns(_ptr(X), _dtype_code(X.dtype), M, K, _ptr(perm), _ptr(Xp), _stream(X, stream)),
           "q4_permute_columns")
    return Xp


def q4_gemm_act_order(X, packed, perm, N, group=GROUP, Y=None, stream=None):
    """Y = X · dequant(W)ᵀ for an act-order blob: q4_permute_columns, then q4_gemm."""
    return q4_gemm(q4_permute_columns(X, perm, stream=stream), packed, N, group, Y, stream=stream)


def q4_gemm_tile_shape(M, N, K, with_workspace=True):
    """(rows, cols) of the workgroup tile q4_gemm uses for M x N x K; (0, 0)
    when M <= 16 (the decode kernel)."""
    return q4_gemm_plan(M, N, K, with_workspace)[:2]


def q4_gemm_plan(M, N, K, with_workspace=True):
    """(rows, cols, splits): q4_gemm's workgroup tile and K splits for M x N x K
    with a workspace or without one; (0, 0, 1) when M <= 16 (the decode kernel)."""
    r, c, s = C.c_int(0), C.c_int(0), C.c_int(0)
    _check(lib().q4_gemm_tile_shape(M, N, K, int(bool(with_workspace)), C.byref(r), C.byref(c), C.byref(s)),
           "q4_gemm_tile_shape")
    return r.value, c.value, s.value


def q4_gemm_launcher(X, packed, N, Y, group=GROUP, workspace=None, stream=None):
    """Checks the operands of q4_gemm once and returns a callable that
    launches it again on the same buffers with the arguments already
    marshalled (for tight launch loops: the C entry point still validates
    every call).  The workspace (allocated here when None and needed) lives
    with the callable."""
    X = _dev(X, name="X")
    _dev(packed, torch.uint8, "packed")
    _dev(Y, X.dtype, "Y")
    M, K = X.shape
    if tuple(Y.shape) != (M, N):
        raise QLError(f"q4_gemm: Y has shape {tuple(Y.shape)}, expected {(M, N)}")
    ws = _workspace(M, N, K, group, X.device, workspace)
    f = lib().q4_gemm
    args = (_ptr(X), _dtype_code(X.dtype), M, K, N, _ptr(packed), packed.numel(), group, _ptr(Y), _ptr(ws),
            0 if ws is None else ws.numel(), _stream(X, stream))

    def launch():
        rc = f(*args)
        if rc != 0:
            _check(rc, "q4_gemm")

    launch.workspace = ws
    return launch


def launcher(name, *args, stream=None):
    """Returns a callable that calls the device entry point `name` (i8_gemm_scaled,
    i8_quant_per_token, ...) with its arguments marshalled once: a tensor
    becomes its data pointer, a torch dtype its ql_dtype code, None a NULL
    pointer, other values pass unchanged, and the stream argument (torch's
    current stream unless one is given) is appended.  For tight launch loops,
    where the checks and output allocations of the functions above would take
    more host time than the kernel takes on the device; the caller keeps the
    tensors alive, and the C entry point still validates every call."""
    f = getattr(lib(), name)
    tensors = [a for a in args if isinstance(a, torch.Tensor)]
    if not tensors or any(t.device.type != "cuda" for t in tensors):
        raise QLError(f"{name}: launcher needs device tensors")
    conv = []
    for a in args:
        if isinstance(a, torch.Tensor):
            conv.append(C.c_void_p(a.data_ptr()))
        elif isinstance(a, torch.dtype):
            conv.append(_dtype_code(a))
        else:
            conv.append(a)
    conv.append(_stream(tensors[0], stream))

    def launch(*_):
        rc = f(*conv)
        if rc != 0:
            _check(rc, name)

    return launch


# ---------------------------------------------------------------- W8A8

def i8_quant_weight_host(W):
    """CPU fp32 [N, K] -> (Bq int8 [N, K], s_b fp32 [N])."""
    W = _host(W, torch.float32)
    N, K = W.shape
    Bq = torch.empty((N, K), dtype=torch.int8)
    s_b = torch.empty(N, dtype=torch.float32)
    _check(lib().i8_quant_weight_host(_ptr(W), N, K, _ptr(Bq), _ptr(s_b)), "i8_quant_weight_host")
    return Bq, s_b


def i8_azp_adj(Bq):
    """CPU int8 [N, K] -> int32 [N] row sums."""
    Bq = _host(Bq, torch.int8)
    N, K = Bq.shape
    adj = torch.empty(N, dtype=torch.int32)
    _check(lib().i8_azp_adj(_ptr(Bq), N, K, _ptr(adj)), "i8_azp_adj")
    return adj


def i8_quant_per_token(X, symmetric=False, stream=None):
    """X fp16/bf16 [M, K] on the device -> (Aq int8 [M, K], s_a fp32 [M], azp int32 [M] or None)."""
    X = _dev(X, name="X")
    M, K = X.shape
    Aq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    s_a = torch.empty(M, dtype=torch.float32, device=X.device)
    azp = None if symmetric else torch.empty(M, dtype=torch.int32, device=X.device)
    _check(lib().i8_quant_per_token(_ptr(X), _dtype_code(X.dtype), M, K, _ptr(Aq), _ptr(s_a), _ptr(azp),
                                    _stream(X, stream)), "i8_quant_per_token")
    return Aq, s_a, azp


def i8_rmsnorm_quant_per_token(X, gamma, eps, symmetric=False, stream=None):
    """RMSNorm(X) · gamma quantized per token, in one kernel.  X fp16/bf16
    [M, K] and gamma [K] of the same dtype on the device; eps > 0.
    Returns (Aq int8 [M, K], s_a fp32 [M], azp int32 [M] or None)."""
    X = _dev(X, name="X")
    _dev(gamma, X.dtype, "gamma")
    M, K = X.shape
    if tuple(gamma.shape) != (K,):
        raise QLError(f"i8_rmsnorm_quant_per_token: gamma has shape {tuple(gamma.shape)}, expected ({K},)")
    Aq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    s_a = torch.empty(M, dtype=torch.float32, device=X.device)
    azp = None if symmetric else torch.empty(M, dtype=torch.int32, device=X.device)
    _check(lib().i8_rmsnorm_quant_per_token(_ptr(X), _dtype_code(X.dtype), M, K, _ptr(gamma), float(eps), _ptr(Aq),
                                            _ptr(s_a), _ptr(azp), _stream(X, stream)), "i8_rmsnorm_quant_per_token")
    return Aq, s_a, azp


def i8_gemm_scaled(Aq, Bq, s_a, s_b, azp=None, azp_adj=None, bias=None, out_dtype=torch.float16,
                   raw=False, out=None, stream=None):
    """out[M, N] = s_a * s_b * (Aq·Bqᵀ - azp * azp_adj) + bias, on the device.
    With raw=True also returns the int32 corrected accumulator."""
    _dev(Aq, torch.int8, "Aq")
    _dev(Bq, torch.int8, "Bq")
    if Aq.dim() != 2 or Bq.dim() != 2:
        raise QLError("i8_gemm_scaled: Aq and Bq must be 2-D")
    M, K = Aq.shape
    N = Bq.shape[0]
    if Bq.shape[1] != K:
        raise QLError("Aq and Bq disagree on K")
    _epilogue_operands("i8_gemm_scaled", M, N, s_a, s_b, azp, azp_adj, bias, out_dtype, out)
    _same_device("i8_gemm_scaled", Aq, Bq, s_a, s_b, azp, azp_adj, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=Aq.device)
    rawt = torch.empty((M, N), dtype=torch.int32, device=Aq.device) if raw else None
    _check(lib().i8_gemm_scaled(_ptr(Aq), _ptr(Bq), M, N, K, _ptr(s_a), s_a.numel(), _ptr(s_b), s_b.numel(),
                                _ptr(azp), _ptr(azp_adj), _ptr(bias), _ptr(out), _dtype_code(out_dtype),
                                _ptr(rawt), _stream(Aq, stream)), "i8_gemm_scaled")
    return (out, rawt) if raw else out


# ---------------------------------------------------------------- W8A8 with FP8 (E4M3) codes

def f8_quant_weight_host(W):
    """CPU fp32 [N, K] -> (Bq uint8 E4M3 codes [N, K], s_b fp32 [N])."""
    W = _host(W, torch.float32)
    N, K = W.shape
    Bq = torch.empty((N, K), dtype=torch.uint8)
    s_b = torch.empty(N, dtype=torch.float32)
    _check(lib().f8_quant_weight_host(_ptr(W), N, K, _ptr(Bq), _ptr(s_b)), "f8_quant_weight_host")
    return Bq, s_b


def f8_quant_per_token(X, stream=None):
    """X fp16/bf16 [M, K] on the device -> (Aq uint8 E4M3 codes [M, K], s_a fp32 [M])."""
    X = _dev(X, name="X")
    M, K = X.shape
    Aq = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    s_a = torch.empty(M, dtype=torch.float32, device=X.device)
    _check(lib().f8_quant_per_token(_ptr(X), _dtype_code(X.dtype), M, K, _ptr(Aq), _ptr(s_a), _stream(X, stream)),
           "f8_quant_per_token")
    return Aq, s_a


def f8_gemm_scaled(Aq, Bq, s_a, s_b, bias=None, out_dtype=torch.float16, out=None, stream=None):
    """out[M, N] = s_a * s_b * (e4m3(Aq)·e4m3(Bq)ᵀ) + bias, on the device."""
    _dev(Aq, torch.uint8, "Aq")
    _dev(Bq, torch.uint8, "Bq")
    if Aq.dim() != 2 or Bq.dim() != 2:
        raise QLError("f8_gemm_scaled: Aq and Bq must be 2-D")
    M, K = Aq.shape
    N = Bq.shape[0]
    if Bq.shape[1] != K:
        raise QLError("Aq and Bq disagree on K")
    _epilogue_operands("f8_gemm_scaled", M, N, s_a, s_b, None, None, bias, out_dtype, out)
    _same_device("f8_gemm_scaled", Aq, Bq, s_a, s_b, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=Aq.device)
    _check(lib().f8_gemm_scaled(_ptr(Aq), _ptr(Bq), M, N, K, _ptr(s_a), s_a.numel(), _ptr(s_b), s_b.numel(),
                                _ptr(bias), _ptr(out), _dtype_code(out_dtype), _stream(Aq, stream)),
           "f8_gemm_scaled")
    return out


# ---------------------------------------------------------------- measurement aid

def read_probe_launcher(src, workgroups, mode=0, nbytes=None, stream=None):
    """Checks a device buffer once and returns a callable that streams
    `nbytes` of it (all of it by default) through ql_read_probe: the plain
    HBM read rate the decode kernel is compared with (mode 0: grid-stride
    reads, mode 1: one contiguous chunk per workgroup)."""
    _dev(src, name="src")
    nbytes = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if nbytes > src.numel() * src.element_size() or nbytes % 16:
        raise QLError(f"ql_read_probe: {nbytes} bytes is not a multiple of 16 within the buffer")
    sink = torch.empty(4 * workgroups, dtype=torch.int32, device=src.device)
    f = lib().ql_read_probe
    args = (_ptr(src), nbytes, _ptr(sink), int(workgroups), int(mode), _stream(src, stream))

    def launch(*_):
        rc = f(*args)
        if rc != 0:
            _check(rc, "ql_read_probe")

    launch.sink = sink                # keeps the sink alive with the callable
    return launch
