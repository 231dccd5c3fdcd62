"""The binding rejects operands whose extent, dtype or device disagrees with
the shapes it passes to the C ABI (which receives only pointers and sizes and
so cannot see a short or mis-shaped buffer): every such case raises before
the library is called, so no kernel is launched.  And the read probe (the
measurement aid) folds every word of the bytes it is given."""

import numpy as np
import pytest
import torch

import quantized_linear_layers_amd as ql

pytestmark = pytest.mark.gpu


def dev(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def host(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def build(spec):
    """{name: (maker, shape, dtype)} -> {name: tensor}; tensors are made inside
    the test, so that collection needs no device."""
    return {k: f(shape, dt) for k, (f, shape, dt) in spec.items()}


def i8_operands(M=32, N=64, K=128):
    return dict(Aq=dev((M, K), torch.int8), Bq=dev((N, K), torch.int8), s_a=dev(M, torch.float32),
                s_b=dev(N, torch.float32), azp=dev(M, torch.int32), azp_adj=dev(N, torch.int32),
                bias=dev(N, torch.float16))


@pytest.mark.parametrize("spec", [
    dict(out=(dev, (32, 63), torch.float16)),               # wrong shape
    dict(out=(host, (32, 64), torch.float16)),              # host memory
    dict(out=(dev, (32, 64), torch.bfloat16)),              # dtype differs from out_dtype
    dict(azp=(dev, 31, torch.int32)),                       # short zero points
    dict(azp_adj=(dev, 63, torch.int32)),                   # short column sums
    dict(bias=(dev, 63, torch.float16)),                    # short bias
    dict(s_a=(dev, 31, torch.float32)),                     # neither 1 nor M scales
    dict(s_b=(dev, 2, torch.float32)),                      # neither 1 nor N scales
])
def test_i8_gemm_rejects_bad_buffers(spec):
    bad = build(spec)
    ops = i8_operands()
    out = bad.pop("out", None)
    ops.update(bad)
    with pytest.raises(ql.QLError):
        ql.i8_gemm_scaled(ops["Aq"], ops["Bq"], ops["s_a"], ops["s_b"], ops["azp"], ops["azp_adj"], ops["bias"],
                          out=out)


@pytest.mark.parametrize("spec", [
    dict(out=(dev, (32, 65), torch.float16)),
    dict(out=(host, (32, 64), torch.float16)),
    dict(bias=(dev, 32, torch.float16)),
    dict(s_a=(dev, 5, torch.float32)),
])
def test_f8_gemm_rejects_bad_buffers(spec):
    bad = build(spec)
    M, N, K = 32, 64, 128
    ops = dict(Aq=dev((M, K), torch.uint8), Bq=dev((N, K), torch.uint8), s_a=dev(M, torch.float32),
               s_b=dev(N, torch.float32), bias=dev(N, torch.float16))
    out = bad.pop("out", None)
    ops.update(bad)
    with pytest.raises(ql.QLError):
        ql.f8_gemm_scaled(ops["Aq"], ops["Bq"], ops["s_a"], ops["s_b"], ops["bias"], out=out)


def test_q4_gemm_rejects_bad_output():
    X = dev((4, 256), torch.float16)
    blob = dev(ql.q4_packed_bytes(64, 256), torch.uint8)
    for Y in (dev((4, 63), torch.float16), dev((64,), torch.float16), dev((4, 64), torch.bfloat16),
              host((4, 64), torch.float16)):
        with pytest.raises(ql.QLError):
            ql.q4_gemm(X, blob, 64, Y=Y)
    with pytest.raises(ql.QLError):
        ql.q4_gemm(dev((256,), torch.float16), blob, 64)
    with pytest.raises(ql.QLError):
        ql.q4_gemm_launcher(X, blob, 64, dev((5, 64), torch.float16))


def test_permute_rejects_bad_output():
    X = dev((4, 256), torch.float16)
    perm = dev(256, torch.int32)
    with pytest.raises(ql.QLError):
        ql.q4_permute_columns(X, perm, Xp=dev((4, 255), torch.float16))
    with pytest.raises(ql.QLError):
        ql.q4_permute_columns(X, dev(255, torch.int32))


@pytest.mark.parametrize("mode,wgs,nbytes", [(0, 2048, 35 << 20), (1, 512, 35 << 20), (0, 7, 4096 + 48),
                                             (1, 300, (1 << 20) + 16), (1, 64, 64)])
def test_read_probe_reads_every_byte(mode, wgs, nbytes):
    """The measurement aid really reads the buffer: the XOR of its sink words
    equals the XOR of all 32-bit words of the bytes it was given (each word is
    folded exactly once, whatever the pattern)."""
    g = torch.Generator().manual_seed(nbytes + mode)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, ((nbytes + 1024) // 4,), dtype=torch.int32, generator=g)
    f = ql.read_probe_launcher(buf.cuda(), wgs, mode, nbytes=nbytes)
    f()
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf[: nbytes // 4].numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(f.sink.cpu().numpy().view(np.uint32))
    assert got == want
