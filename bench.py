"""Throughput of the quantized linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-also] [--no-per-case]

The main line is the W4A16 decode GEMV on the Llama-2-70B-shaped layers, the
bandwidth-bound case (M in {1, 8} x (K, N) in {(8192, 8192), (8192, 28672),
(28672, 8192)}, g = 128, bf16 activations and output, fp16 scales).  One step
runs all six (M, K, N) cases once, in that order.  `value` is the effective
bandwidth of a whole step: algorithmic bytes (packed weights + fp16 scales +
4-bit zeros + X + Y) over the step's time, inputs resident in HBM.  Every
launch of a case reads its own copy of the weights, and a copy is read again
only after more than 1 GiB of other weights (four times the 256 MB Infinity
Cache), so the weights come from HBM, not from cache.

The steps are launched back to back on one stream with their arguments
marshalled once; the timed region is bracketed by HIP events recorded on that
stream.  The step holds nothing but the decode kernel's launches, so the
roofline object's mean launch duration is the timed region's elapsed time over
its launches.  Before the W warm-up steps the step runs for about 250 ms, so
the timed steps start in the state a sustained load settles in.

Beside it, in the same process: each case timed alone (back-to-back launches
over the weight copies), and a plain streaming read of the same weight bytes
(`ql_read_probe`, the achievable HBM read rate) timed the same way, per case
and as a whole step: the read ceiling the decode kernel is measured against.
The `also` object holds the other workloads (7B decode step, W8A8 prefill GEMM
with int8 and with FP8 codes, W4A16 prefill GEMM, W4A16 mid-M), and
`cpu_baseline` the untuned oracle on the host cores.
"""

import argparse
import functools
import json
import os
import sys
import time

import numpy as np
import torch

import workloads as wl

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK = {"bf16": 2.5e15, "f16": 2.5e15, "i8": 5.0e15, "fp8": 5.0e15}   # dense, published
METRIC = "W4A16 GEMV effective GB/s (% HBM peak); W8A8/W4A16 GEMM TOPS (% MFMA peak)"
MALL_DEFEAT_BYTES = 1 << 30

# HBM traffic of the decode kernel per launch (mean over the six cases of a
# step), from two counter runs (FETCH_SIZE, then WRITE_SIZE) each scaled by
# what the same counter reads for a plain device copy of known size in the
# same run.  It belongs to one version of the kernel source: when the source
# hash differs, the figure is stale and `traffic` is reported as null.
TRAFFIC = {"source_sha256": "af016fccc5314c16d42c85e8911383f714a9e16c9ee625605d700f251778e16f",
           "bytes_per_launch": 94264608}


@functools.lru_cache(maxsize=None)
def _weight(w, K, N):
    """fp32 weight draw of a workload's layer, drawn once per process (the
    70B layers take seconds each to draw)."""
    return wl.weight(w, K, N)


def w4a16_bytes(M, K, N, group=128, e=2):
    """Algorithmic bytes of one W4A16 layer: packed codes, fp16 scales, 4-bit
    zero points, X and Y (the data the method has to move, not the fp16 weights
    it avoids)."""
    return K * N // 2 + (K // group) * N * 2 + (K // group) * N // 2 + M * K * e + M * N * e


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _prepare_w4(ql, w, K, N, copies):
    W = _weight(w, K, N)
    wq, s, z = ql.q4_quantize_host(torch.from_numpy(W))
    blob = ql.q4_pack(wq, s, z, N, K)
    return W, [blob.to("cuda") for _ in range(copies)]


def _copies_for(total_bytes):
    """Copies of a buffer of total_bytes such that a loop over them reads more
    than MALL_DEFEAT_BYTES of other copies before it reads one again."""
    return max(2, -(-(MALL_DEFEAT_BYTES + total_bytes) // max(total_bytes, 1)))


# plain-read probe configurations (mode, workgroups); the fastest per layer is
# the read ceiling (grid-stride reads on 2048 workgroups win on tens of MB; on
# hundreds, grid-stride reads on 256 and one contiguous chunk per workgroup on
# 512 or 1024 come within a few percent of each other, box to box)
READ_PROBES = ((0, 2048), (0, 256), (1, 512), (1, 1024))
# back-to-back steps before the W warm-up steps: the first tens of
# milliseconds of work after the weights are prepared run slower (measured:
# 147 us for the 70B step after 30 ms of warm-up, 118-121 us after 60 ms more)
STEP_WARM_MS = 250.0


def _kernel_source_sha():
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_linear_layers_amd", "csrc",
                       "q4_gemv.hip")
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def copy_calibration(mib):
    """A plain device-to-device copy of `mib` MiB, three times: the reference
    the byte counters are scaled by (it reads and writes exactly that much)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# copy calibration: {n} bytes read and written per copy, 3 copies", flush=True)
    del src, dst


# warm-up per timed kernel (--warm-ms): after an idle gap a kernel needs about
# 50 ms of its own back-to-back launches before it runs at its sustained
# speed (measured: the W4A16 prefill 527 us after 10 ms, 439-457 us after
# 50-1000 ms; the int8 GEMM 40.1 us, then 35.2-35.4 us)
WARM_MS = 100.0


def warm(fn_list, ms=30.0, cap=20000):
    """Runs the launches back to back until about `ms` of GPU time has
    elapsed, so that the timed ones start at the speed a sustained load
    settles at (after an idle gap the part takes tens of milliseconds to get
    there, and the first launches run slower than the later ones, so the
    elapsed time is measured batch by batch rather than estimated from the
    first launch)."""
    s = torch.cuda.current_stream()
    done, i, batch = 0.0, 0, 1
    while done < ms and i < cap:
        a, b = _events()
        a.record(s)
        for _ in range(batch):
            for fn in fn_list:
                fn(i)
            i += 1
        b.record(s)
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        done += t
        # next batch: about 10 ms of launches (at least one)
        batch = max(1, min(cap - i, int(batch * 10.0 / max(t, 1e-3))))
    torch.cuda.synchronize()


def time_launches(fn_list, reps, stream, warm_ms=None):
    """Mean ms per launch of each entry: fn(0) .. fn(reps - 1) back to back
    between two HIP events on `stream`, one entry at a time, each after
    `warm_ms` of its own launches (so every kernel is timed at the clock its
    own load settles at, not at the one the previous entry left).  The
    entries are launchers with their arguments marshalled once, so the host
    stays ahead of the device and the interval holds nothing but the kernels."""
    out = np.zeros(len(fn_list))
    for i, fn in enumerate(fn_list):
        warm([fn], WARM_MS if warm_ms is None else warm_ms)
        a, b = _events()
        a.record(stream)
        for r in range(reps):
            fn(r)
        b.record(stream)
        torch.cuda.synchronize()
        out[i] = a.elapsed_time(b) / reps
    return [float(x) for x in out]


def bench_decode(ql, wname, steps, warmup, per_case=True):
    """Runs a W4A16 decode workload; returns a dict of results.

    Every layer (K, N) gets R copies of its blob.  Case j of the layer's nM
    token counts in step r reads copy (r * nM + j) % R, so a copy is read again
    only after R - 1 other reads of that layer, and R is chosen so that those
    and the other layers' reads in between exceed MALL_DEFEAT_BYTES; the
    per-case loops cycle over the same copies, which also exceed it alone."""
    w = wl.WORKLOADS[wname]
    cases = w.all_cases()
    nM = len(w.Ms)
    shapes = list(w.shapes)
    lb = {(K, N): ql.q4_packed_bytes(N, K) for (K, N) in shapes}
    step_wbytes = nM * sum(lb.values())
    need_step = -(-nM * (MALL_DEFEAT_BYTES + max(lb.values())) // step_wbytes)
    R = {L: max(nM + 1, need_step, _copies_for(lb[L])) for L in shapes}
    blobs = {L: _prepare_w4(ql, w, L[0], L[1], R[L])[1] for L in shapes}
    X = {c: wl.activations(w, c[0], c[1], c[2]).cuda() for c in cases}
    Y = {c: torch.empty((c[0], c[2]), dtype=X[c].dtype, device="cuda") for c in cases}
    stream = torch.cuda.current_stream()
    # launchers with the arguments marshalled once (the host cost of a launch
    # must stay below the kernel's microseconds)
    gemv = {c: [ql.q4_gemm_launcher(X[c], b, c[2], Y[c]) for b in blobs[(c[1], c[2])]] for c in cases}
    probe = {(L, p): [ql.read_probe_launcher(b, p[1], p[0]) for b in blobs[L]] for L in shapes for p in READ_PROBES}

    def copy_of(c, r):
        L = (c[1], c[2])
        return (r * nM + w.Ms.index(c[0])) % R[L]

    def step(r):
        for c in cases:
            gemv[c][copy_of(c, r)]()

    best = {}                    # fastest probe configuration of each layer

    def probe_step(r):
        for c in cases:
            probe[((c[1], c[2]), best[(c[1], c[2])])][copy_of(c, r)]()

    def timed(fn, n):
        warm([fn], STEP_WARM_MS)
        for i in range(warmup):
            fn(i)
        a, b = _events()
        a.record(stream)
        for i in range(n):
            fn(warmup + i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    bytes_step = sum(w4a16_bytes(*c) for c in cases)
    ms_step = timed(step, steps)
    res = {"cases": cases, "bytes_step": bytes_step, "ms_step": ms_step,
           "value_gbs": bytes_step / (ms_step * 1e-3) / 1e9,
           "copies": {f"{K}x{N}": R[(K, N)] for (K, N) in shapes}}
    if not per_case:
        return res
    # the plain read of each layer's weight copies, back to back, in every
    # probe configuration; the fastest is that layer's read ceiling
    read_ms = {}
    for L in shapes:
        n = R[L]
        t = {p: time_launches([lambda i, f=probe[(L, p)], n=n: f[i % n]()], max(steps, 2 * n), stream)[0]
             for p in READ_PROBES}
        best[L] = min(t, key=t.get)
        read_ms[L] = t[best[L]]
    # the plain read of the same weight bytes, as a whole step
    ms_probe = timed(probe_step, steps)
    wbytes = sum(lb[(c[1], c[2])] for c in cases)
    res["read_ceiling_step"] = {"us": round(ms_probe * 1e3, 2),
                                "weight_GBps": round(wbytes / (ms_probe * 1e-3) / 1e9, 1),
                                "frac_hbm": round(wbytes / (ms_probe * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "step_us_over_read_us": round(ms_step / ms_probe, 4),
                                "probe_per_layer": {f"{K}x{N}": {"mode": best[(K, N)][0], "workgroups": best[(K, N)][1]}
                                                    for (K, N) in shapes}}
    # each case alone, back to back over its weight copies
    out, kern = [], 0.0
    for c in cases:
        L, n = (c[1], c[2]), R[(c[1], c[2])]
        ms = time_launches([lambda i, c=c, n=n: gemv[c][i % n]()], max(steps, 2 * n), stream)[0]
        kern += ms
        gbs = w4a16_bytes(*c) / (ms * 1e-3) / 1e9
        rd = lb[L] / (read_ms[L] * 1e-3) / 1e9
        out.append({"M": c[0], "K": c[1], "N": c[2], "us": round(ms * 1e3, 3), "GBps": round(gbs, 1),
                    "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "read_us": round(read_ms[L] * 1e3, 3),
                    "read_GBps": round(rd, 1), "frac_of_read": round(gbs / rd, 4)})
    res["per_case"] = out
    res["kernel_ms_step"] = kern
    return res


def _activation_copies(X):
    """Copies of an activation tensor that together exceed the last-level
    cache, so that a loop over them reads its inputs from HBM."""
    return [X.clone() for _ in range(_copies_for(X.numel() * X.element_size()))]


def bench_w8a8(ql, reps):
    w = wl.WORKLOADS["w8a8_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    X = wl.activations(w, M, K, N).cuda()
    Xs = _activation_copies(X)
    Bq, s_b = ql.i8_quant_weight_host(torch.from_numpy(wl.weight(w, K, N)))
    adj = ql.i8_azp_adj(Bq)
    Bq, s_b, adj = Bq.cuda(), s_b.cuda(), adj.cuda()
    bias = wl.bias(w, N).cuda()
    Aq, s_a, azp = ql.i8_quant_per_token(X)
    Aq2, s_a2, azp2 = ql.i8_quant_per_token(X)   # the timed quant launches write here
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    gamma = wl.norm_weight(w, K).cuda()
    lq = [ql.launcher("i8_quant_per_token", x, x.dtype, M, K, Aq2, s_a2, azp2) for x in Xs]
    ln = [ql.launcher("i8_rmsnorm_quant_per_token", x, x.dtype, M, K, gamma, 1e-5, Aq2, s_a2, azp2) for x in Xs]
    lg = ql.launcher("i8_gemm_scaled", Aq, Bq, M, N, K, s_a, M, s_b, N, azp, adj, bias, out, torch.float16, None)
    fq = lambda r: lq[r % len(lq)]()
    fg = lambda r: lg()
    fn = lambda r: ln[r % len(ln)]()
    tq, tg, tn = time_launches([fq, fg, fn], reps, stream)
    ops = 2.0 * M * N * K
    qbytes = M * K * 2 + M * K + M * 4 + M * 4
    return {"workload": w.name, "M": M, "K": K, "N": N,
            "gemm_us": round(tg * 1e3, 2), "gemm_TOPS": round(ops / (tg * 1e-3) / 1e12, 1),
            "gemm_frac_mfma_i8": round(ops / (tg * 1e-3) / MFMA_PEAK["i8"], 4),
            "quant_us": round(tq * 1e3, 2), "quant_GBps": round(qbytes / (tq * 1e-3) / 1e9, 1),
            "rmsnorm_quant_us": round(tn * 1e3, 2), "rmsnorm_quant_GBps": round((qbytes + K * 2) / (tn * 1e-3) / 1e9, 1),
            "end_to_end_us": round((tq + tg) * 1e3, 2)}


def bench_f8(ql, reps):
    """The W8A8 prefill workload with FP8 (E4M3) codes instead of int8."""
    w = wl.WORKLOADS["w8a8_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    X = wl.activations(w, M, K, N).cuda()
    Bq, s_b = ql.f8_quant_weight_host(torch.from_numpy(wl.weight(w, K, N)))
    Bq, s_b = Bq.cuda(), s_b.cuda()
    bias = wl.bias(w, N).cuda()
    Aq, s_a = ql.f8_quant_per_token(X)
    Aq2, s_a2 = ql.f8_quant_per_token(X)         # the timed quant launches write here
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    lq = [ql.launcher("f8_quant_per_token", x, x.dtype, M, K, Aq2, s_a2) for x in _activation_copies(X)]
    lg = ql.launcher("f8_gemm_scaled", Aq, Bq, M, N, K, s_a, M, s_b, N, bias, out, torch.float16)
    fq = lambda r: lq[r % len(lq)]()
    fg = lambda r: lg()
    tq, tg = time_launches([fq, fg], reps, torch.cuda.current_stream())
    ops = 2.0 * M * N * K
    return {"workload": w.name + ", FP8 E4M3 codes", "M": M, "K": K, "N": N,
            "gemm_us": round(tg * 1e3, 2), "gemm_TFLOPS": round(ops / (tg * 1e-3) / 1e12, 1),
            "gemm_frac_mfma_fp8": round(ops / (tg * 1e-3) / MFMA_PEAK["fp8"], 4),
            "quant_us": round(tq * 1e3, 2), "end_to_end_us": round((tq + tg) * 1e3, 2)}


def w8a8_bytes(M, K, N):
    """Algorithmic bytes of one W8A8 layer: the weight codes, the activation
    codes, per-channel fp32 scales, int32 column sums and fp16 bias, per-token
    fp32 scales and int32 zero points, and the fp16 output."""
    return N * K + M * K + N * (4 + 4 + 2) + M * (4 + 4) + M * N * 2


def bench_w8a8_decode(ql, reps):
    """W8A8 with few tokens (the decode kernel) on the Llama-2-70B layer
    shapes and token counts of the headline workload, int8 and FP8 codes from
    the same fp32 weights, weight copies rotated over more than the last-level
    cache.  Beside each layer: the plain read of its weight bytes."""
    w = wl.WORKLOADS["decode_70b"]
    st = torch.cuda.current_stream()
    bias = wl.bias(wl.WORKLOADS["w8a8_prefill"], max(N for _, N in w.shapes))
    per_case = {}
    for (K, N) in w.shapes:
        W = torch.from_numpy(_weight(w, K, N))
        Bq, s_b = ql.i8_quant_weight_host(W)
        adj = ql.i8_azp_adj(Bq).cuda()
        B8, s_b8 = ql.f8_quant_weight_host(W)
        R = _copies_for(N * K)
        Bqs = [Bq.cuda() for _ in range(R)]
        B8s = [B8.cuda() for _ in range(R)]
        del W, Bq, B8
        s_b, s_b8, b = s_b.cuda(), s_b8.cuda(), bias[:N].cuda()
        probes = {p: [ql.read_probe_launcher(x, p[1], p[0]) for x in Bqs] for p in READ_PROBES}
        read_ms = min(time_launches([lambda i, f=f: f[i % R]()], max(reps, 2 * R), st)[0] for f in probes.values())
        for M in w.Ms:
            X = wl.activations(w, M, K, N).cuda()
            Aq, s_a, azp = ql.i8_quant_per_token(X)
            A8, s_a8 = ql.f8_quant_per_token(X)
            out = torch.empty((M, N), dtype=torch.float16, device="cuda")
            li = [ql.launcher("i8_gemm_scaled", Aq, x, M, N, K, s_a, M, s_b, N, azp, adj, b, out, torch.float16, None)
                  for x in Bqs]
            lf = [ql.launcher("f8_gemm_scaled", A8, x, M, N, K, s_a8, M, s_b8, N, b, out, torch.float16) for x in B8s]
            ti, tf = time_launches([lambda r: li[r % R](), lambda r: lf[r % R]()], max(reps, R), st)
            nb = w8a8_bytes(M, K, N)
            per_case[f"{M}x{K}x{N}"] = {
                "int8_us": round(ti * 1e3, 2), "int8_GBps": round(nb / (ti * 1e-3) / 1e9, 1),
                "int8_frac_hbm": round(nb / (ti * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "fp8_us": round(tf * 1e3, 2), "fp8_GBps": round(nb / (tf * 1e-3) / 1e9, 1),
                "fp8_frac_hbm": round(nb / (tf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "read_us": round(read_ms * 1e3, 2),
                "int8_frac_of_read": round(read_ms / ti, 4), "fp8_frac_of_read": round(read_ms / tf, 4)}
        del Bqs, B8s, probes
    return {"workload": "Llama-2-70B-shaped decode layers (M = 1, 8), W8A8 int8 and FP8 codes", "per_case": per_case}


def bench_w4_prefill(ql, reps):
    w = wl.WORKLOADS["w4a16_prefill"]
    M, (K, N) = w.Ms[0], w.shapes[0]
    _, blobs = _prepare_w4(ql, w, K, N, 1)
    X = wl.activations(w, M, K, N).cuda()
    Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
    lf = ql.q4_gemm_launcher(X, blobs[0], N, Y)
    f = lambda r: lf()
    (t,) = time_launches([f], reps, torch.cuda.current_stream())
    ops = 2.0 * M * N * K
    return {"workload": w.name, "M": M, "K": K, "N": N, "us": round(t * 1e3, 1),
            "TFLOPS": round(ops / (t * 1e-3) / 1e12, 1), "frac_mfma_bf16": round(ops / (t * 1e-3) / MFMA_PEAK["bf16"], 4)}


def bench_mid_m(ql, reps):
    """W4A16 with 32 .. 256 tokens (the large-M kernel's small tiles), each
    (M, K, N) case timed on its own, weights rotated over copies larger than
    the last-level cache.  Beside each case: the plain read of the layer's
    weight bytes (read_us) and the case's time against it (frac_of_read)."""
    w = wl.WORKLOADS["mid_m_7b"]
    per_case = {}
    st = torch.cuda.current_stream()
    for (K, N) in w.shapes:
        R = _copies_for(ql.q4_packed_bytes(N, K))
        _, blobs = _prepare_w4(ql, w, K, N, R)
        # the plain read of the same weight copies (fastest probe configuration):
        # no kernel that reads these bytes once can take less time
        probes = {p: [ql.read_probe_launcher(b, p[1], p[0]) for b in blobs] for p in READ_PROBES}
        read_ms = min(time_launches([lambda i, f=f: f[i % R]()], max(reps, 2 * R), st)[0] for f in probes.values())
        for M in w.Ms:
            X = wl.activations(w, M, K, N).cuda()
            Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
            need = ql.q4_gemm_workspace_bytes(M, N, K)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
            launchers = [ql.q4_gemm_launcher(X, blobs[r], N, Y, workspace=ws) for r in range(R)]
            # one entry cycling over all copies (> the last-level cache) per timed block
            fn = lambda r, ls=launchers: ls[r % len(ls)]()
            (t,) = time_launches([fn], max(reps, R), torch.cuda.current_stream())
            # the case's own roofline: the larger of the HBM time of its bytes
            # and the MFMA time of its products
            t_hbm = w4a16_bytes(M, K, N) / (HBM_PEAK_GBS * 1e9)
            t_mfma = 2.0 * M * N * K / MFMA_PEAK["f16"]
            rows, cols, splits = ql.q4_gemm_plan(M, N, K)
            per_case[f"{M}x{K}x{N}"] = {"us": round(t * 1e3, 2),
                                        "TFLOPS": round(2.0 * M * N * K / (t * 1e-3) / 1e12, 1),
                                        "GBps": round(w4a16_bytes(M, K, N) / (t * 1e-3) / 1e9, 1),
                                        "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                                        "frac_roofline": round(max(t_hbm, t_mfma) / (t * 1e-3), 4),
                                        "read_us": round(read_ms * 1e3, 2),
                                        "frac_of_read": round(read_ms / t, 4),
                                        "tile": f"{rows}x{cols}", "k_splits": splits}
        del blobs
    return {"workload": w.name, "per_case": per_case}


def bench_library_refs(reps):
    """The vendor libraries on the same shapes, as context for the GEMM
    figures (not part of the layer): hipBLASLt's bare int8 product through
    torch._int_mm, its FP8 E4M3 product with one scale per tensor through
    torch._scaled_mm, and the dense bf16 product of the W4A16 prefill shape
    through torch.matmul, all on random data, timed like the extra workloads.
    Beside the per-token quant kernel: torch's elementwise kernel with the
    same traffic per value (reads 2 bytes, writes 1: x != 0 into a bool
    tensor) on the W8A8 activation shape, with no reduction in between."""
    st = torch.cuda.current_stream()
    out = {}
    Mq, Kq = 2048, 4096
    Xq = _activation_copies(torch.randn(Mq, Kq, device="cuda", dtype=torch.bfloat16))
    Bq = torch.empty(Mq, Kq, device="cuda", dtype=torch.bool)
    # torch's eager launch costs more host time than this kernel takes on the
    # device, so the launches are captured in a graph (one launch per copy,
    # rotating over copies larger than the last-level cache) and the graph is
    # replayed; eager launches only if capture is not available
    try:
        torch.ne(Xq[0], 0, out=Bq)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for x in Xq:
                torch.ne(x, 0, out=Bq)
        (t,) = time_launches([lambda r: g.replay()], max(10, reps // 5), st)
        t /= len(Xq)
        how = "graph replay"
        del g
    except Exception:
        (t,) = time_launches([lambda r: torch.ne(Xq[r % len(Xq)], 0, out=Bq)], reps, st)
        how = "eager"
    out["elementwise_bf16_to_bool_2048x4096"] = {"us": round(t * 1e3, 2),
                                                 "GBps": round(3 * Mq * Kq / (t * 1e-3) / 1e9, 1), "launch": how}
    del Xq, Bq
    M, N, K = 2048, 4096, 4096
    A = torch.randint(-128, 127, (M, K), dtype=torch.int8, device="cuda")
    B = torch.randint(-127, 127, (N, K), dtype=torch.int8, device="cuda")
    Bt = B.t()
    (t,) = time_launches([lambda r: torch._int_mm(A, Bt)], reps, st)
    out["int8_int_mm_2048x4096x4096"] = {"us": round(t * 1e3, 2), "TOPS": round(2 * M * N * K / (t * 1e-3) / 1e12, 1)}
    try:
        a = (torch.randn(M, K, device="cuda") * 0.5).to(torch.float8_e4m3fn)
        b = (torch.randn(N, K, device="cuda") * 0.5).to(torch.float8_e4m3fn)
        one = torch.tensor(1.0, device="cuda")
        (t,) = time_launches([lambda r: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.float16)],
                             reps, st)
        out["fp8_scaled_mm_per_tensor_2048x4096x4096"] = {"us": round(t * 1e3, 2),
                                                          "TFLOPS": round(2 * M * N * K / (t * 1e-3) / 1e12, 1)}
    except Exception as e:                    # an FP8 path this torch build does not offer
        out["fp8_scaled_mm_per_tensor_2048x4096x4096"] = {"unavailable": str(e)[:120]}
    Mx, Kx, Nx = 4096, 4096, 14336
    X = torch.randn(Mx, Kx, device="cuda", dtype=torch.bfloat16)
    W = torch.randn(Nx, Kx, device="cuda", dtype=torch.bfloat16) * 0.02
    Wt = W.t()
    (t,) = time_launches([lambda r: torch.matmul(X, Wt)], max(10, reps // 3), st)
    out["bf16_dense_matmul_4096x4096x14336"] = {"us": round(t * 1e3, 1),
                                               "TFLOPS": round(2 * Mx * Nx * Kx / (t * 1e-3) / 1e12, 1),
                                               "frac_mfma_bf16": round(2 * Mx * Nx * Kx / (t * 1e-3) / MFMA_PEAK["bf16"], 4)}
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=20.0):
    """The oracle as it is (untuned) on the host cores.

    W4A16 (the headline's unit): explicit fp64 dequant + fp64 BLAS product,
    whole cases of the 70B decode workload in step order until about budget_s
    seconds (the codes of a layer are prepared, untimed, when the sample first
    reaches it).  W8A8: per-token quant + exact integer product + epilogue on
    the M = 2048, K = N = 4096 workload, median of 3."""
    from oracle import w4a16 as ow4
    from oracle import w8a8 as ow8
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = wl.WORKLOADS["decode_70b"]
    cases = w.all_cases()
    prep = {}
    nbytes, done, busy = 0, 0, 0.0
    while busy < budget_s:
        c = cases[done % len(cases)]
        L = (c[1], c[2])
        if L not in prep:
            prep[L] = ow4.quantize_w4(_weight(w, *L))
        X = wl.as_f64(wl.activations(w, *c))
        t0 = time.perf_counter()
        ow4.w4a16_linear(X, *prep[L])
        busy += time.perf_counter() - t0
        nbytes += w4a16_bytes(*c)
        done += 1
    del prep
    # W8A8: quantize the activations, exact integer product, epilogue
    w8 = wl.WORKLOADS["w8a8_prefill"]
    M, (K, N) = w8.Ms[0], w8.shapes[0]
    Xf = wl.as_f64(wl.activations(w8, M, K, N)).astype(np.float32)
    Bq, s_b = ow8.quant_weight_per_channel_sym(wl.weight(w8, K, N))
    adj = ow8.azp_adj(Bq)
    bias = wl.as_f64(wl.bias(w8, N))
    t8 = []
    for _ in range(3):
        t0 = time.perf_counter()
        Aq, s_a, azp = ow8.quant_per_token_asym(Xf)
        ow8.w8a8_linear(Aq, Bq, s_a, s_b, azp, adj, bias)
        t8.append(time.perf_counter() - t0)
    t8m = float(np.median(t8))
    return {"value": round(nbytes / busy / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole cases of the 70B decode workload in step order "
                      f"({done / len(cases):.2f} steps), {busy:.1f} s of oracle time (explicit fp64 dequant + "
                      f"fp64 BLAS product per case; quantization untimed)",
            "cpu_model": _cpu_model(), "blas_threads": int(threads),
            "w8a8": {"workload": w8.name, "median_of_3_s": round(t8m, 4),
                     "GOPS": round(2.0 * M * N * K / t8m / 1e9, 2),
                     "what": "per-token asymmetric int8 quant + exact integer product (fp64 BLAS on integer "
                             "values) + zero-point correction and epilogue"}}


def main():
    global WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--no-per-case", action="store_true",
                    help="time only the main step (no per-case or read-ceiling blocks)")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS, metavar="MS",
                    help="back-to-back launches of a kernel before its timed block in the per-kernel figures")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reference for byte counters)")
    ap.add_argument("--also-only", default="", metavar="NAMES",
                    help="run only these extra workloads (comma-separated: decode_7b, w8a8, fp8, w8a8_decode, "
                         "prefill, mid_m, libref)")
    args = ap.parse_args()
    WARM_MS = args.warm_ms
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the layer would shard "
              "column-parallel with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import quantized_linear_layers_amd as ql
    ql.lib()
    torch.cuda.init()
    dev = torch.cuda.get_device_properties(0)
    print(f"# device: {dev.name} ({getattr(dev, 'gcnArchName', '?')}), {dev.multi_processor_count} CUs", flush=True)

    if args.copy_calib > 0:
        copy_calibration(args.copy_calib)
    main_res = bench_decode(ql, "decode_70b", args.steps, args.warmup, per_case=not args.no_per_case)
    print(f"# decode_70b: {main_res['value_gbs']:.1f} GB/s per step", flush=True)
    if "per_case" in main_res:
        print(f"# decode_70b read ceiling: {main_res['read_ceiling_step']}", flush=True)
        print(f"# decode_70b per case: {main_res['per_case']}", flush=True)
    also = {}
    want = set(filter(None, args.also_only.split(","))) or {"decode_7b", "w8a8", "fp8", "w8a8_decode", "prefill",
                                                            "mid_m", "libref"}
    if not args.no_also:
        if "decode_7b" in want:
            r7 = bench_decode(ql, "decode_7b", args.steps, args.warmup)
            also["decode_7b"] = {"workload": wl.WORKLOADS["decode_7b"].name, "step_GBps": round(r7["value_gbs"], 1),
                                 "ms_step": round(r7["ms_step"], 5),
                                 "frac_hbm": round(r7["value_gbs"] / HBM_PEAK_GBS, 4),
                                 "read_ceiling_step": r7["read_ceiling_step"], "per_case": r7["per_case"]}
            print(f"# decode_7b: {r7['value_gbs']:.1f} GB/s per step", flush=True)
            del r7
        if "w8a8" in want:
            also["w8a8_prefill"] = bench_w8a8(ql, 50)
            print(f"# w8a8: {also['w8a8_prefill']}", flush=True)
        if "fp8" in want:
            also["w8a8_fp8_prefill"] = bench_f8(ql, 50)
            print(f"# w8a8 fp8: {also['w8a8_fp8_prefill']}", flush=True)
        if "w8a8_decode" in want:
            also["w8a8_decode"] = bench_w8a8_decode(ql, 50)
            print(f"# w8a8 decode: {also['w8a8_decode']}", flush=True)
        if "prefill" in want:
            also["w4a16_prefill"] = bench_w4_prefill(ql, 20)
            print(f"# w4a16 prefill: {also['w4a16_prefill']}", flush=True)
        if "mid_m" in want:
            also["w4a16_mid_m"] = bench_mid_m(ql, 20)
            print(f"# w4a16 mid-M: {also['w4a16_mid_m']}", flush=True)
        if "libref" in want:
            also["library_refs"] = bench_library_refs(50)
            print(f"# library references: {also['library_refs']}", flush=True)

    cpu = None if args.no_cpu else cpu_baseline()
    # the step is nothing but the decode kernel's launches: its mean launch
    # duration is the timed region's elapsed time over the launches in it
    launches = len(main_res["cases"])
    launch_ms = main_res["ms_step"] / launches
    achieved = main_res["bytes_step"] / launches / (launch_ms * 1e-3) / 1e9
    traffic = None
    if TRAFFIC is not None and TRAFFIC["source_sha256"] == _kernel_source_sha():
        traffic = TRAFFIC["bytes_per_launch"]
    w70 = wl.WORKLOADS["decode_70b"]
    line = {
        "metric": METRIC,
        "value": round(main_res["value_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 0.015) fp32 weights quantized to uint4 g=128 with fp16 scales; "
                "bf16 N(0, 1) activations)",
        "config": {"workload": w70.name, "cases_MKN": main_res["cases"], "group": 128,
                   "bytes_per_step": main_res["bytes_step"], "weight_copies": main_res["copies"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "q4_gemv_kernel",
                     "algorithmic_bytes_per_launch": round(main_res["bytes_step"] / launches),
                     "launch_us_mean": round(launch_ms * 1e3, 3),
                     "read_ceiling_step": main_res.get("read_ceiling_step"),
                     "per_case": main_res.get("per_case")},
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
