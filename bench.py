"""Throughput of the quantized linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-also]

The main line is the W4A16 decode GEMV on the Llama-2-7B-shaped layers
(M in {1, 4, 16} x (K, N) in {(4096, 4096), (4096, 11008), (11008, 4096)},
g = 128, fp16 activations with 1% outlier channels).  One step runs all nine
(M, K, N) cases once.  `value` is the effective bandwidth of a whole step:
algorithmic bytes (packed weights + fp16 scales + 4-bit zeros + X + Y) over
the step's wall time, inputs resident in HBM.  Each step reads a different
copy of the weights (copies rotate so that the working set exceeds 1 GiB, four
times the 256 MB Infinity Cache), so the weights come from HBM, not cache.

The steps are launched on one stream with their arguments marshalled once
(--graphs replays them as HIP graphs instead, one graph per weight copy, after
checking every graph's outputs bit-for-bit against eager launches; on this
stack graph replay of these short kernels measured slower than stream
launches).  The step contains only the decode kernel, so the roofline
object's mean launch duration is the timed region's elapsed time (HIP events
on the launch stream) over its launches.  `per_case_eager` adds a second pass of eager launches,
each bracketed by HIP events (which adds the event overhead to each figure).
The `also` object holds the other workloads (70B decode, W8A8 prefill GEMM
with int8 and with FP8 codes, W4A16 prefill GEMM).
"""

import argparse
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

# HBM traffic of the decode kernel per launch (mean over the nine cases of a
# step), from two counter runs (FETCH_SIZE, then WRITE_SIZE) each scaled by
# what the same counter reads for a plain device copy of known size in the
# same run.  It belongs to one version of the kernel source: when the source
# hash differs, the figure is stale and `traffic` is reported as null.
TRAFFIC = {"source_sha256": "a520aa56e5ef08ed818808b749d50a30805789505bc0bd79ee906c7941d1fbd3",
           "bytes_per_launch": 19387981}


def w4a16_bytes(M, K, N, group=128, e=2):
    """Algorithmic bytes of one W4A16 layer: packed codes, fp16 scales, 4-bit
    zero points, X and Y (the data the method has to move, not the fp16 weights
    it avoids)."""
    return K * N // 2 + (K // group) * N * 2 + (K // group) * N // 2 + M * K * e + M * N * e


def _events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _prepare_w4(ql, w, K, N, copies):
    W = wl.weight(w, K, N)
    wq, s, z = ql.q4_quantize_host(torch.from_numpy(W))
    blob = ql.q4_pack(wq, s, z, N, K)
    return W, [blob.to("cuda") for _ in range(copies)]


def _copies_for(total_bytes):
    return max(2, -(-MALL_DEFEAT_BYTES // max(total_bytes, 1)))


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


WARM_MS = 10.0                    # warm-up per timed kernel (--warm-ms)


def warm(fn_list, ms=30.0, cap=5000):
    """Runs the launches back to back for about `ms` of GPU time, so that the
    timed ones start at the clock a sustained load settles at (an idle part
    ramps its clock up over the first milliseconds of work)."""
    s = torch.cuda.current_stream()
    a, b = _events()
    a.record(s)
    for fn in fn_list:
        fn(0)
    b.record(s)
    torch.cuda.synchronize()
    n = min(cap, max(1, int(ms / max(a.elapsed_time(b), 1e-3))))
    for i in range(n):
        for fn in fn_list:
            fn(i)
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
    return out


def bench_decode(ql, wname, steps, warmup, use_graphs=False):
    """Runs a W4A16 decode workload; returns a dict of results."""
    w = wl.WORKLOADS[wname]
    cases = w.all_cases()
    shapes = list(w.shapes)
    blob_bytes = sum(ql.q4_packed_bytes(N, K) for (K, N) in shapes)
    R = _copies_for(blob_bytes)
    blobs = {}
    for (K, N) in shapes:
        _, blobs[(K, N)] = _prepare_w4(ql, w, K, N, R)
    X = {c: wl.activations(w, c[0], c[1], c[2]).cuda() for c in cases}
    Y = {c: torch.empty((c[0], c[2]), dtype=X[c].dtype, device="cuda") for c in cases}
    stream = torch.cuda.current_stream()
    # launchers with the arguments marshalled once (the host cost of a
    # launch must stay below the kernel's few microseconds)
    launchers = [[ql.q4_gemm_launcher(X[c], blobs[(c[1], c[2])][r], c[2], Y[c]) for c in cases] for r in range(R)]

    def launch(c, r):
        M, K, N = c
        ql.q4_gemm(X[c], blobs[(K, N)][r], N, Y=Y[c])

    def step(r):
        if use_graphs:            # capture runs on its own stream: marshal per call
            for c in cases:
                launch(c, r)
        else:
            for f in launchers[r]:
                f()

    for r in range(min(R, warmup + 1)):
        step(r)
    torch.cuda.synchronize()
    bytes_step = sum(w4a16_bytes(*c) for c in cases)

    graphs = None
    if use_graphs:
        ref = {}
        for r in range(R):
            step(r)
            torch.cuda.synchronize()
            ref[r] = {c: Y[c].clone() for c in cases}
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        for rep in range(2):                      # every replay must equal the eager result
            for r in range(R):
                for c in cases:
                    Y[c].zero_()
                graphs[r].replay()
                torch.cuda.synchronize()
                for c in cases:
                    if not torch.equal(Y[c], ref[r][c]):
                        raise RuntimeError(f"graph replay {rep} of copy {r} differs from eager on case {c}")

    run = (lambda i: graphs[i % R].replay()) if graphs else (lambda i: step(i % R))
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    a, b = _events()
    a.record(stream)
    for i in range(steps):
        run(i)
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / steps

    # per-case durations (each case alone, back to back over the weight copies)
    fns = [(lambda r, i=i: launchers[r % R][i]()) for i in range(len(cases))]
    per = time_launches(fns, max(steps, 10), stream)
    kern_ms = float(per.sum())
    per_case = []
    for c, ms in zip(cases, per):
        gbs = w4a16_bytes(*c) / (ms * 1e-3) / 1e9
        per_case.append({"M": c[0], "K": c[1], "N": c[2], "us": round(ms * 1e3, 3),
                         "GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
    return {
        "cases": cases, "bytes_step": bytes_step, "ms_step": ms_step,
        "value_gbs": bytes_step / (ms_step * 1e-3) / 1e9,
        "kernel_ms_step": kern_ms, "kernel_gbs": bytes_step / (kern_ms * 1e-3) / 1e9,
        "per_case": per_case, "copies": R, "graphs": bool(graphs),
    }


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
    the last-level cache."""
    w = wl.WORKLOADS["mid_m_7b"]
    per_case = {}
    for (K, N) in w.shapes:
        R = _copies_for(ql.q4_packed_bytes(N, K))
        _, blobs = _prepare_w4(ql, w, K, N, R)
        for M in w.Ms:
            X = wl.activations(w, M, K, N).cuda()
            Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
            launchers = [ql.q4_gemm_launcher(X, blobs[r], N, Y) for r in range(R)]
            # one entry cycling over all copies (> the last-level cache) per timed block
            fn = lambda r, ls=launchers: ls[r % len(ls)]()
            (t,) = time_launches([fn], max(reps, R), torch.cuda.current_stream())
            per_case[f"{M}x{K}x{N}"] = {"us": round(t * 1e3, 2),
                                        "TFLOPS": round(2.0 * M * N * K / (t * 1e-3) / 1e12, 1),
                                        "GBps": round(w4a16_bytes(M, K, N) / (t * 1e-3) / 1e9, 1)}
        del blobs
    return {"workload": w.name, "per_case": per_case}


def cpu_baseline(budget_s=20.0):
    """The oracle (explicit dequant + fp64 product), untuned, on the host cores,
    over whole steps of the 7B decode workload until about budget_s seconds."""
    from oracle import w4a16 as ow4
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = wl.WORKLOADS["decode_7b"]
    cases = w.all_cases()
    prep = {}
    for (K, N) in w.shapes:
        prep[(K, N)] = ow4.quantize_w4(wl.weight(w, K, N))
    Xs = {c: wl.as_f64(wl.activations(w, *c)) for c in cases}
    nbytes, t0, done = 0, time.perf_counter(), 0
    while True:
        for c in cases:
            q, s, z = prep[(c[1], c[2])]
            ow4.w4a16_linear(Xs[c], q, s, z)
            nbytes += w4a16_bytes(*c)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} case runs cycling over the 9 (M, K, N) decode cases of the 7B workload "
                      f"({done / len(cases):.1f} steps) in {dt:.1f} s "
                      f"(explicit fp64 dequant + fp64 BLAS product per case; quantization untimed)"}


def main():
    global WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS, metavar="MS",
                    help="back-to-back launches of a kernel before its timed block (small under a profiler)")
    ap.add_argument("--graphs", action="store_true", help="replay the decode steps as HIP graphs")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reference for byte counters)")
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
    main_res = bench_decode(ql, "decode_7b", args.steps, args.warmup, use_graphs=args.graphs)
    print(f"# decode_7b: {main_res['value_gbs']:.1f} GB/s per step, kernels {main_res['kernel_gbs']:.1f} GB/s",
          flush=True)
    also = {}
    if not args.no_also:
        r70 = bench_decode(ql, "decode_70b", max(10, args.steps // 2), args.warmup, use_graphs=args.graphs)
        also["decode_70b"] = {"workload": wl.WORKLOADS["decode_70b"].name, "step_GBps": round(r70["value_gbs"], 1),
                              "kernel_GBps": round(r70["kernel_gbs"], 1),
                              "frac_hbm": round(r70["kernel_gbs"] / HBM_PEAK_GBS, 4), "per_case": r70["per_case"]}
        print(f"# decode_70b: kernels {r70['kernel_gbs']:.1f} GB/s", flush=True)
        also["w8a8_prefill"] = bench_w8a8(ql, 50)
        print(f"# w8a8: {also['w8a8_prefill']}", flush=True)
        also["w8a8_fp8_prefill"] = bench_f8(ql, 50)
        print(f"# w8a8 fp8: {also['w8a8_fp8_prefill']}", flush=True)
        also["w4a16_prefill"] = bench_w4_prefill(ql, 20)
        print(f"# w4a16 prefill: {also['w4a16_prefill']}", flush=True)
        also["w4a16_mid_m"] = bench_mid_m(ql, 20)
        print(f"# w4a16 mid-M: {also['w4a16_mid_m']}", flush=True)

    cpu = None if args.no_cpu else cpu_baseline()
    # the step is nothing but the decode kernel's launches: its mean launch
    # duration is the timed region's elapsed time over the launches in it
    launches = len(main_res["cases"])
    launch_ms = main_res["ms_step"] / launches
    achieved = main_res["bytes_step"] / launches / (launch_ms * 1e-3) / 1e9
    traffic = None
    if TRAFFIC is not None and TRAFFIC["source_sha256"] == _kernel_source_sha():
        traffic = TRAFFIC["bytes_per_launch"]
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
        "dtype": "f16",
        "data": "synthetic (seeded N(0, 0.02) fp32 weights quantized to uint4 g=128; fp16 N(0, 1) "
                "activations with 1% channels x20)",
        "config": {"workload": wl.WORKLOADS["decode_7b"].name, "cases_MKN": main_res["cases"], "group": 128,
                   "bytes_per_step": main_res["bytes_step"], "weight_copies": main_res["copies"],
                   "hip_graphs": main_res["graphs"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "q4_gemv_kernel",
                     "algorithmic_bytes_per_launch": round(main_res["bytes_step"] / launches),
                     "launch_us_mean": round(launch_ms * 1e3, 3),
                     "per_case_eager": main_res["per_case"]},
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
