"""Builds libqlinear.so in-tree with hipcc for gfx950.

    python -m quantized_linear_layers_amd.build        (or __graft_entry__.build())

Every source is compiled (in parallel) on each call; objects go to ``_build/``
at the repository root and the shared library next to this file.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlinear.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]
SOURCES = {
    "abi.cpp": [],
    "host_quant.cpp": ["-ffp-contract=off"],
    # "-amdgpu-kernarg-preload-count=n": the kernels' first n arguments are
    # preloaded into scalar registers at wave launch (no argument loads
    # before the first copy)
    "q4_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=9"],
    "q4_gemm.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"],
    "i8_quant.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-kernarg-preload-count=8"],
    "i8_gemm.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=6"],
    "i8_gemm_small.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=6"],
    "i8_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=5"],
    "act_order.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"],
    "read_probe.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=4"],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqlinear.so)")


def _compile(src, extra, verbose):
    out = os.path.join(OBJ, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + COMMON + extra + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    return out, msg.strip()


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = [ex.submit(_compile, s, e, verbose) for s, e in SOURCES.items()]
        objs = []
        for f in futs:
            o, msg = f.result()
            if msg and verbose:
                print(msg)
            objs.append(o)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
