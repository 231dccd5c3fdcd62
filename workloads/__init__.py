"""Seeded synthetic workloads shared by the oracle side and the device side.

This module holds NO arithmetic of the method (no quantization, packing,
dequantization or products): only the workload descriptions and the
seeded random draws of their fp32 weights, 16-bit activations and biases.
Both the tests/bench (device side) and the oracle consume these draws.

Recipe (the same for every workload): one NumPy ``default_rng`` per tensor,
seeded with ``SeedSequence([seed, workload_id, M, K, N, tensor_id])`` where
tensor_id is 0 = W, 1 = X, 2 = outlier channel set, 3 = bias, 4 = RMSNorm gain.  W is drawn
with M = 0 so that every M of a (K, N) layer shares one weight.  W =
standard_normal((N, K)) * w_std (fp32); X = standard_normal((M, K)) + x_mean
(fp32); if the workload has outliers, round(0.01 * K) input channels, chosen
without replacement, are scaled by 20 in every row; X is then rounded
(nearest-even) to the activation dtype by torch's CPU cast.
"""

from dataclasses import dataclass
from typing import Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    mode: str                     # "w4a16" or "w8a8"
    Ms: Tuple[int, ...]
    shapes: Tuple[Tuple[int, int], ...]   # (K, N) pairs
    x_dtype: str                  # "f16" or "bf16"; the output uses the same dtype
    w_std: float
    x_mean: float = 0.0
    outliers: bool = False
    bias_std: float = 0.0
    group: int = 128
    seed: int = 0

    def all_cases(self):
        """(M, K, N) triples of this workload."""
        return [(M, K, N) for (K, N) in self.shapes for M in self.Ms]


WORKLOADS = {
    "tiny_gemv": Workload(0, "W4A16 tiny GEMV (M=1, K=N=256, g=128)", "w4a16",
                          (1,), ((256, 256),), "f16", 0.02),
    "decode_7b": Workload(1, "W4A16 decode, Llama-2-7B-shaped layers", "w4a16",
                          (1, 4, 16), ((4096, 4096), (4096, 11008), (11008, 4096)),
                          "f16", 0.02, outliers=True),
    "decode_70b": Workload(2, "W4A16 decode, Llama-2-70B-shaped layers", "w4a16",
                           (1, 8), ((8192, 8192), (8192, 28672), (28672, 8192)),
                           "bf16", 0.015),
    "w8a8_prefill": Workload(3, "W8A8 prefill GEMM (M=2048, K=N=4096)", "w8a8",
                             (2048,), ((4096, 4096),), "f16", 0.02, x_mean=0.3,
                             bias_std=0.1),
    "w4a16_prefill": Workload(4, "W4A16 prefill GEMM (M=4096, K=4096, N=14336)", "w4a16",
                              (4096,), ((4096, 14336),), "bf16", 0.02),
    "mid_m_7b": Workload(5, "W4A16 mid-M (batched decode), Llama-2-7B-shaped layers", "w4a16",
                         (32, 64, 128, 256), ((4096, 4096), (4096, 11008), (11008, 4096)),
                         "f16", 0.02, outliers=True),
}


def _rng(wl, M, K, N, t):
    return np.random.default_rng(np.random.SeedSequence([wl.seed, wl.wid, M, K, N, t]))


def weight(wl, K, N):
    """fp32 [N, K] weight draw, shared by every M of this (K, N) layer."""
    r = _rng(wl, 0, K, N, 0)
    return (r.standard_normal((N, K), dtype=np.float32) * np.float32(wl.w_std)).astype(np.float32)


def activations_f32(wl, M, K, N):
    """fp32 [M, K] activation draw before the cast to the 16-bit dtype."""
    r = _rng(wl, M, K, N, 1)
    X = r.standard_normal((M, K), dtype=np.float32)
    if wl.x_mean:
        X = X + np.float32(wl.x_mean)
    if wl.outliers and K > 0:
        n_out = int(round(0.01 * K))
        idx = _rng(wl, M, K, N, 2).choice(K, n_out, replace=False)
        X[:, idx] *= np.float32(20)
    return X


def activations(wl, M, K, N):
    """16-bit activations as a CPU torch tensor [M, K] (fp16 or bf16)."""
    import torch
    dt = torch.float16 if wl.x_dtype == "f16" else torch.bfloat16
    return torch.from_numpy(activations_f32(wl, M, K, N)).to(dt)


def bias(wl, N):
    """fp16 bias [N] (W8A8 workload), as a CPU torch tensor."""
    import torch
    r = _rng(wl, 0, 0, N, 3)
    b = r.standard_normal(N, dtype=np.float32) * np.float32(wl.bias_std)
    return torch.from_numpy(b).to(torch.float16)


def norm_weight(wl, K):
    """RMSNorm gain [K] in the activation dtype, as a CPU torch tensor:
    1 + 0.2 * N(0, 1) (tensor id 4)."""
    import torch
    r = _rng(wl, 0, K, 0, 4)
    g = r.standard_normal(K, dtype=np.float32) * np.float32(0.2) + np.float32(1.0)
    dt = torch.float16 if wl.x_dtype == "f16" else torch.bfloat16
    return torch.from_numpy(g).to(dt)


def as_f64(t):
    """Exact float64 NumPy copy of a CPU torch tensor of any float dtype."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
