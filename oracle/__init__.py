"""CPU oracle for the quantized linear layer (test infrastructure only).

This package is the independent reference that the HIP path is checked
against.  It is NOT part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``quantized_linear_layers_amd`` (no
kernels, headers, helpers, tables or constants); the only module both sides
use is ``workloads`` (seeded input draws, which hold none of the method's
arithmetic).

Everything here is plain NumPy: explicit quantize / dequantize, then an fp64
matrix product, and an exact integer product for W8A8.  Decisions that turn
floating point into an integer code are taken in IEEE fp32 (true division,
round-half-to-even), because that is the precision the device takes them in;
everything else is fp64.

Sources, cited by page title and the page's own section heading:

[QK]  "第 9 章 量化 Kernel：INT8 / FP8 / INT4" (Quantization kernels:
      INT8 / FP8 / INT4), chapter 9 of the online book "CUDA 算子工程：手写
      FlashAttention v2 之路", yangyitao.com.
[LQ]  "LLM 与 AIGC 量化：从数值格式到 W4A4" (LLM and AIGC quantization: from
      number formats to W4A4), valdrada.cn.
[VE]  "vLLM W8A8 量化 GEMM 的 CUTLASS Epilogue 设计：反量化融合的数学推导与源码
      实现" (the CUTLASS epilogue design of vLLM's W8A8 GEMM), blog.gitcode.com.
[CP]  "CUDA-Practice：07 FP16 带宽翻倍、INT8 dp4a 指令与混合精度工程学",
      smarter.xin.

Every function is pinned by a ``-m "not gpu"`` test against values the pages
print, closed forms, invariants or brute force (tests/test_oracle_*.py).
"""

from . import fp8, numerics, quant, rmsnorm, w4a16, w8a8  # noqa: F401
