"""CPU oracle for the W8A8 dynamic-quant linear and its FP8 per-token-group variant.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or constant generator with
the HIP kernels under ``fp8_dynamic_quant_amd/csrc``.

The oracle is plain, slow and written to be checked by eye against the pages:

* "DeepSeek-V4 W8A8 性能分析：小 M、NZ 布局与测量方法" (akiyangdev.github.io),
  section 一 (the BF16 X -> dynamic quant -> INT8 X + per-token scale ->
  quant matmul -> BF16 Y chain, and the tuple-reuse snippet), sections 五/六
  (expert-local M_e, grouped matmul over group_list).
* SGLang PR #34277 summary (prhub.com.cn), sections 功能与动机 and 实现拆解
  plus the kernel write-logic and wrapper snippets under 关键文件 (per-token
  group FP8 quant with UE8M0 exponents written packed 4 per int32 into the
  [G, ceil(HG/4), align4(T)] layout, tail-byte zero fill, logical view).
* "重塑大模型推理数据流：DeepSeek V4 950 低精度优化全复盘" (0539edu.com),
  section 2.3 (RMSNorm+quant and SwiGLU+quant fusion) and 3.2 (tokens sorted
  by expert id before the gather).

Modules:
  numerics    bf16 / E4M3FN / UE8M0 encodings written from the format definitions,
              and the fixed-sequence f32 exp used inside SiLU.
  int8_linear per-token INT8 quant, INT32 GEMM, scale epilogue, fused composition.
  fp8_group   per-token-group FP8 quant, packed UE8M0 writer, grouped FP8 contraction.
  moe         expert sort, RMSNorm+quant, segmented GEMM, SwiGLU+requant.
"""

from . import numerics, int8_linear, fp8_group, moe  # noqa: F401
