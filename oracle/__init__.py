"""CPU oracle for the MXFP4 block-scaled MoE expert path (TEST INFRASTRUCTURE ONLY).

This package is the slow, obviously-correct fp64 reference that the HIP kernels
are checked against. It is not part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It imports nothing from ``mxfp4_block_scaled_amd`` and shares no
code, table or constant with the HIP sources.

Sources cited throughout (the pages are web articles; sections are named by
their headings):

* [DS4-FP4] "DGX Spark 原生 FP4 矩阵指令：DwarfStar 如何利用 Blackwell 加速推理"
  - section 一 (what the FP4 MMA is: E2M1 = 1 sign / 2 exponent / 1 mantissa
  bit, UE8M0 block scale, no dequantisation before the MMA), section 二 (only
  routed experts are FP4; dense and MoE entry points), section 三 (K-shape
  guard that errors out instead of silently taking a wrong path).
* [TRITON-FP4] "【DeepSeek V4】Triton FP4 优化实战：近距离感受老黄的刀法"
  - "FP4 MoE GEMM 是什么？" (256 experts, 6 active per token, 2 FC per expert),
  "第二步：Fused Dequant+Matmul Kernel" (expert FC1 is 4096x7168; packed FP4
  with even columns in the low nibble, odd columns in the high nibble).
* [MTT-DSV4] "Domestic GPUs are awesome! Moore thread full-link adaptation
  DeepSeek-V4" - the fused "SwiGLU + FP8 quant" pattern, MoE routing (Top-k),
  dispatch/combine.
* [FP8-GGUF] "企业官网建设流程全解析" (ik_llama.cpp FP8 GGUF PR) - section 一:
  E4M3 = 4 exponent + 3 mantissa bits.
* [OCP-MX] The OCP Microscaling Formats (MX) v1.0 specification: the shared
  scale X = floor(log2(amax)) - emax_elem, E8M0 scale with bias 127, element
  conversion with round-to-nearest-even and clamping to the largest normal.

Readings of points the pages leave open are listed in the module docstrings
where they are used.
"""

from .mx import (  # noqa: F401
    E2M1_EMAX,
    E4M3_EMAX,
    e2m1_decode,
    e4m3_decode,
    ue8m0_decode,
    pack_e2m1,
    unpack_e2m1,
    bf16_bits_to_f64,
    mx_scale_byte,
    round_to_grid,
    mx_quantize,
    mx_dequantize,
    dequant_weights,
    ue4m3_decode,
    dequant_nvfp4_weights,
)
from .moe import (  # noqa: F401
    dense_gemm,
    w4a16_gemm,
    q8_quantize,
    lut_int8_weights,
    q8_gemm,
    route_topk,
    permute,
    swiglu,
    moe_layer,
    fc1_swiglu_rows,
    fc1_abs_terms,
    group_max_terms,
    fc2_rows,
    combine,
    row_normalised_error,
)
