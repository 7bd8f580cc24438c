"""CPU oracle for the block-scaled FP8 GEMM path.  TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct restatement of the FP8
fine-grained quantization scheme and the GEMMs that consume it, written in
numpy with float64 accumulation.  It exists to check the HIP kernels; only the
test suite, the smoke entry point and the CPU-baseline leg of the benchmark may
import it.  The product path (the C-ABI library and its Python binding) never
imports, links or calls anything here, and this package never imports the
product path.

What the method computes comes from these pages (cited by title and section):

* "DeepSeek-V3 技术报告深度解读" (sherconan.github.io), section 3
  "FP8 混合精度训练": every GEMM of a layer (forward, activation gradient,
  weight gradient) runs in FP8; activations are quantized per 1x128 tile and
  weights per 128x128 block; partial sums are moved into FP32 after each
  128-element stretch of the contraction.
* deepseek.csdn.net page, section 二(四) "FP8 低精度训练", and the qqstock.cn
  page, section "FP8 低精度訓練：精度與效率的平衡": the same tile/block
  granularity (instead of one scale per tensor) and FP32 accumulation of the
  matrix-multiply partials.

The pages do not fix the 8-bit format, the scale rule, the rounding or the
layouts.  The readings taken here (OCP E4M3 "fn", scale = amax/448 in IEEE
binary32, binary32 division then round-to-nearest-even with saturation,
row-major layouts, tiles along each GEMM's contraction) are listed with the
reason for each in the design notes of the repository.

Modules
-------
e4m3      exact decode table and RNE/saturating encoder for OCP E4M3
bf16      bfloat16 <-> float conversions (exact decode, RNE encode)
quantize  1x128 activation tiles, 128x128 weight blocks, transposed tiles,
          re-tiling of a cached (FP8) activation along its rows
gemm      block-scaled GEMMs: forward (NT), activation gradient (NN),
          weight gradient (per-row scales on both operands), MoE grouped
moe       MoE dispatch layout (expert-major, 128-padded segments), dispatch
          payload (gather + 1x128 quantize), combine (gate-weighted sum, bf16)

Pinning: every function here is checked by the CPU tests against facts that do
not come from this code (closed forms, exhaustive enumeration, exact rational
brute force, textbook special cases).  No function here is "parity unpinned".
"""

from .e4m3 import E4M3_MAX, e4m3_decode_table, e4m3_decode, e4m3_encode
from .bf16 import bf16_to_f32, f32_to_bf16_rne, f64_to_bf16_rne
from .quantize import (quantize_act_1x128, quantize_act_1x128_t, quantize_w_128x128, dequantize_act_1x128,
                       requantize_act_1x128_t, quantize_per_tensor)
from .gemm import gemm_fprop, gemm_dgrad, gemm_wgrad, grouped_gemm, gemm_dequant_reference
from .moe import moe_max_rows, moe_route, moe_permute_quantize, moe_combine, moe_combine_exact

__all__ = [
    "E4M3_MAX", "e4m3_decode_table", "e4m3_decode", "e4m3_encode",
    "bf16_to_f32", "f32_to_bf16_rne", "f64_to_bf16_rne",
    "quantize_act_1x128", "quantize_act_1x128_t", "quantize_w_128x128", "dequantize_act_1x128",
    "requantize_act_1x128_t", "quantize_per_tensor",
    "gemm_fprop", "gemm_dgrad", "gemm_wgrad", "grouped_gemm", "gemm_dequant_reference",
    "moe_max_rows", "moe_route", "moe_permute_quantize", "moe_combine", "moe_combine_exact",
]
