"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module holds no part of the FP8 method: it only draws random bf16 inputs
(and the MoE routing: top-k expert ids, gate weights, counts) of the shapes
and value distributions of the benchmark configurations.  Both the CPU oracle and the HIP library are fed
from here; neither imports the other.

Shapes follow the pages' model: hidden size 7168, MLA query latent 1536 and
KV latent 512 with 128 heads of 128 (K) + 128 (V), MoE with 256 routed experts
and top-8 routing, expert FFN width 2048 (gate and up fused: 4096)
("DeepSeek-V3 技术报告深度解读", section 2; deepseek.csdn.net page, section 一).

Recipe (host side, numpy PCG64):
  * seed = configuration number; ``SeedSequence(seed).spawn(4)`` gives the
    streams for (A / X / dY, B / W, outlier choice, routing);
  * values are drawn as float32 normals, outliers are multiplied in float32,
    and the result is rounded to bf16 (nearest, ties to even);
  * "1% of channels/rows" is round(0.01 * dim) distinct indices chosen without
    replacement.
Expert weights of the MoE configuration (256 x 4096 x 7168, 7.5 G values) are
too large to draw on the host in reasonable time; ``device_expert_weights``
draws them on the GPU with a seeded torch generator instead, and tests copy
back the experts they check.
"""

from .configs import CONFIGS, config_by_name
from .gen import (
    f32_to_bf16_bits,
    gemm_inputs,
    layer_inputs,
    wgrad_inputs,
    moe_routing,
    moe_dispatch_inputs,
    grouped_inputs_host,
    device_expert_weights,
    normal_bf16,
)

__all__ = [
    "CONFIGS", "config_by_name", "f32_to_bf16_bits", "gemm_inputs", "layer_inputs", "wgrad_inputs",
    "moe_routing", "moe_dispatch_inputs", "grouped_inputs_host", "device_expert_weights", "normal_bf16",
]
