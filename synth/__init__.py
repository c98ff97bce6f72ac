"""Seeded synthetic workloads for the int4-expert / int8-router MoE block.

This module is shared by the CPU oracle and the HIP path.  It holds only
random-number generation, the workload shapes and the bf16 bit-pattern
rounding of freshly drawn values; none of the MoE method's arithmetic
(dequantisation, routing, SwiGLU, LoRA, combine) lives here.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    workload,
    f32_to_bf16_bits,
    expert_tensors,
    router_tensors,
    tokens,
    zipf_bias,
    prerouter_tensors,
    prerouter_feat_tensors,
)
