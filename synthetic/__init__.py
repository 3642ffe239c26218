"""Seeded synthetic inputs for the NVFP4 W4A4 routed-expert MoE block.

This package only draws random numbers and shapes them: bf16 activations,
fp32 router logits and bf16 expert weights.  It holds none of the method's
arithmetic (no quantisation, no scale derivation, no routing), so both the
CPU oracle and the GPU library can take their inputs from it.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    activations,
    router_logits,
    expert_weights,
    calibration_batch,
    bad_scale_slots,
    outlier_channels,
)
