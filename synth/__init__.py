"""Seeded synthetic inputs for the local-expert MoE block.

This package only draws random inputs (activations, router weights, MXFP4 expert
weights, norm weights, shared-expert weights) with the shapes and value
distributions of the five workloads. It holds none of the block's arithmetic, so
the GPU library and the CPU oracle can both be fed the same bytes from it.
"""

from .configs import CONFIGS, PROJ_CONFIGS, MoeConfig, ProjConfig, get_config  # noqa: F401
from .inputs import make_inputs, make_proj_inputs, f32_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
