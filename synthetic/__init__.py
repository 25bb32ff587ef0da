"""Seeded synthetic inputs (no layer arithmetic); shared by the oracle tests and the HIP tests."""
from .moe_inputs import (CONFIGS, LayerShape, bf16_bits_to_f32, f32_to_bf16_bits, gen_bias,  # noqa: F401
                         gen_expert, gen_expert_encoded, gen_experts, gen_layer, gen_router,
                         gen_shared, gen_x, quantise_mxfp4, quantise_mxfp8)
