"""CPU oracle (float64) for the BailingMoeV3 sparse MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The HIP library never calls it and shares no code
with it.
"""
from .moe_oracle import (E4M3_MAX, Dispatch, Routing, act_mxfp8, bf16_to_f64, dispatch,  # noqa: F401
                         e4m3_value, expert_forward, expert_hidden, moe_layer, mxfp4_dequant,
                         mxfp8_dequant, mxfp8_quantise, route, router_logits, swiglu,
                         update_expert_bias)
