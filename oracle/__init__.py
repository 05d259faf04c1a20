"""fp64 CPU oracle of the GLM-5.3-Flash routed MoE MLP -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  The product path (routed_expert_mlp_amd) never does,
and this package imports nothing from it.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (RoutedWeights, bf16_linear, bf16_mlp, decode_bf16, decode_e2m1,  # noqa: F401
                         decode_e4m3, dense_ffn, dequant_fp8_block, dequant_nvfp4, expert_rows,
                         fp8_linear, moe_layer, nvfp4_linear, routed_expert_fp8,
                         round_bf16, route, routed_expert, router_logits, select_topk, sigmoid,
                         silu, swiglu_clamped, unpack_codes)
