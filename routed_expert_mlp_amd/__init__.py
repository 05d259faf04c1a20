"""MI355X (gfx950) routed MoE MLP of GLM-5.3-Flash: HIP kernels behind a C ABI.

The compute lives in lib/libmoe_mlp.so (built from csrc/ by
`python -m routed_expert_mlp_amd.build`); capi.py is its ctypes binding.
"""
from .capi import (Config, KIND_DENSE, KIND_ROUTED, MoeMlpError, Weights, lib,  # noqa: F401
                   moe_mlp_decode, moe_mlp_prefill, moe_mlp_status_string, moe_mlp_workspace_size,
                   moe_nvfp4_dequant, moe_router_topk, workspace)
