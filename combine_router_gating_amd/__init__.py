"""MI355X-native single-GPU MoE layer forward: route -> permute -> grouped
SwiGLU experts -> weighted combine, as HIP kernels behind a C interface
(include/moe.h, built into libmoe.so)."""
from .moe import (
    moe_accumulate_tokens_per_expert,
    moe_clock_probe,
    moe_combine,
    gemm_queue,
    moe_forward,
    moe_grouped_fc1_swiglu,
    moe_grouped_fc1_swiglu_gather,
    moe_grouped_fc1_swiglu_gather_shared,
    moe_grouped_fc2,
    moe_grouped_fc2_combine,
    moe_grouped_fc2_shared,
    moe_grouped_mlp,
    moe_grouped_fc1_swiglu_mxfp8,
    moe_grouped_fc1_swiglu_mxfp8_shared,
    moe_grouped_fc2_mxfp8,
    moe_grouped_fc2_mxfp8_shared,
    moe_grouped_fc2_combine_mxfp8,
    moe_max_rows,
    moe_mxfp8_quantize,
    moe_mxfp8_quantize_weight,
    moe_permute,
    moe_route,
    moe_route_capacity,
    moe_route_permute,
    moe_router_aux_loss,
    moe_update_expert_bias,
    route_desc,
)
from ._lib import LIB_PATH, MoEError, load

__all__ = [
    "moe_accumulate_tokens_per_expert", "moe_router_aux_loss", "moe_update_expert_bias",
    "gemm_queue", "moe_clock_probe", "moe_combine", "moe_forward", "moe_grouped_fc1_swiglu", "moe_grouped_fc1_swiglu_gather",
    "moe_grouped_fc1_swiglu_gather_shared", "moe_grouped_fc2_shared",
    "moe_grouped_fc2", "moe_grouped_fc2_combine", "moe_grouped_fc1_swiglu_mxfp8", "moe_grouped_fc1_swiglu_mxfp8_shared", "moe_grouped_fc2_mxfp8", "moe_grouped_fc2_mxfp8_shared", "moe_grouped_fc2_combine_mxfp8", "moe_mxfp8_quantize",
    "moe_mxfp8_quantize_weight", "moe_grouped_mlp",
    "moe_max_rows", "moe_permute", "moe_route", "moe_route_capacity", "moe_route_permute", "route_desc", "LIB_PATH",
    "MoEError", "load",
]
