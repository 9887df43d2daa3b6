"""Plain, slow CPU oracle of the MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py may import it.  The
product (combine_router_gating_amd) never imports, calls or loads it, and it
imports nothing from the product.

Everything is NumPy: floating point in float64 with one rounding at each
point where the layer stores a tensor, except where the pages fix fp32 (the
sigmoid scores used for expert selection, see fp32spec).
"""
from . import mx
from .fp32spec import exp_spec, log1p_spec, sigmoid_spec, softplus_spec, sqrtsoftplus_spec
from .moe import (
    round_bf16,
    round_to,
    router_logits,
    topk_indices,
    score_and_select,
    get_capacity,
    capacity_mask,
    apply_token_dropping,
    drop_by_position,
    route,
    aux_loss,
    accumulate_tokens,
    update_expert_bias,
    permute,
    swiglu_rows,
    grouped_experts,
    combine,
    moe_forward,
    token_outputs,
)

__all__ = [
    "mx",
    "exp_spec", "log1p_spec", "sigmoid_spec", "softplus_spec", "sqrtsoftplus_spec", "round_bf16", "round_to", "router_logits",
    "topk_indices", "score_and_select", "get_capacity", "capacity_mask",
    "apply_token_dropping", "drop_by_position", "aux_loss", "accumulate_tokens",
    "update_expert_bias",
    "route", "permute", "swiglu_rows", "grouped_experts", "combine",
    "moe_forward", "token_outputs",
]
