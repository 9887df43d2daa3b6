"""moe_route_permute_noalloc (workspace in the library's static scratch)
against moe_route_permute (caller workspace): every output bit for bit, on
two calls in a row, the second with a smaller layer."""
import pytest
import torch

import combine_router_gating_amd as moe
import datagen
from gpu_helpers import log

DEV = "cuda:0"
KEYS = ("probs", "routing_map", "tokens_per_expert", "permuted_x", "permuted_probs",
        "sorted_token", "row_id_map", "expert_offsets", "logits")


def _call(cfg, inp, noalloc):
    return moe.moe_route_permute(
        inp["x"], inp["w_router"], K=cfg.K, b_router=inp.get("b_router"),
        expert_bias=inp.get("expert_bias"), score=cfg.score, pre_softmax=cfg.pre_softmax,
        capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity, want_logits=True,
        noalloc=noalloc)


def _check_equal(a, b, what):
    N = int(a["expert_offsets"][-1].item())
    assert N == int(b["expert_offsets"][-1].item()), what
    for k in KEYS:
        x, y = a[k], b[k]
        if k in ("permuted_x", "permuted_probs", "sorted_token"):
            x, y = x[:N], y[:N]  # rows past N are undefined
        assert torch.equal(x, y), f"{what}: {k}"


@pytest.mark.gpu
def test_noalloc_route_permute_matches_workspace_call_twice():
    # first call: the largest layer the scratch holds; second: a smaller one
    big = datagen.CONFIGS["dsv3"]
    small = datagen.MoEConfig("noalloc-small", T=777, h=256, E=64, K=2, f=128, dtype="bf16",
                              capacity_factor=1.25, gate_bias="zipf")
    for cfg in (big, small):
        log(f"noalloc route+permute: {cfg}")
        inp = datagen.make_inputs(cfg, seed=4, device=DEV, with_experts=False)
        got = _call(cfg, inp, noalloc=True)
        torch.cuda.synchronize()
        ref = _call(cfg, inp, noalloc=False)
        torch.cuda.synchronize()
        _check_equal(got, ref, cfg.name)
