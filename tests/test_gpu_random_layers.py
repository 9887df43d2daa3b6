"""Seeded sweep over layer shapes, routing options and launch options.

Each case draws a small layer (experts, top-k, sizes, score function, gate
bias, selection-only expert bias, capacity with either drop policy and
optional padding, shared expert) and two sets of launch options (gathering
FC1, fused route + permute, fused combine, folded or overlapped shared
expert, tile queue).  The first forward is compared with the oracle:
logits at the fp32 tolerance, routing map bit-exact given the GPU's logits,
output at the layer tolerance.  The second option set must give the same
output bits (the options change where data is read and when kernels run,
not the arithmetic).  MXFP8 cases (their oracle chain is in
test_gpu_mxfp8.py) are checked for routing, equal bits across the two
option sets, bit-exact x quantisation, and the FC2 + combine chain the
oracle computes from the GPU's act codes.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from combine_router_gating_amd.layer import MoELayerForward
from gpu_helpers import (assert_close, f64, log, logits_floor, mx_dequantize_tiled,
                         shared_weights_from, untile)
from oracle import mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 64


def _draw(i):
    rng = np.random.default_rng(7000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    precision = "bf16"
    u = rng.random()
    if u < 0.2:
        dtype = "f32"
    else:
        dtype = "bf16"
        if u > 0.8:
            precision = "mxfp8"
    if precision == "mxfp8":
        h, f, fs_choices = pick([128, 256, 384]), pick([128, 256, 512]), [128, 256]
    elif dtype == "bf16":
        h, f, fs_choices = pick([64, 128, 192, 320]), pick([64, 128, 256, 448]), [64, 192]
    else:
        h, f, fs_choices = pick([8, 40, 64, 96]), pick([16, 24, 64, 80]), [16, 48]
    E = pick([1, 2, 3, 8, 16, 33, 64])
    K = int(rng.integers(1, min(E, 8) + 1))
    # some layers large enough for the tile queue (>= 192 rows per expert)
    T = int(rng.integers(1, 400)) if rng.random() < 0.6 else int(192 * E // K + rng.integers(0, 200))
    T = min(T, 2500)
    score = pick(["softmax", "sigmoid"])
    pre_softmax = bool(rng.random() < 0.5) if score == "softmax" else True
    capacity_factor, min_capacity, policy, pad = 0.0, 0, "position", False
    if rng.random() < 0.4:
        capacity_factor = pick([0.3, 0.8, 1.25, 3.0])
        min_capacity = pick([0, 0, 4])
        policy = pick(["position", "probs"])
        pad = bool(rng.random() < 0.3)
    cfg = datagen.MoEConfig(
        f"rand{i}", T=T, h=h, E=E, K=K, f=f, dtype=dtype, score=score, pre_softmax=pre_softmax,
        capacity_factor=capacity_factor, min_capacity=min_capacity,
        gate_bias="zipf" if rng.random() < 0.3 else None,
        expert_bias=bool(score == "sigmoid" and rng.random() < 0.6),
        shared_f=pick(fs_choices) if rng.random() < 0.35 else 0)

    def options():
        return dict(gather=bool(rng.random() < 0.6), overlap_shared=bool(rng.random() < 0.4),
                    fuse_route_permute=bool(rng.random() < 0.7),
                    fuse_combine=bool(rng.random() < 0.7), fold_shared=bool(rng.random() < 0.6),
                    tile_queue=bool(rng.random() < 0.7))

    return cfg, policy, pad, precision, options(), options()


def _check_mxfp8_chain(layer, inp, cfg, r, out):
    """MXFP8 layer: x quantised bit-exactly; FC2, the shared expert's FC2 and
    the combine recomputed by the oracle from the GPU's act codes (exact
    inputs) and quantised weights match the output at the bf16 tolerance."""
    xc, xs = mx.mx_quantize(f64(inp["x"]))
    np.testing.assert_array_equal(layer.xq[0].cpu().numpy(), xc)
    np.testing.assert_array_equal(layer.xq[1].cpu().numpy(), xs)
    pm = oracle.permute(f64(inp["x"]), r["routing_map"], r["probs"], cfg.K)
    np.testing.assert_array_equal(layer.tokens_per_expert.cpu().numpy(), pm["tokens_per_expert"])
    N = int(pm["expert_offsets"][-1])
    act = mx.mx_dequantize(layer.actq[0].cpu().numpy()[:N], untile(layer.actq[1])[:N])
    wd = mx_dequantize_tiled(*layer.wq["w_down"])
    off = pm["expert_offsets"]
    y = np.zeros((N, cfg.h))
    for e in range(cfg.E):
        y[off[e]:off[e + 1]] = act[off[e]:off[e + 1]] @ wd[e].T
    y = oracle.round_bf16(y)
    shared = None
    if cfg.shared_f:
        sact = mx_dequantize_tiled(*layer.shared_actq)
        swd = mx_dequantize_tiled(*layer.wq["shared_down"])[0]
        shared = oracle.round_bf16(sact @ swd.T)
    ref = oracle.combine(y, pm["permuted_probs"], pm["row_id_map"], "bf16", shared)
    assert_close(f64(out), ref, "bf16", "out (MXFP8 chain)")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer_against_the_oracle(i):
    cfg, policy, pad, precision, opt_a, opt_b = _draw(i)
    log(f"random layer {i}: {cfg} policy={policy} pad={pad} {precision} A={opt_a} B={opt_b}")
    inp = datagen.make_inputs(cfg, seed=100 + i, device=DEV)
    kw = dict(K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
              capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity,
              drop_policy=policy, pad_to_capacity=pad, precision=precision)
    a = MoELayerForward(inp, **kw, **opt_a)
    out_a = a.forward().clone()
    torch.cuda.synchronize()
    b = MoELayerForward(inp, **kw, **opt_b)
    out_b = b.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), "option sets A and B differ"
    assert torch.equal(a.routing_map, b.routing_map)

    logits = a.logits.cpu().numpy()
    ref_logits = oracle.router_logits(f64(inp["x"]), f64(inp["w_router"]),
                                      f64(inp["b_router"]) if "b_router" in inp else None)
    assert_close(logits, ref_logits, "f32", "logits", floor=logits_floor(cfg.h))
    eb = inp["expert_bias"].cpu().numpy() if "expert_bias" in inp else None
    if precision == "mxfp8":
        r = oracle.route(logits=logits, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                         expert_bias=eb, capacity_factor=cfg.capacity_factor,
                         min_capacity=cfg.min_capacity, drop_policy=policy, pad_to_capacity=pad)
        np.testing.assert_array_equal(a.routing_map.cpu().numpy(), r["routing_map"])
        _check_mxfp8_chain(a, inp, cfg, r, out_a)
        return
    ref = oracle.moe_forward(f64(inp["x"]), None, None,
                             (f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"])),
                             K=cfg.K, dtype=cfg.dtype, score=cfg.score, pre_softmax=cfg.pre_softmax,
                             expert_bias=eb, capacity_factor=cfg.capacity_factor,
                             min_capacity=cfg.min_capacity, drop_policy=policy,
                             pad_to_capacity=pad, shared=shared_weights_from(inp), logits=logits)
    np.testing.assert_array_equal(a.routing_map.cpu().numpy(), ref["routing_map"])
    np.testing.assert_array_equal(a.tokens_per_expert.cpu().numpy(), ref["tokens_per_expert"])
    assert_close(f64(out_a), ref["out"], cfg.dtype, "out")
