"""GPU parity of the routing variants: sqrtsoftplus scores, the probs drop
policy, padding to capacity (route, permute and the whole layer), the
load-balancing loss value and the expert-bias controller.

Where a float decides an integer (which tokens an expert keeps under the
probs policy), the oracle takes that decision on the GPU's own fp32 pre-drop
probs: the capacity step is compared given identical inputs, bit-exactly.
"""
import numpy as np
import pytest
import torch

import combine_router_gating_amd as moe
import datagen
import oracle
from gpu_helpers import assert_close, f64, log, shared_weights_from

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _route_logits(logits, K, **kw):
    return moe.moe_route(None, None, K=K, logits_in=torch.from_numpy(logits).to(DEV),
                         want_scores=True, **kw)


def _np(t):
    return t.cpu().numpy()


# ------------------------------------------------------------ sqrtsoftplus

def test_sqrtsoftplus_bits_match_the_oracle():
    xs = np.concatenate([np.linspace(-90, 90, 400000), np.linspace(19, 21, 100000),
                         np.float32([0.0, -0.0, 20.0, 1e-30, -1e-30, 86.0, -86.0, -86.01])])
    xs = xs.astype(np.float32)
    E = 500
    xs = np.concatenate([xs, np.zeros((-len(xs)) % E, np.float32)]).reshape(-1, E)
    r = _route_logits(xs, 4, score="sqrtsoftplus")
    torch.cuda.synchronize()
    got = _np(r["scores"])
    ref = oracle.sqrtsoftplus_spec(xs)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    ref_r = oracle.route(logits=xs, K=4, score="sqrtsoftplus")
    np.testing.assert_array_equal(_np(r["routing_map"]), ref_r["routing_map"])


@pytest.mark.parametrize("T,E,K", [(37, 8, 2), (65, 128, 8), (20, 1000, 6), (16, 3, 3)])
def test_sqrtsoftplus_routing_with_ties_and_bias(T, E, K):
    log(f"sqrtsoftplus ties: T={T} E={E} K={K}")
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    logits[0] = 0.5
    eb = (rng.integers(-2, 3, size=E) * 0.25).astype(np.float32)
    r = _route_logits(logits, K, score="sqrtsoftplus", expert_bias=torch.from_numpy(eb).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.route(logits=logits, K=K, score="sqrtsoftplus", expert_bias=eb)
    np.testing.assert_array_equal(_np(r["routing_map"]), ref["routing_map"])
    np.testing.assert_array_equal(_np(r["tokens_per_expert"]), ref["tokens_per_expert"])
    assert_close(_np(r["probs"]), ref["probs"], "f32", "probs")


# ------------------------------------------------------- capacity variants

CAP_CASES = [(200, 8, 2, 0.5, 0), (1000, 16, 1, 1.0, 0), (97, 4, 2, 0.1, 3), (300, 64, 4, 0.25, 1),
             (64, 8, 8, 0.01, 0), (50, 5, 1, 0.05, 0), (40, 4, 2, 3.0, 0), (33, 6, 2, 0.0001, 40),
             (517, 256, 8, 0.5, 0)]


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("policy,pad", [("probs", False), ("probs", True), ("position", True)])
@pytest.mark.parametrize("T,E,K,cf,minc", CAP_CASES)
def test_capacity_variants_given_prob_bits(score, policy, pad, T, E, K, cf, minc):
    log(f"capacity {policy} pad={pad} {score}: T={T} E={E} K={K} cf={cf} min={minc}")
    rng = np.random.default_rng(T + E + K)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 2.0                                   # hot expert
    logits[rng.integers(0, T, T // 3)] = logits[0]        # duplicate rows: equal probs
    kw = dict(score=score)
    r0 = _route_logits(logits, K, **kw)                   # pre-drop, same kernels and bits
    r = _route_logits(logits, K, capacity_factor=cf, min_capacity=minc, drop_policy=policy,
                      pad_to_capacity=pad, **kw)
    torch.cuda.synchronize()
    cap = oracle.get_capacity(T * K, E, cf, minc)
    fp, fm = oracle.apply_token_dropping(_np(r0["probs"]), _np(r0["routing_map"]), cap, policy, pad)
    np.testing.assert_array_equal(_np(r["routing_map"]), fm)
    np.testing.assert_array_equal(_np(r["probs"]), fp)
    np.testing.assert_array_equal(_np(r["tokens_per_expert"]), fm.sum(axis=0))
    if pad:
        assert r["max_rows"] == E * min(cap, T)


@pytest.mark.parametrize("policy,pad", [("probs", False), ("probs", True), ("position", True)])
def test_capacity_variants_full_size_switch(policy, pad):
    cfg = datagen.CONFIGS["switch"]
    log(f"switch full size {policy} pad={pad}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV, with_experts=False)
    kw = dict(K=cfg.K, b_router=inp["b_router"], score=cfg.score, want_logits=True)
    r0 = moe.moe_route(inp["x"], inp["w_router"], **kw)
    r = moe.moe_route(inp["x"], inp["w_router"], capacity_factor=cfg.capacity_factor,
                      drop_policy=policy, pad_to_capacity=pad, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(r["logits"]), _np(r0["logits"]))
    cap = oracle.get_capacity(cfg.T * cfg.K, cfg.E, cfg.capacity_factor)
    assert cap == 160
    fp, fm = oracle.apply_token_dropping(_np(r0["probs"]), _np(r0["routing_map"]), cap, policy, pad)
    np.testing.assert_array_equal(_np(r["routing_map"]), fm)
    np.testing.assert_array_equal(_np(r["probs"]), fp)
    np.testing.assert_array_equal(_np(r["tokens_per_expert"]), fm.sum(axis=0))


@pytest.mark.parametrize("T,E,K,cap_f", [(70, 8, 2, 0.5), (40, 4, 1, 4.0), (37, 96, 3, 1.0), (37, 96, 3, 40.0)])
def test_permute_padded_map(T, E, K, cap_f):
    """Padded maps give tokens more than K entries (all E when the capacity
    reaches T, E > 64 exercises the per-entry copy path); rows, probs and
    combine slots match the oracle bit for bit."""
    log(f"permute padded: T={T} E={E} K={K} cf={cap_f}")
    rng = np.random.default_rng(T * E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = _route_logits(logits, K, capacity_factor=cap_f, drop_policy="probs", pad_to_capacity=True)
    x = torch.from_numpy(rng.standard_normal((T, 64)).astype(np.float32)).to(DEV)
    pm = moe.moe_permute(x, r["routing_map"], r["probs"], K, r["max_rows"])
    torch.cuda.synchronize()
    ref = oracle.permute(_np(x), _np(r["routing_map"]), _np(r["probs"]), K)
    N = int(ref["expert_offsets"][-1])
    assert N == r["max_rows"]
    np.testing.assert_array_equal(_np(pm["expert_offsets"]), ref["expert_offsets"])
    np.testing.assert_array_equal(_np(pm["sorted_token"])[:N], ref["sorted_token"])
    np.testing.assert_array_equal(_np(pm["row_id_map"]), ref["row_id_map"])
    np.testing.assert_array_equal(_np(pm["permuted_probs"])[:N], ref["permuted_probs"])
    np.testing.assert_array_equal(_np(pm["permuted_x"])[:N], ref["permuted_x"])


LAYERS = [
    datagen.MoEConfig("cap-probs", T=515, h=128, E=16, K=1, f=256, dtype="bf16",
                      capacity_factor=1.25, gate_bias="zipf"),
    datagen.MoEConfig("cap-probs-sig", T=257, h=256, E=64, K=4, f=128, dtype="bf16",
                      score="sigmoid", expert_bias=True, shared_f=128, capacity_factor=0.6),
    datagen.MoEConfig("cap-f32", T=99, h=64, E=4, K=2, f=96, dtype="f32", capacity_factor=0.5),
]


@pytest.mark.parametrize("pad", [False, True])
@pytest.mark.parametrize("cfg", LAYERS, ids=lambda c: c.name)
def test_layer_probs_policy(cfg, pad):
    log(f"layer probs policy pad={pad}: {cfg}")
    inp = datagen.make_inputs(cfg, seed=2, device=DEV)
    kw = dict(K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax)
    r0 = moe.moe_route(inp["x"], inp["w_router"], b_router=inp.get("b_router"),
                       expert_bias=inp.get("expert_bias"), **kw)
    res = moe.moe_forward(inp, capacity_factor=cfg.capacity_factor, drop_policy="probs",
                          pad_to_capacity=pad, **kw)
    plain = moe.moe_forward(inp, capacity_factor=cfg.capacity_factor, drop_policy="probs",
                            pad_to_capacity=False, **kw)
    torch.cuda.synchronize()
    cap = oracle.get_capacity(cfg.T * cfg.K, cfg.E, cfg.capacity_factor)
    fp, fm = oracle.apply_token_dropping(_np(r0["probs"]), _np(r0["routing_map"]), cap, "probs", pad)
    np.testing.assert_array_equal(_np(res["routing_map"]), fm)
    pm = oracle.permute(f64(inp["x"]), fm, fp, cfg.K)
    w = (f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"]))
    act, y = oracle.grouped_experts(pm["permuted_x"], pm["tokens_per_expert"], w, cfg.dtype)
    sh = shared_weights_from(inp)
    shared_out = oracle.swiglu_rows(f64(inp["x"]), *sh, cfg.dtype)[1] if sh else None
    out = oracle.combine(y, pm["permuted_probs"], pm["row_id_map"], cfg.dtype, shared_out)
    np.testing.assert_array_equal(_np(res["row_id_map"]), pm["row_id_map"])
    N = int(pm["expert_offsets"][-1])
    np.testing.assert_array_equal(_np(res["sorted_token"])[:N], pm["sorted_token"])
    assert_close(f64(res["expert_out"][:N]), y, cfg.dtype, "expert_out")
    assert_close(f64(res["out"]), out, cfg.dtype, "out")
    # padding rows carry prob 0: the output equals the unpadded layer's bit for bit
    np.testing.assert_array_equal(_np(res["out"].float()), _np(plain["out"].float()))


# ------------------------------------------------------ router side outputs

@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrtsoftplus"])
@pytest.mark.parametrize("T,E,K", [(1, 4, 2), (63, 8, 2), (1000, 64, 1), (8192, 256, 8), (129, 1000, 6)])
def test_aux_loss_matches_the_oracle(score, T, E, K):
    log(f"aux loss {score}: T={T} E={E} K={K}")
    rng = np.random.default_rng(T + E)
    logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    r = _route_logits(logits, K, score=score)
    loss = moe.moe_router_aux_loss(r["scores"], r["tokens_per_expert"], K=K, score=score)
    torch.cuda.synchronize()
    ref = oracle.aux_loss(_np(r["scores"]), _np(r["tokens_per_expert"]), K, score)
    got = float(loss.item())
    assert abs(got - ref) <= 1e-5 * abs(ref) + 1e-7, (got, ref)


def test_aux_loss_uniform_scores_is_one():
    T, E, K = 640, 16, 2
    r = _route_logits(np.zeros((T, E), np.float32), K)
    loss = moe.moe_router_aux_loss(r["scores"], r["tokens_per_expert"], K=K)
    assert abs(float(loss.item()) - 1.0) < 1e-5


def test_expert_bias_controller_matches_the_oracle():
    rng = np.random.default_rng(21)
    E = 300
    local = torch.zeros((E,), dtype=torch.int64, device=DEV)
    ref_local = np.zeros(E, np.int64)
    bias0 = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    bias = torch.from_numpy(bias0.copy()).to(DEV)
    for step in range(3):
        n = rng.integers(0, 500, E).astype(np.int32)
        n[:5] = 250  # some counts at the mean of others
        moe.moe_accumulate_tokens_per_expert(torch.from_numpy(n).to(DEV), local)
        ref_local = oracle.accumulate_tokens(ref_local, n)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(local), ref_local)
    moe.moe_update_expert_bias(local, bias, 1e-3, reset=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(bias), oracle.update_expert_bias(ref_local, bias0, 1e-3))
    assert not _np(local).any()
    # exact sign decision near 2^24 counts
    c = torch.tensor([16777217, 16777217, 16777218], dtype=torch.int64, device=DEV)
    b = torch.zeros((3,), dtype=torch.float32, device=DEV)
    moe.moe_update_expert_bias(c, b, 1.0, reset=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(b), np.float32([1, 1, -1]))
    assert _np(c).tolist() == [16777217, 16777217, 16777218]
