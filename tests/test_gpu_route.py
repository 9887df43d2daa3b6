"""GPU parity of the router against the oracle.

Logits: within the fp32 tolerance of the oracle's float64 gating linear.
Routing: bit-exact routing_map and tokens_per_expert given the GPU's own
fp32 logits; probs within the fp32 tolerance.
"""
import numpy as np
import pytest
import torch

import combine_router_gating_amd as moe
import datagen
import oracle
from gpu_helpers import assert_close, f64, log, logits_floor, routing_ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _route_gpu(cfg, inp, **kw):
    return moe.moe_route(inp["x"], inp["w_router"], K=cfg.K, b_router=inp.get("b_router"),
                         expert_bias=inp.get("expert_bias"), score=cfg.score,
                         pre_softmax=cfg.pre_softmax, capacity_factor=cfg.capacity_factor,
                         min_capacity=cfg.min_capacity, want_logits=True, want_scores=True, **kw)


@pytest.mark.parametrize("name", ["tiny", "switch", "mixtral", "qwen3", "dsv3"])
def test_route_full_size(name):
    cfg = datagen.CONFIGS[name]
    log(f"route full size: {cfg}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV, with_experts=False)
    r = _route_gpu(cfg, inp)
    torch.cuda.synchronize()
    logits = r["logits"].cpu().numpy()
    ref_logits = oracle.router_logits(f64(inp["x"]), f64(inp["w_router"]),
                                      f64(inp["b_router"]) if "b_router" in inp else None)
    assert_close(logits, ref_logits, "f32", "logits", floor=logits_floor(cfg.h))
    eb = inp["expert_bias"].cpu().numpy() if "expert_bias" in inp else None
    ref = routing_ref(cfg, logits, eb)
    np.testing.assert_array_equal(r["routing_map"].cpu().numpy(), ref["routing_map"])
    np.testing.assert_array_equal(r["tokens_per_expert"].cpu().numpy(), ref["tokens_per_expert"])
    assert_close(r["probs"].cpu().numpy(), ref["probs"], "f32", "probs")
    if cfg.score == "sigmoid":
        np.testing.assert_array_equal(r["scores"].cpu().numpy(), ref["scores"])  # same fp32 bits
    else:
        assert_close(r["scores"].cpu().numpy(), ref["scores"], "f32", "scores")
    n = r["tokens_per_expert"].cpu().numpy()
    dropped = int(ref["map_pre"].sum() - ref["routing_map"].sum())
    assert int(n.sum()) == cfg.T * cfg.K - dropped
    if cfg.capacity_factor > 0:
        assert r["capacity"] == oracle.get_capacity(cfg.T * cfg.K, cfg.E, cfg.capacity_factor)
        assert n.max() <= r["capacity"]
        log(f"  capacity {r['capacity']}, dropped {dropped}")


@pytest.mark.parametrize("score,pre", [("softmax", True), ("softmax", False), ("sigmoid", True)])
@pytest.mark.parametrize("T,E,K", [(37, 8, 2), (100, 64, 1), (65, 128, 8), (33, 256, 8),
                                   (20, 1000, 6), (16, 3, 3), (1, 1, 1), (50, 20, 3),
                                   (40, 100, 4), (30, 250, 8), (21, 257, 3)])
def test_route_ties_from_given_logits(score, pre, T, E, K):
    """Integer-valued logits (many exact ties) and all-equal rows: the lowest
    expert index must win every tie, bit-exactly."""
    log(f"route ties: {score} pre={pre} T={T} E={E} K={K}")
    rng = np.random.default_rng(T * 1000 + E + K)
    logits = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
    logits[0] = 0.5
    if T > 3:
        logits[3] = logits[3, 0]  # all-equal row
    lg = torch.from_numpy(logits).to(DEV)
    eb = None
    if score == "sigmoid":
        eb_np = (rng.integers(-2, 3, size=E) * 0.25).astype(np.float32)
        eb = torch.from_numpy(eb_np).to(DEV)
    r = moe.moe_route(None, None, K=K, expert_bias=eb, score=score, pre_softmax=pre,
                      logits_in=lg)
    torch.cuda.synchronize()
    ref = oracle.route(logits=logits, K=K, score=score, pre_softmax=pre,
                       expert_bias=None if eb is None else eb.cpu().numpy())
    np.testing.assert_array_equal(r["routing_map"].cpu().numpy(), ref["routing_map"])
    np.testing.assert_array_equal(r["tokens_per_expert"].cpu().numpy(), ref["tokens_per_expert"])
    assert_close(r["probs"].cpu().numpy(), ref["probs"], "f32", "probs")
    if eb is None:
        assert r["routing_map"][0].cpu().numpy()[:K].all()  # all-equal row picks 0..K-1


def test_sigmoid_bits_match_the_oracle():
    """Every fp32 sigmoid score equals the oracle's bit for bit (the choice
    depends on these bits), including saturated ties near 1."""
    xs = np.concatenate([np.linspace(-90, 90, 400000), np.linspace(15, 18, 100000),
                         np.float32([0.0, -0.0, 1e-30, -1e-30, 86.0, -86.0, -86.01])]).astype(np.float32)
    E = 500
    xs = np.concatenate([xs, np.zeros((-len(xs)) % E, np.float32)]).reshape(-1, E)
    r = moe.moe_route(None, None, K=4, score="sigmoid", logits_in=torch.from_numpy(xs).to(DEV),
                      want_scores=True)
    torch.cuda.synchronize()
    got = r["scores"].cpu().numpy()
    ref = oracle.sigmoid_spec(xs)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    ref_r = oracle.route(logits=xs, K=4, score="sigmoid")
    np.testing.assert_array_equal(r["routing_map"].cpu().numpy(), ref_r["routing_map"])


@pytest.mark.parametrize("T,E,K,cf,minc", [(200, 8, 2, 0.5, 0), (1000, 16, 1, 1.0, 0),
                                           (97, 4, 2, 0.1, 3), (300, 64, 4, 0.25, 1),
                                           (64, 8, 8, 0.01, 0), (50, 5, 1, 0.05, 0),
                                           (20003, 4, 1, 0.9, 0), (70001, 8, 2, 0.8, 0)])
def test_capacity_drop_keeps_earliest(T, E, K, cf, minc):
    log(f"capacity: T={T} E={E} K={K} cf={cf} min={minc}")
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 2.0  # hot expert
    r = moe.moe_route(None, None, K=K, capacity_factor=cf, min_capacity=minc,
                      logits_in=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.route(logits=logits, K=K, capacity_factor=cf, min_capacity=minc)
    np.testing.assert_array_equal(r["routing_map"].cpu().numpy(), ref["routing_map"])
    np.testing.assert_array_equal(r["tokens_per_expert"].cpu().numpy(), ref["tokens_per_expert"])
    np.testing.assert_array_equal(r["probs"].cpu().numpy() == 0, ref["probs"] == 0)
    assert_close(r["probs"].cpu().numpy(), ref["probs"], "f32", "probs")


def test_route_empty_batch():
    w = torch.zeros((4, 16), dtype=torch.float32, device=DEV)
    x = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    r = moe.moe_route(x, w, K=2)
    torch.cuda.synchronize()
    assert r["tokens_per_expert"].cpu().tolist() == [0, 0, 0, 0]
    assert r["routing_map"].shape == (0, 4)


@pytest.mark.parametrize("T,h,E,K", [(1000, 96, 8, 2), (777, 160, 40, 1), (300, 256, 100, 4),
                                     (129, 2048, 64, 1), (2000, 512, 200, 8), (65, 4096, 300, 6),
                                     (33, 32, 3, 2)])
def test_gating_bf16_ragged_tiles(T, h, E, K):
    """The MFMA gating linear on shapes that leave ragged token, expert and
    k tiles (each expert-tile width, several h splits): logits within the
    fp32 tolerance of the float64 oracle, routing bit-exact given them."""
    log(f"gating ragged: T={T} h={h} E={E} K={K}")
    g = torch.Generator().manual_seed(T * 7 + E)
    x = torch.randn((T, h), generator=g).to(torch.bfloat16)
    w = torch.randn((E, h), generator=g) / h ** 0.5
    b = torch.randn((E,), generator=g) * 0.1
    r = moe.moe_route(x.to(DEV), w.to(DEV), K=K, b_router=b.to(DEV), want_logits=True)
    torch.cuda.synchronize()
    logits = r["logits"].cpu().numpy()
    ref_logits = oracle.router_logits(f64(x), f64(w), f64(b))
    assert_close(logits, ref_logits, "f32", "logits", floor=logits_floor(h))
    ref = oracle.route(logits=logits, K=K)
    np.testing.assert_array_equal(r["routing_map"].cpu().numpy(), ref["routing_map"])
    np.testing.assert_array_equal(r["tokens_per_expert"].cpu().numpy(), ref["tokens_per_expert"])


def test_route_logits_in_unaligned_matches_aligned():
    """Logits handed over at an address that is not 16-byte aligned take the
    scalar path of the top-k kernel and give the same bits."""
    T, E, K = 70, 64, 4
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    flat = torch.zeros(T * E + 1, dtype=torch.float32, device=DEV)
    flat[1:] = torch.from_numpy(logits.ravel()).to(DEV)
    unaligned = flat[1:].view(T, E)
    assert unaligned.data_ptr() % 16 != 0
    a = moe.moe_route(None, None, K=K, logits_in=torch.from_numpy(logits).to(DEV))
    b = moe.moe_route(None, None, K=K, logits_in=unaligned)
    torch.cuda.synchronize()
    for k in ("routing_map", "probs", "tokens_per_expert"):
        assert torch.equal(a[k], b[k]), k
