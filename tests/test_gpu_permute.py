"""GPU parity of the permute and the combine.

Index outputs (sorted_token, row_id_map, expert_offsets) are bit-exact
against the oracle; permuted rows are exact copies; the combine is within
the layer tolerance of the oracle and bitwise reproducible.
"""
import numpy as np
import pytest
import torch

import combine_router_gating_amd as moe
import datagen
import oracle
from gpu_helpers import assert_close, f64, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _routing(T, E, K, seed, cf=0.0, hot=0.0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += hot
    r = moe.moe_route(None, None, K=K, capacity_factor=cf,
                      logits_in=torch.from_numpy(logits).to(DEV))
    return logits, r


@pytest.mark.parametrize("T,h,E,K,cf,dt", [
    (1, 8, 1, 1, 0.0, torch.bfloat16),
    (17, 16, 4, 2, 0.0, torch.float32),
    (300, 256, 8, 2, 0.0, torch.bfloat16),
    (333, 136, 64, 4, 0.3, torch.bfloat16),
    (129, 2048, 16, 1, 0.5, torch.bfloat16),
    (64, 7168, 256, 8, 0.0, torch.bfloat16),
    (40, 64, 1000, 6, 0.0, torch.float32),
    (20, 32, 1024, 64, 0.0, torch.float32),
])
def test_permute_matches_oracle(T, h, E, K, cf, dt):
    log(f"permute: T={T} h={h} E={E} K={K} cf={cf} {dt}")
    logits, r = _routing(T, E, K, seed=T * 7 + E, cf=cf, hot=1.0)
    x = torch.randn((T, h), device=DEV).to(dt)
    pm = moe.moe_permute(x, r["routing_map"], r["probs"], K, r["max_rows"])
    torch.cuda.synchronize()
    rmap = r["routing_map"].cpu().numpy()
    ref = oracle.permute(f64(x), rmap, r["probs"].cpu().numpy(), K)
    N = int(ref["expert_offsets"][-1])
    np.testing.assert_array_equal(pm["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
    np.testing.assert_array_equal(pm["sorted_token"][:N].cpu().numpy(), ref["sorted_token"])
    np.testing.assert_array_equal(pm["row_id_map"].cpu().numpy(), ref["row_id_map"])
    np.testing.assert_array_equal(f64(pm["permuted_x"][:N]), ref["permuted_x"])  # exact copies
    np.testing.assert_array_equal(pm["permuted_probs"][:N].cpu().numpy(), ref["permuted_probs"])


@pytest.mark.parametrize("name", ["switch", "qwen3", "dsv3"])
def test_permute_full_size(name):
    cfg = datagen.CONFIGS[name]
    log(f"permute full size: {cfg}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV, with_experts=False)
    r = moe.moe_route(inp["x"], inp["w_router"], K=cfg.K, b_router=inp.get("b_router"),
                      expert_bias=inp.get("expert_bias"), score=cfg.score,
                      pre_softmax=cfg.pre_softmax, capacity_factor=cfg.capacity_factor)
    pm = moe.moe_permute(inp["x"], r["routing_map"], r["probs"], cfg.K, r["max_rows"])
    torch.cuda.synchronize()
    rmap = r["routing_map"].cpu().numpy()
    ref = oracle.permute(np.zeros((cfg.T, 1)), rmap, r["probs"].cpu().numpy(), cfg.K)
    N = int(ref["expert_offsets"][-1])
    np.testing.assert_array_equal(pm["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
    np.testing.assert_array_equal(pm["sorted_token"][:N].cpu().numpy(), ref["sorted_token"])
    np.testing.assert_array_equal(pm["row_id_map"].cpu().numpy(), ref["row_id_map"])
    np.testing.assert_array_equal(pm["permuted_probs"][:N].cpu().numpy(), ref["permuted_probs"])
    # rows are exact copies of x (checked with a library gather on the device)
    gathered = inp["x"].index_select(0, pm["sorted_token"][:N].long())
    assert torch.equal(pm["permuted_x"][:N], gathered)


@pytest.mark.parametrize("T,h,E,K,dt,shared", [
    (1, 8, 1, 1, torch.float32, False),
    (77, 24, 8, 2, torch.float32, True),
    (300, 256, 8, 2, torch.bfloat16, False),
    (129, 2056, 16, 3, torch.bfloat16, True),
    (64, 7168, 256, 8, torch.bfloat16, True),
    (50, 64, 128, 12, torch.bfloat16, False),  # K past one group of 8 loads
    (20, 32, 1024, 64, torch.float32, True),   # the largest K and E
])
def test_combine_matches_oracle(T, h, E, K, dt, shared):
    log(f"combine: T={T} h={h} E={E} K={K} {dt} shared={shared}")
    logits, r = _routing(T, E, K, seed=T + h, cf=0.6 if E > 1 else 0.0, hot=1.0)
    x = torch.randn((T, h), device=DEV).to(dt)
    pm = moe.moe_permute(x, r["routing_map"], r["probs"], K, r["max_rows"])
    rows = pm["permuted_x"].shape[0]
    y = torch.randn((rows, h), device=DEV).to(dt)
    sh = torch.randn((T, h), device=DEV).to(dt) if shared else None
    out = moe.moe_combine(y, pm["permuted_probs"], pm["row_id_map"], sh)
    out2 = moe.moe_combine(y, pm["permuted_probs"], pm["row_id_map"], sh)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # fixed order: bitwise reproducible
    dts = "bf16" if dt == torch.bfloat16 else "f32"
    ref = oracle.combine(f64(y), pm["permuted_probs"].cpu().numpy(), pm["row_id_map"].cpu().numpy(),
                         dts, None if sh is None else f64(sh))
    assert_close(f64(out), ref, dts, "combine")


def test_permute_then_combine_is_identity():
    """Top-1, unit probs, output rows = permuted rows: combine returns x."""
    T, h, E = 500, 64, 16
    _, r = _routing(T, E, 1, seed=5)
    x = torch.randn((T, h), device=DEV).to(torch.bfloat16)
    pm = moe.moe_permute(x, r["routing_map"], r["probs"], 1, r["max_rows"])
    ones = torch.ones_like(pm["permuted_probs"])
    back = moe.moe_combine(pm["permuted_x"], ones, pm["row_id_map"])
    torch.cuda.synchronize()
    assert torch.equal(back, x)


def test_permute_empty_batch():
    x = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    rmap = torch.zeros((0, 4), dtype=torch.uint8, device=DEV)
    probs = torch.zeros((0, 4), dtype=torch.float32, device=DEV)
    pm = moe.moe_permute(x, rmap, probs, 2, 0)
    out = moe.moe_combine(pm["permuted_x"], pm["permuted_probs"], pm["row_id_map"])
    torch.cuda.synchronize()
    assert pm["expert_offsets"].cpu().tolist() == [0] * 5
    assert out.shape == (0, 16)


ROUTE_PERMUTE_CASES = [
    # T, h, E, K, score, capacity_factor, drop_policy, pad, copy_rows
    (1000, 64, 16, 2, "softmax", 0.0, "position", False, True),
    (515, 128, 16, 1, "softmax", 1.25, "position", False, True),
    (2003, 256, 64, 1, "softmax", 1.0, "position", False, False),
    (300, 64, 8, 2, "softmax", 0.5, "probs", False, True),
    (300, 64, 8, 2, "softmax", 0.5, "position", True, False),
    (64, 32, 256, 8, "sigmoid", 0.0, "position", False, True),
    (77, 64, 5, 5, "softmax", 4.0, "position", False, True),  # capacity above T: nothing dropped
]


@pytest.mark.parametrize("T,h,E,K,score,cf,policy,pad,copy_rows", ROUTE_PERMUTE_CASES)
def test_route_permute_is_bitwise_route_then_permute(T, h, E, K, score, cf, policy, pad, copy_rows):
    log(f"route+permute: T={T} h={h} E={E} K={K} {score} cf={cf} {policy} pad={pad} copy={copy_rows}")
    g = torch.Generator().manual_seed(T + E * 7)
    x = torch.randn((T, h), generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn((E, h), generator=g) / h ** 0.5).to(DEV)
    w[0] += 0.3  # a popular expert, so that capacities drop entries
    eb = (torch.randn((E,), generator=g) * 0.1).to(DEV) if score == "sigmoid" else None
    kw = dict(K=K, score=score, expert_bias=eb, capacity_factor=cf, drop_policy=policy,
              pad_to_capacity=pad)
    a = moe.moe_route(x, w, **kw)
    pa = moe.moe_permute(x, a["routing_map"], a["probs"], K, a["max_rows"], copy_rows=copy_rows)
    b = moe.moe_route_permute(x, w, copy_rows=copy_rows, **kw)
    torch.cuda.synchronize()
    for k in ("probs", "routing_map", "tokens_per_expert"):
        assert torch.equal(a[k], b[k]), k
    N = int(a["tokens_per_expert"].sum())
    for k in ("row_id_map", "expert_offsets"):
        assert torch.equal(pa[k], b[k]), k
    for k in ("permuted_probs", "sorted_token") + (("permuted_x",) if copy_rows else ()):
        assert torch.equal(pa[k][:N], b[k][:N]), k


FC2_COMBINE_CASES = [
    # T, h, f, E, capacity_factor, hot: the 64-, 128- and 256-row launches
    (515, 128, 256, 16, 1.0, 2.0),     # drops, ~32 rows per expert
    (2000, 256, 128, 16, 1.25, 1.0),   # capacity 157 (256-row tiles of 128 columns)
    (1500, 128, 128, 16, 0.0, 0.0),    # dropless, ~94 rows per expert (128-row tiles)
    (3000, 128, 192, 8, 0.0, 0.0),     # dropless, ~375 rows per expert
    (1, 64, 64, 4, 0.0, 0.0),
    (40, 64, 128, 4, 0.05, 3.0),       # most tokens dropped
]


@pytest.mark.parametrize("T,h,f,E,cf,hot", FC2_COMBINE_CASES)
def test_fc2_combine_is_bitwise_fc2_then_combine(T, h, f, E, cf, hot):
    log(f"fc2+combine: T={T} h={h} f={f} E={E} cf={cf}")
    g = torch.Generator().manual_seed(T + h + E)
    x = torch.randn((T, h), generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn((E, h), generator=g) / h ** 0.5).to(DEV)
    w[0] += hot / h ** 0.5
    wg = (torch.randn((E, f, h), generator=g) * 0.05).to(torch.bfloat16).to(DEV)
    wu = (torch.randn((E, f, h), generator=g) * 0.05).to(torch.bfloat16).to(DEV)
    wd = (torch.randn((E, h, f), generator=g) * 0.05).to(torch.bfloat16).to(DEV)
    r = moe.moe_route_permute(x, w, K=1, capacity_factor=cf)
    tpe = r["tokens_per_expert"]
    act = moe.moe_grouped_fc1_swiglu(r["permuted_x"], tpe, wg, wu)
    y = moe.moe_grouped_fc2(act, tpe, wd)
    ref = moe.moe_combine(y, r["permuted_probs"], r["row_id_map"])
    out = torch.full((T, h), float("nan"), dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_fc2_combine(act, tpe, wd, r["permuted_probs"], r["sorted_token"],
                                r["row_id_map"], out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_fused_calls_on_an_empty_batch():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((8, 64), dtype=torch.float32, device=DEV)
    r = moe.moe_route_permute(x, w, K=1, capacity_factor=1.0)
    torch.cuda.synchronize()
    assert r["tokens_per_expert"].cpu().tolist() == [0] * 8
    assert r["expert_offsets"].cpu().tolist() == [0] * 9
    act = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((8, 64, 128), dtype=torch.bfloat16, device=DEV)
    out = moe.moe_grouped_fc2_combine(act, r["tokens_per_expert"], wd, r["permuted_probs"],
                                      r["sorted_token"], r["row_id_map"])
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
