"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something other than its own code:
hand-derived worked examples (tests/golden), closed forms, brute force on
tiny inputs, invariants of the method, or a library routine for a special
case.  No GPU is used.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(v):
    return float(eval(v, {"math": math})) if isinstance(v, str) else float(v)


# ----------------------------------------------------------------- rounding

def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.float32([0.0, -0.0, 1.0, -1.0]),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_ties_to_even_by_hand():
    # bf16 spacing just above 1 is 2^-7
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0                 # tie -> even (1.0)
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie -> even
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    # a value exactly between two fp32 neighbours that double rounding would break
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.round_bf16(v) == 1.0 + 2.0 ** -7


# ------------------------------------------------------------ fp32 sigmoid

def _ulp_f32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


def test_exp_spec_accuracy():
    y = -np.linspace(0, 86, 400001).astype(np.float32)
    got = oracle.exp_spec(y).astype(np.float64)
    ref = np.exp(y.astype(np.float64))
    err = np.abs(got - ref) / _ulp_f32(ref.astype(np.float32))
    assert err.max() <= 2.0, err.max()
    assert oracle.exp_spec(np.float32([0.0]))[0] == 1.0
    assert oracle.exp_spec(np.float32([-100.0]))[0] == 0.0


def test_sigmoid_spec_accuracy_and_symmetry():
    x = np.linspace(-30, 30, 600001).astype(np.float32)
    got = oracle.sigmoid_spec(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    err = np.abs(got - ref) / _ulp_f32(ref.astype(np.float32))
    assert err.max() <= 3.0, err.max()
    assert oracle.sigmoid_spec(np.float32([0.0]))[0] == np.float32(0.5)
    s = oracle.sigmoid_spec(x).astype(np.float64) + oracle.sigmoid_spec(-x).astype(np.float64)
    assert np.abs(s - 1.0).max() < 2e-7


def test_sigmoid_spec_is_monotone_on_a_sweep():
    x = np.linspace(-20, 20, 200001).astype(np.float32)
    s = oracle.sigmoid_spec(x)
    assert np.all(np.diff(s.astype(np.float64)) >= 0)


# ----------------------------------------------------------------- top-k

def _brute_topk(row, K):
    """The K-subset whose members all beat every non-member under
    (value descending, index ascending), found by trying every subset."""
    E = len(row)

    def beats(a, b):
        return row[a] > row[b] or (row[a] == row[b] and a < b)

    winners = [S for S in itertools.combinations(range(E), K)
               if all(beats(a, b) for a in S for b in range(E) if b not in S)]
    assert len(winners) == 1
    return set(winners[0])


@pytest.mark.parametrize("E,K", [(1, 1), (4, 2), (6, 3), (8, 1), (10, 3), (5, 5)])
def test_topk_brute_force_with_ties(E, K):
    rng = np.random.default_rng(E * 10 + K)
    for _ in range(200):
        row = rng.integers(-2, 3, size=E).astype(np.float32)  # many ties
        got = oracle.topk_indices(row[None, :], K)[0]
        assert set(got.tolist()) == _brute_topk(row, K)
        # selection order: value descending, index ascending among ties
        keys = [(-row[i], i) for i in got]
        assert keys == sorted(keys)


def test_topk_all_equal_rows_choose_lowest_indices():
    v = np.full((3, 9), 0.25, np.float32)
    assert oracle.topk_indices(v, 4).tolist() == [[0, 1, 2, 3]] * 3


def test_topk_signed_zero_is_a_tie():
    v = np.float32([[-0.0, 0.0, -1.0]])
    assert oracle.topk_indices(v, 1).tolist() == [[0]]


# ------------------------------------------------------ gating linear

def test_router_logits_golden_with_and_without_bias():
    """The gating linear against hand-derived logits: a dropped bias, a bias
    added after rounding, or fp32 accumulation each change a value."""
    g = json.load(open(os.path.join(GOLDEN, "router_logits_worked.json")))
    x, w, b = (np.array(g[k], np.float64) for k in ("x", "w", "b"))
    got = oracle.router_logits(x, w, b)
    assert got.dtype == np.float32
    assert got.tolist() == g["logits"], g["cite"]
    assert oracle.router_logits(x, w).tolist() == g["logits_no_bias"], g["cite"]
    # bf16-representable inputs given as bf16-rounded float32 give the same
    assert oracle.router_logits(x.astype(np.float32), w.astype(np.float32),
                                b.astype(np.float32)).tolist() == g["logits"]


def test_router_logits_transposes_the_weight():
    """logits[t, e] pairs token t with weight row e (a square case, where a
    transposed operand would still have the right shape)."""
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert oracle.router_logits(x, w).tolist() == [[1.0, 3.0], [2.0, 4.0]]
    assert oracle.router_logits(x, w, np.array([10.0, 20.0])).tolist() == [[11.0, 23.0],
                                                                             [12.0, 24.0]]


# ------------------------------------------------------ routing worked cases

def test_routing_golden_cases():
    data = json.load(open(os.path.join(GOLDEN, "routing_worked.json")))
    for c in data["cases"]:
        logits = np.array([[_ev(v) for v in r] for r in c["logits"]], np.float32)
        bias = np.array(c["expert_bias"], np.float32) if "expert_bias" in c else None
        probs, rmap, _ = oracle.score_and_select(logits, c["K"], c["score"], c["pre_softmax"], bias)
        assert rmap.tolist() == c["map"], c["cite"]
        exp = np.array([[_ev(v) for v in r] for r in c["probs"]])
        np.testing.assert_allclose(probs, exp, rtol=2e-6, atol=1e-7, err_msg=c["cite"])


def test_softmax_branches_relate():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((64, 16)).astype(np.float32)
    for K in (1, 2, 5):
        p_pre, m_pre, full = oracle.score_and_select(logits, K, "softmax", True)
        p_ren, m_ren, _ = oracle.score_and_select(logits, K, "softmax", False)
        assert np.array_equal(m_pre, m_ren)
        np.testing.assert_allclose(p_ren.sum(1), 1.0, rtol=1e-6)
        assert np.all(p_pre.sum(1) <= 1.0 + 1e-6)
        # renormalised probs are the pre-softmax probs divided by their sum
        np.testing.assert_allclose(p_ren, p_pre / p_pre.sum(1, keepdims=True), rtol=1e-6, atol=1e-9)
        # pre-softmax probs are the full softmax on the chosen experts
        np.testing.assert_allclose(p_pre, np.where(m_pre == 1, full, 0.0), rtol=1e-6, atol=0)
    p_all, m_all, full = oracle.score_and_select(logits, 16, "softmax", True)
    assert m_all.min() == 1
    np.testing.assert_allclose(p_all.sum(1), 1.0, rtol=1e-6)
    e = np.exp(logits.astype(np.float64))
    np.testing.assert_allclose(p_all, e / e.sum(1, keepdims=True), rtol=1e-6)


def test_sigmoid_routing_properties():
    rng = np.random.default_rng(4)
    # distinct logits in a range where fp32 sigmoid is strictly increasing
    logits = (rng.permuted(np.tile(np.arange(32), (50, 1)), axis=1) * 0.1 - 1.6).astype(np.float32)
    p0, m0, s = oracle.score_and_select(logits, 4, "sigmoid")
    # sigmoid is increasing: with no bias the choice equals top-k on logits
    _, m_l, _ = oracle.score_and_select(logits, 4, "softmax", True)
    assert np.array_equal(m0, m_l)
    np.testing.assert_allclose(p0.sum(1), 1.0, rtol=1e-6)
    # probs depend on the bias only through the choice
    bias = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    pb, mb, _ = oracle.score_and_select(logits, 4, "sigmoid", expert_bias=bias)
    s64 = s.astype(np.float64) * mb
    np.testing.assert_allclose(pb, s64 / s64.sum(1, keepdims=True), rtol=1e-6)
    # a bias that makes one expert win everywhere
    big = np.zeros(32, np.float32)
    big[7] = 10.0
    _, mbig, _ = oracle.score_and_select(logits, 4, "sigmoid", expert_bias=big)
    assert mbig[:, 7].all()


# --------------------------------------------------------------- capacity

def test_capacity_switch_layer_by_hand():
    # 8192 tokens, top-1, 64 experts, factor 1.25: 8192*1.25/64 = 160 exactly
    assert oracle.get_capacity(8192 * 1, 64, 1.25) == 160
    assert oracle.get_capacity(10, 3, 1.0) == 4          # ceil(3.33)
    assert oracle.get_capacity(10, 3, 1.0, min_capacity=6) == 6


def test_capacity_golden():
    c = json.load(open(os.path.join(GOLDEN, "capacity_worked.json")))
    T, E = c["T"], c["E"]
    assert oracle.get_capacity(T * c["K"], E, c["capacity_factor"]) == c["capacity"]
    logits = np.full((T, E), -1.0, np.float32)
    logits[np.arange(T), c["route_to"]] = 1.0
    r = oracle.route(logits=logits, K=1, capacity_factor=c["capacity_factor"])
    assert r["routing_map"].sum(1).tolist() == c["kept"]
    assert r["tokens_per_expert"].tolist() == c["tokens_per_expert"]
    x = np.arange(T, dtype=np.float64)[:, None] * np.ones((1, 3))
    pm = oracle.permute(x, r["routing_map"], r["probs"], 1)
    assert pm["sorted_token"].tolist() == c["sorted_token"]
    assert pm["expert_offsets"].tolist() == c["expert_offsets"]
    assert pm["row_id_map"].tolist() == c["row_id_map"]
    # dropped entries have prob 0 and no renormalisation happens elsewhere
    assert np.all(r["probs"][r["routing_map"] == 0] == 0)
    kept = r["routing_map"] == 1
    np.testing.assert_array_equal(r["probs"][kept], r["probs_pre"][kept])


def _brute_drop(rmap, cap):
    keep = np.zeros_like(rmap)
    for e in range(rmap.shape[1]):
        n = 0
        for t in range(rmap.shape[0]):
            if rmap[t, e]:
                if n < cap:
                    keep[t, e] = 1
                n += 1
    return keep


@pytest.mark.parametrize("seed", range(6))
def test_capacity_drop_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, E, K = int(rng.integers(1, 60)), int(rng.integers(1, 9)), 1
    K = int(rng.integers(1, E + 1))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 1.5  # skew load so drops happen
    cf = float(rng.choice([0.25, 0.5, 1.0, 1.5]))
    r = oracle.route(logits=logits, K=K, capacity_factor=cf)
    cap = oracle.get_capacity(T * K, E, cf)
    expect = r["map_pre"] if cap >= T else _brute_drop(r["map_pre"], cap)
    np.testing.assert_array_equal(r["routing_map"], expect)
    n = r["tokens_per_expert"]
    assert np.all(n <= max(cap, 0) if cap < T else n <= T)
    dropped = int(r["map_pre"].sum() - r["routing_map"].sum())
    assert int(n.sum()) == T * K - dropped
    # a factor large enough to fit every token is the dropless result
    r_big = oracle.route(logits=logits, K=K, capacity_factor=float(E) * 2)
    r_none = oracle.route(logits=logits, K=K)
    np.testing.assert_array_equal(r_big["routing_map"], r_none["routing_map"])
    np.testing.assert_array_equal(r_big["probs"], r_none["probs"])


# ---------------------------------------------------------------- permute

@pytest.mark.parametrize("seed", range(5))
def test_permute_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    T, E = int(rng.integers(1, 80)), int(rng.integers(1, 12))
    K = int(rng.integers(1, E + 1))
    h = 5
    x = rng.standard_normal((T, h))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    cf = float(rng.choice([0.0, 0.5, 1.0]))
    r = oracle.route(logits=logits, K=K, capacity_factor=cf)
    pm = oracle.permute(x, r["routing_map"], r["probs"], K)
    N = int(r["tokens_per_expert"].sum())
    assert pm["permuted_x"].shape == (N, h)
    np.testing.assert_array_equal(pm["tokens_per_expert"], r["tokens_per_expert"])
    np.testing.assert_array_equal(np.diff(pm["expert_offsets"]), r["tokens_per_expert"])
    # rows are sorted by (expert, token), each pair once
    pairs = list(zip(pm["row_expert"].tolist(), pm["sorted_token"].tolist()))
    assert pairs == sorted(set(pairs))
    for e, t in pairs:
        assert r["routing_map"][t, e] == 1
    np.testing.assert_array_equal(pm["permuted_x"], x[pm["sorted_token"]])
    # unpermute: every used slot of row_id_map points back at a copy of x[t]
    rid = pm["row_id_map"]
    for t in range(T):
        used = rid[t][rid[t] >= 0]
        assert len(used) == r["routing_map"][t].sum()
        assert np.all(rid[t][len(used):] == -1)
        for row in used:
            np.testing.assert_array_equal(pm["permuted_x"][row], x[t])
        assert list(pm["row_expert"][used]) == sorted(pm["row_expert"][used])
    # permute then unpermute with unit weights and top-1 is the identity
    if K == 1 and cf == 0.0:
        ones = np.ones(N, np.float32)
        back = oracle.combine(pm["permuted_x"], ones, rid, "f32")
        np.testing.assert_array_equal(back, oracle.round_to(x, "f32"))


# ---------------------------------------------------------------- experts

def test_swiglu_golden():
    c = json.load(open(os.path.join(GOLDEN, "swiglu_worked.json")))
    x = np.array([[c["x"]]])
    wg, wu, wd = (np.array([[_ev(c[k])]]) for k in ("w_gate", "w_up", "w_down"))
    act, y = oracle.swiglu_rows(x, wg, wu, wd, "f32")
    assert math.isclose(act[0, 0], _ev(c["act"]), rel_tol=1e-7)
    assert math.isclose(y[0, 0], _ev(c["y"]), rel_tol=1e-7)
    out = oracle.combine(y, np.float32([c["prob"]]), np.array([[0]]), "f32",
                         shared_out=np.array([[c["shared"]]]))
    assert math.isclose(out[0, 0], _ev(c["out"]), rel_tol=1e-7)


def test_single_expert_is_dense_swiglu_library():
    rng = np.random.default_rng(7)
    T, h, f = 33, 24, 40
    x = rng.standard_normal((T, h))
    wg, wu, wd = (rng.standard_normal(s) * 0.2 for s in ((f, h), (f, h), (h, f)))
    act, y = oracle.grouped_experts(x, np.array([T]), (wg[None], wu[None], wd[None]), "f32")
    X = torch.from_numpy(x)
    ref_act = torch.nn.functional.silu(torch.nn.functional.linear(X, torch.from_numpy(wg))) \
        * torch.nn.functional.linear(X, torch.from_numpy(wu))
    ref_act = ref_act.to(torch.float32).to(torch.float64)
    np.testing.assert_allclose(act, ref_act.numpy(), rtol=1e-6, atol=1e-7)
    ref_y = torch.nn.functional.linear(torch.from_numpy(act), torch.from_numpy(wd)).to(torch.float32)
    np.testing.assert_array_equal(y, ref_y.to(torch.float64).numpy())


@pytest.mark.parametrize("score,pre", [("softmax", True), ("softmax", False), ("sigmoid", True)])
def test_shared_weights_reduce_to_dense_times_prob_sum(score, pre):
    """All experts sharing weights: out = SwiGLU(x) * sum_k p (+ shared)."""
    rng = np.random.default_rng(11)
    T, h, E, K, f = 40, 16, 6, 3, 24
    x = oracle.round_bf16(rng.standard_normal((T, h)))
    w_r = rng.standard_normal((E, h)).astype(np.float32) / 4
    wg, wu, wd = (oracle.round_bf16(rng.standard_normal(s) * 0.2) for s in ((f, h), (f, h), (h, f)))
    sh = tuple(oracle.round_bf16(rng.standard_normal(s) * 0.2) for s in ((f, h), (f, h), (h, f)))
    shared_w = (np.repeat(wg[None], E, 0), np.repeat(wu[None], E, 0), np.repeat(wd[None], E, 0))
    res = oracle.moe_forward(x, w_r, None, shared_w, K=K, dtype="bf16", score=score,
                             pre_softmax=pre, shared=sh, capacity_factor=0.8)
    _, y = oracle.swiglu_rows(x, wg, wu, wd, "bf16")
    _, ys = oracle.swiglu_rows(x, *sh, "bf16")
    psum = res["probs"].astype(np.float64).sum(1, keepdims=True)
    expect = oracle.round_bf16(y * psum + ys)
    np.testing.assert_array_equal(res["out"], expect)
    # a token whose every slot was dropped gets only the shared output
    empty = res["routing_map"].sum(1) == 0
    np.testing.assert_array_equal(res["out"][empty], oracle.round_bf16(ys[empty]))


def test_zero_down_projection_gives_zero_and_combine_is_linear():
    rng = np.random.default_rng(12)
    T, h, E, K, f = 20, 8, 4, 2, 12
    x = rng.standard_normal((T, h))
    w_r = rng.standard_normal((E, h)).astype(np.float32)
    wg, wu = rng.standard_normal((E, f, h)), rng.standard_normal((E, f, h))
    res = oracle.moe_forward(x, w_r, None, (wg, wu, np.zeros((E, h, f))), K=K, dtype="f32")
    assert np.all(res["out"] == 0)
    wd = rng.standard_normal((E, h, f))
    res = oracle.moe_forward(x, w_r, None, (wg, wu, wd), K=K, dtype="f32")
    y, p, rid = res["expert_out"], res["permuted_probs"], res["row_id_map"]
    a = oracle.combine(y, p, rid, "f32")
    b = oracle.combine(y, (2 * p).astype(np.float32), rid, "f32")
    np.testing.assert_allclose(b, 2 * a, rtol=1e-6, atol=1e-30)


def test_token_outputs_match_the_permuted_pipeline():
    rng = np.random.default_rng(13)
    T, h, E, K, f = 50, 16, 8, 2, 24
    x = oracle.round_bf16(rng.standard_normal((T, h)))
    w_r = rng.standard_normal((E, h)).astype(np.float32)
    ws = tuple(oracle.round_bf16(rng.standard_normal(s) * 0.1) for s in ((E, f, h), (E, f, h), (E, h, f)))
    res = oracle.moe_forward(x, w_r, None, ws, K=K, dtype="bf16", capacity_factor=0.6)
    got = oracle.token_outputs(range(T), x, res["routing_map"], res["probs"], ws, "bf16")
    np.testing.assert_array_equal(got, res["out"])
