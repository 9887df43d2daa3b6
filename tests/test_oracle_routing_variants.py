"""Pins of the oracle's routing variants: the probs drop policy, padding to
capacity, the sqrt-softplus score, the load-balancing loss value and the
expert-bias controller.  Each is checked against hand-derived cases
(tests/golden), closed forms, brute force or invariants; no GPU is used."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(v):
    return float(eval(v, {"math": math})) if isinstance(v, str) else float(v)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _probs_map(g):
    T, E = g["T"], g["E"]
    probs = np.zeros((T, E), np.float32)
    rmap = np.zeros((T, E), np.uint8)
    for t, (e, p) in enumerate(zip(g["route_to"], g["prob"])):
        probs[t, e] = p
        rmap[t, e] = 1
    return probs, rmap


# ------------------------------------------------------- capacity variants

@pytest.mark.parametrize("case", range(4))
def test_capacity_variants_worked(case):
    g = _golden("capacity_probs_worked.json")
    c = g["cases"][case]
    probs, rmap = _probs_map(g)
    fp, fm = oracle.apply_token_dropping(probs, rmap, c["capacity"], c["policy"], c["pad"])
    np.testing.assert_array_equal(fm, np.array(c["final_map"], np.uint8))
    np.testing.assert_array_equal(fm.sum(axis=0), c["tokens_per_expert"])
    np.testing.assert_array_equal(fp, probs * fm)
    if "sorted_token" in c:
        x = np.arange(g["T"], dtype=np.float64)[:, None] * np.ones((1, 4))
        pm = oracle.permute(x, fm, fp, g["K"])
        np.testing.assert_array_equal(pm["sorted_token"], c["sorted_token"])
        np.testing.assert_allclose(pm["permuted_probs"], np.float32(c["permuted_probs"]))
        np.testing.assert_array_equal(pm["row_id_map"], c["row_id_map"])


def _random_routing(rng, T, E, K):
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 1.5
    logits[rng.integers(0, T, T // 4)] = np.round(logits[rng.integers(0, T, T // 4)])  # ties
    return oracle.route(logits=logits, K=K)


@pytest.mark.parametrize("T,E,K,cap", [(40, 4, 1, 7), (33, 6, 2, 5), (25, 3, 3, 9), (12, 5, 2, 1)])
def test_probs_policy_keeps_the_largest_probs(T, E, K, cap):
    """Brute-force check of the probs policy: for each expert the kept set
    has min(cap, n_e) routed tokens and no dropped routed token outranks a
    kept one under (prob descending, token ascending)."""
    r = _random_routing(np.random.default_rng(T * E + K), T, E, K)
    p0, m0 = r["probs"], r["routing_map"]
    fp, fm = oracle.apply_token_dropping(p0, m0, cap, "probs", False)
    for e in range(E):
        routed = [t for t in range(T) if m0[t, e]]
        kept = [t for t in routed if fm[t, e]]
        dropped = [t for t in routed if not fm[t, e]]
        assert len(kept) == min(cap, len(routed))
        for a in kept:
            for b in dropped:
                assert (p0[a, e] > p0[b, e]) or (p0[a, e] == p0[b, e] and a < b)
    assert not (fm & (1 - m0)).any()
    np.testing.assert_array_equal(fp, p0 * fm)


def test_probs_policy_equals_position_policy_for_equal_probs():
    """With every routed prob equal (top-1 over E = 1: prob 1), ranking by
    probs falls back to token order, i.e. the position policy."""
    T, E = 30, 1
    probs = np.ones((T, E), np.float32)
    rmap = np.ones((T, E), np.uint8)
    a = oracle.apply_token_dropping(probs, rmap, 11, "probs", False)
    b = oracle.apply_token_dropping(probs, rmap, 11, "position", False)
    np.testing.assert_array_equal(a[1], b[1])
    assert a[1][:11].all() and not a[1][11:].any()


def test_probs_policy_increasing_probs_keeps_the_last_tokens():
    T = 20
    probs = np.linspace(0.1, 0.9, T).astype(np.float32)[:, None]
    rmap = np.ones((T, 1), np.uint8)
    _, fm = oracle.apply_token_dropping(probs, rmap, 6, "probs", False)
    assert fm[-6:].all() and not fm[:-6].any()


@pytest.mark.parametrize("policy", ["position", "probs"])
@pytest.mark.parametrize("T,E,K,cap", [(40, 4, 1, 13), (33, 6, 2, 12), (16, 8, 2, 3)])
def test_padding_to_capacity_invariants(policy, T, E, K, cap):
    r = _random_routing(np.random.default_rng(T + E + cap), T, E, K)
    p0, m0 = r["probs"], r["routing_map"]
    fp_pad, fm_pad = oracle.apply_token_dropping(p0, m0, cap, policy, True)
    fp, fm = oracle.apply_token_dropping(p0, m0, cap, policy, False)
    np.testing.assert_array_equal(fm_pad.sum(axis=0), np.full(E, min(cap, T)))
    np.testing.assert_array_equal(fm_pad & m0, fm)           # same routed entries kept
    np.testing.assert_array_equal(fp_pad, fp)                # padding carries prob 0
    # padding entries are the earliest unrouted tokens
    for e in range(E):
        pad_rows = np.nonzero(fm_pad[:, e] & (1 - m0[:, e]))[0]
        unrouted = np.nonzero(1 - m0[:, e])[0]
        np.testing.assert_array_equal(pad_rows, unrouted[:len(pad_rows)])


def test_capacity_at_least_tokens_keeps_everything_and_pads_everything():
    r = _random_routing(np.random.default_rng(3), 10, 4, 2)
    p0, m0 = r["probs"], r["routing_map"]
    fp, fm = oracle.apply_token_dropping(p0, m0, 10, "probs", False)
    np.testing.assert_array_equal(fm, m0)
    _, fm_pad = oracle.apply_token_dropping(p0, m0, 10, "probs", True)
    assert fm_pad.all()


@pytest.mark.parametrize("policy", ["position", "probs"])
def test_padded_layer_output_equals_unpadded(policy):
    """Padding adds rows with prob 0, so the layer output is unchanged."""
    rng = np.random.default_rng(5)
    T, h, E, K, f = 24, 16, 4, 2, 32
    x = rng.standard_normal((T, h))
    wr = rng.standard_normal((E, h)) / 4
    w = (rng.standard_normal((E, f, h)) * 0.3, rng.standard_normal((E, f, h)) * 0.3,
         rng.standard_normal((E, h, f)) * 0.3)
    kw = dict(K=K, dtype="f32", capacity_factor=0.75, drop_policy=policy)
    a = oracle.moe_forward(x, wr, None, w, pad_to_capacity=False, **kw)
    b = oracle.moe_forward(x, wr, None, w, pad_to_capacity=True, **kw)
    assert b["tokens_per_expert"].tolist() == [a["capacity"]] * E
    np.testing.assert_array_equal(a["out"], b["out"])


# ------------------------------------------------------------ sqrtsoftplus

def _ulp(v):
    return np.spacing(np.abs(np.asarray(v, np.float32))).astype(np.float64)


def test_log1p_spec_accuracy():
    u = np.linspace(0, 1, 400001).astype(np.float32)
    got = oracle.log1p_spec(u).astype(np.float64)
    ref = np.log1p(u.astype(np.float64))
    m = u > 0
    assert (np.abs(got - ref)[m] / _ulp(ref[m])).max() <= 3.0
    assert oracle.log1p_spec(np.float32([0.0]))[0] == 0.0


def test_sqrtsoftplus_spec_accuracy_and_special_values():
    x = np.linspace(-86, 40, 1000001).astype(np.float32)
    got = oracle.sqrtsoftplus_spec(x).astype(np.float64)
    ref = np.sqrt(np.log1p(np.exp(x.astype(np.float64))))
    assert (np.abs(got - ref) / _ulp(ref)).max() <= 2.0
    assert np.all(np.diff(oracle.sqrtsoftplus_spec(x)) >= 0)      # monotone: same order
    big = np.float32([20.5, 100.0, 1e6])
    np.testing.assert_array_equal(oracle.sqrtsoftplus_spec(big), np.sqrt(big))
    assert oracle.sqrtsoftplus_spec(np.float32([-100.0]))[0] == 0.0
    z = oracle.sqrtsoftplus_spec(np.float32([0.0]))[0]
    assert abs(float(z) - math.sqrt(math.log(2.0))) <= float(_ulp(z))


def test_sqrtsoftplus_routing_without_bias_selects_top_logits():
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((200, 12)).astype(np.float32) * 3
    for K in (1, 3, 5):
        r = oracle.route(logits=logits, K=K, score="sqrtsoftplus")
        top = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        ref = np.zeros_like(r["routing_map"])
        np.put_along_axis(ref, top, 1, axis=1)
        np.testing.assert_array_equal(r["routing_map"], ref)
        np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, rtol=1e-6)


def test_sqrtsoftplus_bias_changes_choice_not_weights():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((64, 8)).astype(np.float32)
    bias = np.float32([5, 0, 0, 0, 0, 0, 0, 5])
    r = oracle.route(logits=logits, K=2, score="sqrtsoftplus", expert_bias=bias)
    assert r["routing_map"][:, 0].all() and r["routing_map"][:, 7].all()
    s = oracle.sqrtsoftplus_spec(logits).astype(np.float64)
    ref = s[:, [0, 7]] / (s[:, [0, 7]].sum(axis=1, keepdims=True) + 1e-20)
    np.testing.assert_allclose(r["probs"][:, [0, 7]], ref, rtol=1e-6)


# ----------------------------------------------------- aux loss, expert bias

def test_aux_loss_worked():
    g = _golden("aux_bias_worked.json")["aux"]
    logits = np.array([[_ev(v) for v in row] for row in g["logits"]], np.float32)
    r = oracle.route(logits=logits, K=g["K"])
    np.testing.assert_array_equal(r["tokens_per_expert"], g["tokens_per_expert"])
    loss = oracle.aux_loss(r["scores"], r["tokens_per_expert"], g["K"], "softmax")
    assert abs(loss - _ev(g["loss"])) < 1e-6


@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrtsoftplus"])
def test_aux_loss_is_one_when_either_side_is_uniform(score):
    rng = np.random.default_rng(11)
    T, E, K = 64, 8, 2
    # equal logits: P uniform, any routing
    r = oracle.route(logits=np.zeros((T, E), np.float32), K=K, score=score)
    assert abs(oracle.aux_loss(r["scores"], r["tokens_per_expert"], K, score) - 1.0) < 1e-12
    # uniform counts, random P
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits=logits, K=K, score=score)
    n = np.full(E, T * K // E)
    assert abs(oracle.aux_loss(r["scores"], n, K, score) - 1.0) < 1e-6  # fp32 scores sum to 1


def test_aux_loss_all_on_one_expert_tends_to_E():
    T, E, K = 50, 6, 1
    logits = np.zeros((T, E), np.float32)
    logits[:, 2] = 60.0
    r = oracle.route(logits=logits, K=K)
    assert r["tokens_per_expert"].tolist() == [0, 0, T, 0, 0, 0]
    assert abs(oracle.aux_loss(r["scores"], r["tokens_per_expert"], K) - E) < 1e-12


def test_expert_bias_step_worked():
    g = _golden("aux_bias_worked.json")["bias"]
    new = oracle.update_expert_bias(np.array(g["counts"]), np.float32(g["bias"]), g["rate"])
    ref = np.float32(g["bias"]) + np.float32(g["sign"]) * np.float32(g["rate"])
    np.testing.assert_array_equal(new, ref)


def test_expert_bias_sign_is_decided_exactly():
    """Counts near 2^24: the mean 50331652/3 is not an fp32 value and a
    rounded mean compared with a rounded count could give the wrong sign;
    the exact decision is mean > count for experts 0, 1 and mean < count for
    expert 2."""
    c = np.array([16777217, 16777217, 16777218], np.int64)
    new = oracle.update_expert_bias(c, np.zeros(3, np.float32), 1.0)
    np.testing.assert_array_equal(new, np.float32([1, 1, -1]))
    acc = oracle.accumulate_tokens(oracle.accumulate_tokens(np.zeros(3, np.int64), [1, 2, 3]), [4, 5, 6])
    np.testing.assert_array_equal(acc, [5, 7, 9])
