"""The MoE layer forward, written out plainly in NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (web pages; cited by title and section):
  [MC]  "MoE我们喜欢你（三）：Megatron Core MoE 源码路径解析" — §2 main path
        (route -> dispatch -> experts -> combine, shared expert added after),
        §3 gating, §4 TopKRouter routing, §5 score functions, §8 token
        dropping, §9 dispatcher layouts, §10 grouped experts, §11 shared expert.
  [DS]  "MoE Internals: DeepSpeed-Megatron Expert Parallel Implementation" —
        §3 launch knobs (capacity factor, minimum capacity), §8 the forward
        steps (flatten, gate, capacity, permute, experts, unpermute+combine).
  [MG]  "Scalable Training of Mixture-of-Experts Models with Megatron Core"
        (daily-arxiv summary) — overall framework: router + dispatcher +
        experts, four-stage forward.

Readings taken where the pages are silent are listed next to each function.
Floating point is float64 with one rounding wherever the layer stores a
tensor (logits, probs: fp32; expert activations and outputs: the layer dtype).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence, Tuple, Union

import numpy as np

from .fp32spec import sigmoid_spec, sqrtsoftplus_spec

F32 = np.float32
F64 = np.float64

# --------------------------------------------------------------------------
# rounding to the storage dtypes
# --------------------------------------------------------------------------


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range: a value
    m * 2^ex with 0.5 <= |m| < 1 is rounded to a multiple of 2^(ex-8), and
    never to a finer step than the subnormal quantum 2^-133.  Returns float64.
    """
    a = np.asarray(a, dtype=F64)
    out = a.copy()
    mask = np.isfinite(a) & (a != 0.0)
    _, ex = np.frexp(a[mask])
    q = np.maximum(ex - 8, -133)
    out[mask] = np.ldexp(np.rint(np.ldexp(a[mask], -q)), q)
    big = np.abs(out) > 3.3895313892515355e38  # largest finite bf16
    out[big] = np.copysign(np.inf, out[big])
    return out


def round_to(a, dtype: str) -> np.ndarray:
    """Round float64 values to the layer's storage dtype ("bf16" or "f32")."""
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=F64).astype(F32).astype(F64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# router: gating, score function, top-k   ([MC] §3, §4, §5)
# --------------------------------------------------------------------------


def router_logits(x, w_router, b_router=None) -> np.ndarray:
    """Gating linear in the router dtype: logits[t,e] = x[t]·w[e] (+ b[e]).

    [MC] §3: the router casts its input to the router dtype (fp32 here) and
    applies a linear gate with an optional bias.  bf16 inputs convert to
    fp32 exactly.  Accumulated in float64, rounded once to fp32.
    """
    acc = np.asarray(x, F64) @ np.asarray(w_router, F64).T
    if b_router is not None:
        acc = acc + np.asarray(b_router, F64)[None, :]
    return acc.astype(F32)


def topk_indices(values, K: int) -> np.ndarray:
    """Per row, the indices of the K largest values in selection order.

    Order: larger value first; among equal values the lower expert index
    first (reading: the pages leave tie-breaking open and name it a source
    of train/serve mismatch, [MC] §3; lowest index wins).  A stable sort of
    the negated values gives exactly that order.
    """
    v = np.asarray(values)
    order = np.argsort(-v, axis=1, kind="stable")
    return order[:, :K]


def _softmax64(v) -> np.ndarray:
    v = np.asarray(v, F64)
    m = v.max(axis=-1, keepdims=True)
    e = np.exp(v - m)
    return e / e.sum(axis=-1, keepdims=True)


def score_and_select(logits, K: int, score: str = "softmax", pre_softmax: bool = True,
                     expert_bias=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Top-k routing with a score function ([MC] §5).

    softmax, pre_softmax=True:  scores = softmax over all E; the k largest
        scores are chosen and their scores are the probs.  Softmax is
        strictly increasing in the logit, so the choice is made on the fp32
        logits themselves (the exact-arithmetic order; a rounded exp could
        only add spurious ties).
    softmax, pre_softmax=False: the k largest logits are chosen and the
        probs are the softmax over those k logits (they sum to 1).
    sigmoid: s = sigmoid(logit) in fp32 (evaluated by fp32spec.sigmoid_spec).
        With an expert bias the choice is made on s + bias (one fp32 add) and
        the probs come from the unbiased s of the chosen experts; the probs
        are s / (sum of chosen s + 1e-20).
    sqrtsoftplus: as sigmoid with s = sqrt(softplus(logit)) in fp32
        (fp32spec.sqrtsoftplus_spec); the page handles both the same way.

    Returns (probs [T,E] fp32, zero off the map; routing_map [T,E] uint8;
    scores [T,E] fp32 = the score function over all E: the full softmax for
    both softmax modes, s for sigmoid and sqrtsoftplus).
    """
    l = np.asarray(logits, F32)
    T, E = l.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    rows = np.arange(T)[:, None]
    if score == "softmax":
        sel = topk_indices(l, K)
        full = _softmax64(l)
        if pre_softmax:
            p_sel = full[rows, sel]
        else:
            p_sel = _softmax64(l[rows, sel])
        scores = full.astype(F32)
    elif score in ("sigmoid", "sqrtsoftplus"):
        s = sigmoid_spec(l) if score == "sigmoid" else sqrtsoftplus_spec(l)
        key = s if expert_bias is None else (s + np.asarray(expert_bias, F32)[None, :]).astype(F32)
        sel = topk_indices(key, K)
        s_sel = s[rows, sel].astype(F64)
        p_sel = s_sel / (s_sel.sum(axis=1, keepdims=True) + 1e-20)
        scores = s
    else:
        raise ValueError(score)
    probs = np.zeros((T, E), F32)
    rmap = np.zeros((T, E), np.uint8)
    probs[rows, sel] = p_sel.astype(F32)
    rmap[rows, sel] = 1
    return probs, rmap, scores


# --------------------------------------------------------------------------
# capacity and token dropping   ([MC] §8, [DS] §3)
# --------------------------------------------------------------------------


def get_capacity(num_tokens: int, num_experts: int, capacity_factor: float,
                 min_capacity: int = 0) -> int:
    """Per-expert capacity: ceil(num_tokens * capacity_factor / num_experts).

    [MC] §8 calls get_capacity with num_tokens = T*K but does not print it;
    reading: the usual ceiling of the even share times the factor, raised to
    the minimum capacity knob of [DS] §3.  The factor is taken as the fp32
    value the C interface receives, and the division is done in double.
    """
    cf = float(np.float32(capacity_factor))
    cap = int(math.ceil(float(num_tokens) * cf / float(num_experts)))
    return max(cap, int(min_capacity))


def capacity_mask(probs, routing_map, capacity: int, drop_policy: str = "position") -> np.ndarray:
    """The per-expert capacity mask of [MC] §8 (uint8 [T, E]).

    When the capacity is at least the token count the mask is all ones (no
    expert can receive more than T tokens).  Otherwise, for each expert, the
    mask marks `capacity` of the T tokens, the first ones in this order:
      "position": routed tokens before unrouted ones, each in ascending token
                  order (the page ranks the routing-map entries themselves;
                  reading: among equal entries the earliest token first);
      "probs":    larger routing prob first, among equal probs the earlier
                  token (the page ranks the routing probs; same tie reading).
    Unrouted tokens have prob 0, so they only enter the mask when fewer than
    `capacity` tokens were routed to the expert.
    """
    p = np.asarray(probs, F32)
    m = np.asarray(routing_map, np.uint8)
    T, E = m.shape
    if capacity >= T:
        return np.ones((T, E), np.uint8)
    mask = np.zeros((T, E), np.uint8)
    t = np.arange(T)
    for e in range(E):
        if drop_policy == "position":
            order = np.lexsort((t, -m[:, e].astype(np.int64)))  # map desc, then t asc
        elif drop_policy == "probs":
            order = np.lexsort((t, -p[:, e].astype(F64)))       # prob desc, then t asc
        else:
            raise ValueError(drop_policy)
        mask[order[:capacity], e] = 1
    return mask


def apply_token_dropping(probs, routing_map, capacity: int, drop_policy: str = "position",
                         pad_to_capacity: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Capacity dropping ([MC] §8): final map = the capacity mask when
    padding to capacity, else routing map AND mask; final probs = probs *
    final map (nothing is re-routed or renormalised).  Returns (probs
    fp32, map uint8)."""
    mask = capacity_mask(probs, routing_map, capacity, drop_policy)
    m = np.asarray(routing_map, np.uint8)
    final_map = mask if pad_to_capacity else (m & mask)
    final_probs = (np.asarray(probs, F32) * final_map).astype(F32)
    return final_probs, final_map.astype(np.uint8)


def drop_by_position(probs, routing_map, capacity: int) -> Tuple[np.ndarray, np.ndarray]:
    """Capacity dropping with the "position" policy and no padding: each
    expert keeps the first `capacity` tokens routed to it, in ascending
    token order; dropped entries get map 0 and prob 0."""
    return apply_token_dropping(probs, routing_map, capacity, "position", False)


def route(x=None, w_router=None, b_router=None, *, K: int, score: str = "softmax",
          pre_softmax: bool = True, expert_bias=None, capacity_factor: float = 0.0,
          min_capacity: int = 0, drop_policy: str = "position", pad_to_capacity: bool = False,
          logits=None) -> Dict[str, np.ndarray]:
    """The router: gating -> score/top-k -> optional capacity drop ([MC] §4).

    Pass `logits` to route given fp32 logits (skipping the gating linear).
    Returns logits, scores, pre-drop probs/map, final probs/map and
    tokens_per_expert (= routing_map summed over tokens, int32).
    """
    if logits is None:
        logits = router_logits(x, w_router, b_router)
    logits = np.asarray(logits, F32)
    probs0, map0, scores = score_and_select(logits, K, score, pre_softmax, expert_bias)
    T, E = logits.shape
    if capacity_factor > 0:
        cap = get_capacity(T * K, E, capacity_factor, min_capacity)
        probs, rmap = apply_token_dropping(probs0, map0, cap, drop_policy, pad_to_capacity)
    else:
        cap = -1
        probs, rmap = probs0, map0
    return {
        "logits": logits, "scores": scores, "probs_pre": probs0, "map_pre": map0,
        "probs": probs, "routing_map": rmap, "capacity": cap,
        "tokens_per_expert": rmap.sum(axis=0).astype(np.int32),
    }


# --------------------------------------------------------------------------
# router side outputs: load-balancing loss value, expert-bias controller
#   ([MC] §6, §7)
# --------------------------------------------------------------------------


def aux_loss(scores, tokens_per_expert, K: int, score: str = "softmax") -> float:
    """Forward value of the switch load-balancing loss, E * sum_i f_i * P_i
    ([MC] §6).

    f_i = tokens_per_expert[i] / (T * K): the share of the T*K routing
          assignments that expert i actually received (the final map, after
          any dropping: the page applies the loss after token dropping, §4);
    P_i = mean over tokens of the router's probability mass on expert i: the
          full softmax for softmax scoring; for sigmoid and sqrtsoftplus the
          scores normalised per token to sum 1 (+1e-20, as for the probs).
    Uniform routing gives exactly 1.  No coefficient is applied.
    """
    s = np.asarray(scores, F64)
    T, E = s.shape
    if T == 0:
        return 0.0
    if score != "softmax":
        s = s / (s.sum(axis=1, keepdims=True) + 1e-20)
    P = s.mean(axis=0)
    f = np.asarray(tokens_per_expert, F64) / float(T * K)
    return float(E * np.sum(f * P))


def accumulate_tokens(local_tokens_per_expert, tokens_per_expert) -> np.ndarray:
    """The controller's running count ([MC] §7): local += this batch's
    tokens_per_expert (int64)."""
    return (np.asarray(local_tokens_per_expert, np.int64) +
            np.asarray(tokens_per_expert, np.int64)).astype(np.int64)


def update_expert_bias(local_tokens_per_expert, expert_bias, update_rate: float) -> np.ndarray:
    """One step of the loss-free balance controller ([MC] §7): an expert
    loaded above the mean count moves its bias down by the rate, one below
    the mean moves it up, one at the mean keeps it.

    bias_new = bias + sign(mean - count) * rate, one fp32 add.  Reading: the
    sign is decided exactly (sign(sum - E*count) in integers), so no
    rounding of the mean can flip it.  On one GPU there is no all-reduce.
    """
    c = np.asarray(local_tokens_per_expert, np.int64)
    E = c.shape[0]
    d = int(c.sum()) - E * c
    sign = np.sign(d).astype(F32)
    return (np.asarray(expert_bias, F32) + sign * F32(update_rate)).astype(F32)


# --------------------------------------------------------------------------
# dispatch preprocess: permute to expert-major order   ([MC] §2, §9; [DS] §8)
# --------------------------------------------------------------------------


def permute(x, routing_map, probs, K: int) -> Dict[str, np.ndarray]:
    """Token rows from token-major to expert-major order.

    Row order: every (expert e, token t) with routing_map[t,e] = 1, sorted by
    e and then by t (reading: the page says expert-major; ascending token
    order inside an expert makes the order unique).
      permuted_x[i]     = x[t_i]           (exact copy)
      permuted_probs[i] = probs[t_i, e_i]
      sorted_token[i]   = t_i
      expert_offsets    = [0, n_0, n_0+n_1, ...]  (E+1 entries)
      row_id_map[t, k]  = row of token t's k-th weighted entry (map 1 and
                          prob != 0) in ascending expert order, -1 for
                          unused slots (K columns).  Entries with prob 0
                          (capacity padding) have rows but add nothing to
                          the combine, so they take no slot; a token has at
                          most K nonzero probs.
    """
    rmap = np.asarray(routing_map).astype(bool)
    T, E = rmap.shape
    e_idx, t_idx = np.nonzero(rmap.T)            # row-major over [E, T]: e, then t
    counts = rmap.sum(axis=0).astype(np.int64)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    row_id_map = np.full((T, K), -1, np.int32)
    slot = np.zeros(T, np.int64)
    # visit rows token by token in ascending expert order to fill the slots
    order = np.lexsort((e_idx, t_idx))
    pr = np.asarray(probs, F32)
    for i in order:
        t = t_idx[i]
        if pr[t, e_idx[i]] == 0:
            continue
        k = slot[t]
        if k >= K:
            raise ValueError(f"token {t} has more than K={K} nonzero probs")
        row_id_map[t, k] = i
        slot[t] = k + 1
    return {
        "permuted_x": np.asarray(x)[t_idx],
        "permuted_probs": np.asarray(probs, F32)[t_idx, e_idx],
        "sorted_token": t_idx.astype(np.int32),
        "row_expert": e_idx.astype(np.int32),
        "row_id_map": row_id_map,
        "expert_offsets": offsets.astype(np.int32),
        "tokens_per_expert": counts.astype(np.int32),
    }


# --------------------------------------------------------------------------
# experts: SwiGLU MLP per expert   ([MC] §10; [DS] §5)
# --------------------------------------------------------------------------


def swiglu_rows(xr, w_gate, w_up, w_down, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """SwiGLU expert MLP on rows xr: y = W_down (silu(W_gate x) * (W_up x)).

    The pages name the expert an MLP ([DS] §5, [MC] §10) without the
    activation; the layer shapes ask for SwiGLU: silu(g) = g * sigmoid(g),
    no biases.  Weight layouts: w_gate, w_up [f, h]; w_down [h, f].
    Products accumulate in float64; the activation is stored in the layer
    dtype (one rounding), then the down projection is rounded once more.
    Returns (act [rows, f], y [rows, h]), both float64 holding dtype values.
    """
    xr = np.asarray(xr, F64)
    g = xr @ np.asarray(w_gate, F64).T
    u = xr @ np.asarray(w_up, F64).T
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    act = round_to(silu * u, dtype)
    y = round_to(act @ np.asarray(w_down, F64).T, dtype)
    return act, y


WeightSource = Union[Sequence[np.ndarray], Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]]


def _expert_weights(weights: WeightSource, e: int):
    if callable(weights):
        return weights(e)
    wg, wu, wd = weights
    return wg[e], wu[e], wd[e]


def grouped_experts(permuted_x, tokens_per_expert, weights: WeightSource,
                    dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """All local experts over their contiguous row ranges ([MC] §10).

    The grouped GEMM computes, for each expert e, the SwiGLU MLP of the rows
    [off_e, off_e + n_e) of the expert-major input.  Here it is a plain loop
    over experts.  `weights` is (w_gate [E,f,h], w_up [E,f,h], w_down
    [E,h,f]) or a callable e -> (w_gate[e], w_up[e], w_down[e]).
    Returns (act [N, f], expert_out [N, h]).
    """
    px = np.asarray(permuted_x, F64)
    n = np.asarray(tokens_per_expert, np.int64)
    N = int(n.sum())
    acts, ys = [], []
    off = 0
    for e in range(len(n)):
        if n[e] == 0:
            continue
        wg, wu, wd = _expert_weights(weights, e)
        a, y = swiglu_rows(px[off:off + n[e]], wg, wu, wd, dtype)
        acts.append(a)
        ys.append(y)
        off += int(n[e])
    if N == 0:
        return np.zeros((0, 0)), np.zeros((0, px.shape[1] if px.ndim == 2 else 0))
    return np.concatenate(acts), np.concatenate(ys)


# --------------------------------------------------------------------------
# combine: unpermute and weight   ([MC] §2, §11; [DS] §8)
# --------------------------------------------------------------------------


def combine(expert_out, permuted_probs, row_id_map, dtype: str, shared_out=None) -> np.ndarray:
    """out[t] = sum over t's used slots k (ascending) of p[row] * y[row]
    (+ shared_out[t]), accumulated in float64, rounded once to dtype.

    The router probs weight the expert outputs at combine time ([MC] §2:
    combine takes the expert output and the probs; [DS] §8: unpermute and
    combine with the gate weights).  The shared expert's output is added
    without a weight ([MC] §2, §11).  A token with no used slot gets 0
    (+ shared).
    """
    y = np.asarray(expert_out, F64)
    p = np.asarray(permuted_probs, F64)
    rid = np.asarray(row_id_map)
    T, K = rid.shape
    H = y.shape[1] if y.ndim == 2 and y.shape[0] else (np.asarray(shared_out).shape[1] if shared_out is not None else 0)
    out = np.zeros((T, H), F64)
    for k in range(K):
        r = rid[:, k]
        used = r >= 0
        out[used] += p[r[used], None] * y[r[used]]
    if shared_out is not None:
        out += np.asarray(shared_out, F64)
    return round_to(out, dtype)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------


def moe_forward(x, w_router, b_router, weights: WeightSource, *, K: int, dtype: str,
                score: str = "softmax", pre_softmax: bool = True, expert_bias=None,
                capacity_factor: float = 0.0, min_capacity: int = 0,
                drop_policy: str = "position", pad_to_capacity: bool = False,
                shared: Optional[Sequence[np.ndarray]] = None,
                logits=None) -> Dict[str, np.ndarray]:
    """route -> permute -> experts -> combine (+ shared expert) ([MC] §2).

    `shared` = (shared_gate [fs,h], shared_up [fs,h], shared_down [h,fs]) or
    None.  Pass `logits` to route from given fp32 logits.
    """
    r = route(x, w_router, b_router, K=K, score=score, pre_softmax=pre_softmax,
              expert_bias=expert_bias, capacity_factor=capacity_factor,
              min_capacity=min_capacity, drop_policy=drop_policy,
              pad_to_capacity=pad_to_capacity, logits=logits)
    pm = permute(x, r["routing_map"], r["probs"], K)
    act, y = grouped_experts(pm["permuted_x"], pm["tokens_per_expert"], weights, dtype)
    shared_out = None
    if shared is not None:
        _, shared_out = swiglu_rows(x, shared[0], shared[1], shared[2], dtype)
    out = combine(y, pm["permuted_probs"], pm["row_id_map"], dtype, shared_out)
    res = dict(r)
    res.update(pm)
    res.update({"act": act, "expert_out": y, "shared_out": shared_out, "out": out})
    return res


def token_outputs(tokens, x, routing_map, probs, weights: WeightSource, dtype: str,
                  shared: Optional[Sequence[np.ndarray]] = None) -> np.ndarray:
    """The layer output for selected tokens only, straight from the routing.

    For each token t: sum over its routed experts in ascending order of
    probs[t,e] * SwiGLU_e(x[t]) (+ the shared expert of x[t]), float64,
    rounded once.  Needs the batch routing (capacity couples tokens) but
    only the experts these tokens use, so it scales to full-size layers.
    """
    x = np.asarray(x)
    rmap = np.asarray(routing_map)
    p = np.asarray(probs, F64)
    cache = {}
    outs = []
    for t in tokens:
        acc = np.zeros(x.shape[1], F64)
        for e in np.nonzero(rmap[t])[0]:
            if e not in cache:
                cache[e] = _expert_weights(weights, int(e))
            wg, wu, wd = cache[e]
            _, y = swiglu_rows(x[t:t + 1], wg, wu, wd, dtype)
            acc += p[t, e] * y[0]
        if shared is not None:
            _, ys = swiglu_rows(x[t:t + 1], shared[0], shared[1], shared[2], dtype)
            acc += ys[0]
        outs.append(acc)
    return round_to(np.stack(outs) if outs else np.zeros((0, x.shape[1])), dtype)
