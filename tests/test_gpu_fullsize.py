"""Full-size parity of the layer as the benchmark runs it (route + permute
as one call, gathering FC1, shared expert folded into the routed launches),
on whole experts and on 256 tokens.

For the DeepSeek-V3-, Mixtral- and Qwen3-shaped layers: every row and every column
of act and expert_out for the busiest expert, for an expert whose last
m-tile is ragged, and (DeepSeek-V3-shaped) for the smallest expert; and the
layer output of 256 random tokens, element by element, at the bf16
tolerance.  The oracle's routing is computed from the GPU's fp32 logits and
must equal the GPU's bit for bit.  Expert weights are brought to the host
one expert at a time."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from combine_router_gating_amd.layer import MoELayerForward
from gpu_helpers import assert_close, f64, log, routing_ref

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M_TILE = 256  # rows per m-tile of these layers' FC1 and FC2 launches


def _weights(inp, e):
    return f64(inp["w_gate"][e]), f64(inp["w_up"][e]), f64(inp["w_down"][e])


def _token_outputs_by_expert(toks, x, rmap, probs, inp, shared, dtype):
    """oracle layer output of the given tokens: each expert's SwiGLU on the
    sampled tokens routed to it (weights loaded once per expert), weighted
    by the probs and summed in ascending expert order, + the shared expert,
    rounded once."""
    toks = np.asarray(toks)
    acc = np.zeros((len(toks), x.shape[1]))
    sub = rmap[toks]
    for e in np.nonzero(sub.any(axis=0))[0]:
        sel = np.nonzero(sub[:, e])[0]
        wg, wu, wd = _weights(inp, int(e))
        _, y = oracle.swiglu_rows(x[toks[sel]], wg, wu, wd, dtype)
        acc[sel] += probs[toks[sel], e][:, None] * y
    if shared is not None:
        _, ys = oracle.swiglu_rows(x[toks], shared[0], shared[1], shared[2], dtype)
        acc += ys
    return oracle.round_to(acc, dtype)


@pytest.mark.parametrize("name", ["dsv3", "mixtral", "qwen3"])
def test_bench_layer_whole_experts_and_256_tokens(name):
    cfg = datagen.CONFIGS[name]
    log(f"full-size whole experts: {cfg}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                            capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity,
                            gather=True)
    assert layer.fold_shared == ("shared_gate" in inp)
    out = layer.forward()
    torch.cuda.synchronize()
    logits = layer.logits.cpu().numpy()
    eb = inp["expert_bias"].cpu().numpy() if "expert_bias" in inp else None
    ref = routing_ref(cfg, logits, eb)
    rmap = ref["routing_map"]
    np.testing.assert_array_equal(layer.routing_map.cpu().numpy(), rmap)
    n = ref["tokens_per_expert"]
    np.testing.assert_array_equal(layer.tokens_per_expert.cpu().numpy(), n)
    offs = np.concatenate([[0], np.cumsum(n)])
    np.testing.assert_array_equal(layer.expert_offsets.cpu().numpy(), offs)
    st = layer.sorted_token.cpu().numpy()
    xs = f64(inp["x"])

    busiest = int(np.argmax(n))
    ragged = [e for e in np.argsort(-n) if n[e] > M_TILE and n[e] % M_TILE not in (0,)
              and e != busiest]
    experts = [busiest] + ([int(ragged[0])] if ragged else [])
    nz = np.nonzero(n)[0]
    smallest = int(nz[np.argmin(n[nz])])
    if n[smallest] < 64 and smallest not in experts:
        experts.append(smallest)  # a one-tile expert with mostly padding rows
    for e in experts:
        rows = np.arange(offs[e], offs[e + 1])
        log(f"  expert {e}: {len(rows)} rows (last m-tile {len(rows) % M_TILE or M_TILE} rows)")
        wg, wu, wd = _weights(inp, e)
        act, y = oracle.swiglu_rows(xs[st[rows]], wg, wu, wd, cfg.dtype)
        idx = torch.from_numpy(rows).to(DEV)
        assert_close(f64(layer.act[idx]), act, cfg.dtype, f"act[{name}, e={e}]")
        assert_close(f64(layer.expert_out[idx]), y, cfg.dtype, f"expert_out[{name}, e={e}]")
    if layer.shared:
        # the folded shared expert on 256 whole rows (one dense m-tile)
        sw = tuple(f64(inp[k]) for k in ("shared_gate", "shared_up", "shared_down"))
        t0 = 1024
        sact, sy = oracle.swiglu_rows(xs[t0:t0 + M_TILE], *sw, cfg.dtype)
        assert_close(f64(layer.shared_act[t0:t0 + M_TILE]), sact, cfg.dtype, "shared_act")
        assert_close(f64(layer.shared_out[t0:t0 + M_TILE]), sy, cfg.dtype, "shared_out")
    else:
        sw = None
    toks = np.sort(np.random.default_rng(7).choice(cfg.T, size=256, replace=False))
    exp = _token_outputs_by_expert(toks, xs, rmap, ref["probs"], inp, sw, cfg.dtype)
    assert_close(f64(out)[toks], exp, cfg.dtype, f"out[{name}, 256 tokens]")
