"""GPU checks of the fused/overlapped layer variants.

The gathering FC1 (rows read through sorted_token instead of a permuted
copy) and the shared expert on a second stream change where data is read
and when kernels run, not the arithmetic: outputs must equal the plain
path bit for bit, and the plain path is itself checked against the oracle
elsewhere.  A small layer is also compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

import combine_router_gating_amd as moe
import datagen
import oracle
from combine_router_gating_amd.layer import MoELayerForward
from gpu_helpers import assert_close, f64, log, shared_weights_from

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CFGS = [
    datagen.MoEConfig("g-bf16", T=300, h=256, E=8, K=2, f=512, dtype="bf16"),
    datagen.MoEConfig("g-cap", T=515, h=128, E=16, K=1, f=256, dtype="bf16", capacity_factor=1.25,
                      gate_bias="zipf"),
    datagen.MoEConfig("g-sig", T=257, h=256, E=64, K=8, f=128, dtype="bf16", score="sigmoid",
                      expert_bias=True, shared_f=192),
    datagen.MoEConfig("g-f32", T=99, h=64, E=4, K=4, f=96, dtype="f32", shared_f=64,
                      capacity_factor=0.5),
]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_gather_fc1_equals_permuted_fc1(cfg):
    log(f"gather fc1: {cfg}")
    inp = datagen.make_inputs(cfg, seed=3, device=DEV)
    kw = dict(K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
              capacity_factor=cfg.capacity_factor)
    a = moe.moe_forward(inp, gather=False, **kw)
    b = moe.moe_forward(inp, gather=True, **kw)
    torch.cuda.synchronize()
    N = int(a["expert_offsets"][-1].item())
    assert b["permuted_x"] is None
    assert torch.equal(a["act"][:N], b["act"][:N])
    assert torch.equal(a["out"], b["out"])
    # and the gathered activation against the oracle
    st = a["sorted_token"][:N].cpu().numpy()
    w = (f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"]))
    act, _ = oracle.grouped_experts(f64(inp["x"])[st], a["tokens_per_expert"].cpu().numpy(), w,
                                    cfg.dtype)
    assert_close(f64(b["act"][:N]), act, cfg.dtype, "act")


def test_gather_clamps_out_of_range_indices():
    """sorted_token entries outside [0, T) are clamped, never dereferenced."""
    T, h, f, E = 64, 128, 128, 2
    x = torch.randn(T, h, device=DEV).to(torch.bfloat16)
    wg = (torch.randn(E, f, h, device=DEV) * 0.05).to(torch.bfloat16)
    wu = (torch.randn(E, f, h, device=DEV) * 0.05).to(torch.bfloat16)
    counts = torch.tensor([40, 24], dtype=torch.int32, device=DEV)
    st = torch.arange(64, dtype=torch.int32, device=DEV)
    st[5] = -7
    st[9] = 10 ** 6
    got = moe.moe_grouped_fc1_swiglu_gather(x, st, counts, wg, wu)
    idx = st.clamp(0, T - 1).long()
    ref = moe.moe_grouped_fc1_swiglu(x[idx].contiguous(), counts, wg, wu)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("name", ["tiny", "switch", "dsv3"])
def test_layer_options_give_identical_outputs(name):
    cfg = datagen.CONFIGS[name]
    if name == "dsv3":
        cfg = cfg.replace(T=1024)
    log(f"layer options: {cfg}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV)
    kw = dict(K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
              capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity)
    outs = []
    for gather, overlap, fuse, fcmb, fold in ((False, False, False, False, False),
                                              (True, False, True, True, True),
                                              (True, True, True, False, False),
                                              (False, True, False, True, True),
                                              (False, False, True, True, False),
                                              (True, False, False, False, True)):
        layer = MoELayerForward(inp, gather=gather, overlap_shared=overlap,
                                fuse_route_permute=fuse, fuse_combine=fcmb, fold_shared=fold,
                                **kw)
        for _ in range(2):
            out = layer.forward()
        torch.cuda.synchronize()
        outs.append(out.clone())
    for o in outs[1:]:
        assert torch.equal(outs[0], o)


def test_layer_overlap_graph_capture_replays():
    cfg = datagen.MoEConfig("g-graph", T=512, h=256, E=16, K=2, f=256, dtype="bf16", shared_f=128)
    inp = datagen.make_inputs(cfg, seed=5, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, gather=True, overlap_shared=True)
    layer.forward()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward()
    plain = MoELayerForward(inp, K=cfg.K)
    for seed in (6, 7, 8):
        new = datagen.make_inputs(cfg, seed=seed, device=DEV, with_experts=False)
        inp["x"].copy_(new["x"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = plain.forward()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay with seed {seed}"


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
@pytest.mark.parametrize("fold", [False, True])
def test_tile_queue_graph_capture_replays(precision, fold):
    """Experts of ~512 rows, so the grouped GEMMs run their tile-queue
    launches (with the shared expert's tiles in the same queue when folded):
    the queue's counters are reset by the launches themselves, never by a
    memset, so a captured forward replays correctly many times, with eager
    calls that use the same queue in between; every replay equals a layer
    without a queue bit for bit, and the counters end at zero."""
    cfg = datagen.MoEConfig("g-graph-queue", T=2048, h=256, E=8, K=2, f=512, dtype="bf16",
                            shared_f=256)
    log(f"tile queue graph ({precision}, fold={fold}): {cfg}")
    inp = datagen.make_inputs(cfg, seed=12, device=DEV)
    kw = dict(K=cfg.K, gather=True, precision=precision)
    layer = MoELayerForward(inp, fold_shared=fold, overlap_shared=False, tile_queue=True, **kw)
    plain = MoELayerForward(inp, fold_shared=False, overlap_shared=False, tile_queue=False, **kw)
    assert layer.queue is not None
    layer.forward()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward()
    for seed in (13, 14, 15, 16):
        new = datagen.make_inputs(cfg, seed=seed, device=DEV, with_experts=False)
        inp["x"].copy_(new["x"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = layer.forward().clone()  # the same queue, outside the graph
        ref = plain.forward()
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay with seed {seed}"
        assert torch.equal(eager, ref), f"eager call after replay, seed {seed}"
        assert int(torch.count_nonzero(layer.queue).item()) == 0


def test_small_layer_with_options_against_the_oracle():
    cfg = CFGS[2]
    inp = datagen.make_inputs(cfg, seed=9, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, score=cfg.score, gather=True, overlap_shared=True)
    out = layer.forward()
    torch.cuda.synchronize()
    logits = layer.logits.cpu().numpy()
    ref = oracle.moe_forward(f64(inp["x"]), None, None,
                             (f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"])),
                             K=cfg.K, dtype=cfg.dtype, score=cfg.score,
                             expert_bias=inp["expert_bias"].cpu().numpy(),
                             shared=shared_weights_from(inp), logits=logits)
    np.testing.assert_array_equal(layer.routing_map.cpu().numpy(), ref["routing_map"])
    assert_close(f64(out), ref["out"], cfg.dtype, "out")


PAD_CFGS = [
    # capacity 1.25 of a skewed top-1 router: some experts get fewer routed
    # tokens than the capacity and are padded with tokens routed elsewhere
    datagen.MoEConfig("pad-top1", T=515, h=128, E=16, K=1, f=256, dtype="bf16",
                      capacity_factor=1.25, gate_bias="zipf"),
    # capacity >= T: every token reaches every expert, all but one row of
    # each token carry prob 0
    datagen.MoEConfig("pad-all", T=96, h=128, E=4, K=1, f=128, dtype="bf16",
                      capacity_factor=8.0),
]


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
@pytest.mark.parametrize("policy", ["position", "probs"])
@pytest.mark.parametrize("cfg", PAD_CFGS, ids=lambda c: c.name)
def test_fused_combine_with_padding_to_capacity(cfg, policy, precision):
    """FC2 with the top-1 combine on a padded map: a token's padded rows
    (prob 0, in other experts) must not overwrite its output.  The fused
    output equals FC2 followed by the combine bit for bit, and the bf16
    layer matches the oracle."""
    log(f"fused combine, padded map ({policy}, {precision}): {cfg}")
    inp = datagen.make_inputs(cfg, seed=11, device=DEV)
    kw = dict(K=cfg.K, capacity_factor=cfg.capacity_factor, drop_policy=policy,
              pad_to_capacity=True, gather=True, precision=precision)
    fused = MoELayerForward(inp, fuse_combine=True, **kw)
    plain = MoELayerForward(inp, fuse_combine=False, **kw)
    assert fused.fused_combine and not plain.fused_combine
    a = fused.forward().clone()
    b = plain.forward().clone()
    torch.cuda.synchronize()
    N = int(fused.expert_offsets[-1].item())
    # the padding really gave some token rows beyond its combine slot
    assert N > int((fused.row_id_map >= 0).sum().item())
    assert torch.equal(a, b)
    if precision == "bf16":
        ref = oracle.moe_forward(f64(inp["x"]), None, None,
                                 (f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"])),
                                 K=cfg.K, dtype=cfg.dtype, capacity_factor=cfg.capacity_factor,
                                 drop_policy=policy, pad_to_capacity=True,
                                 logits=fused.logits.cpu().numpy())
        np.testing.assert_array_equal(fused.routing_map.cpu().numpy(), ref["routing_map"])
        assert_close(f64(a), ref["out"], cfg.dtype, "out")


@pytest.mark.parametrize("T,E,K,f,fs,h", [(1024, 256, 8, 2048, 2048, 512),  # DSv3-like experts
                                          (300, 8, 2, 512, 192, 256),
                                          (77, 16, 1, 128, 320, 128)])
def test_shared_expert_folded_into_the_routed_launches(T, E, K, f, fs, h):
    """FC1 and FC2 with the shared expert's tiles appended: routed and shared
    outputs bitwise the separate calls (the shared ones as an E = 1 GEMM of
    T rows); also with no routed rows at all."""
    cfg = datagen.MoEConfig("fold", T=T, h=h, E=E, K=K, f=f, dtype="bf16", score="sigmoid",
                            expert_bias=True, shared_f=fs)
    log(f"folded shared expert: {cfg}")
    inp = datagen.make_inputs(cfg, seed=13, device=DEV)
    r = moe.moe_route_permute(inp["x"], inp["w_router"], K=K, score="sigmoid",
                              expert_bias=inp["expert_bias"], copy_rows=False)
    x, st, tpe = inp["x"], r["sorted_token"], r["tokens_per_expert"]
    act, sact = moe.moe_grouped_fc1_swiglu_gather_shared(
        x, st, tpe, inp["w_gate"], inp["w_up"], inp["shared_gate"], inp["shared_up"])
    y, sout = moe.moe_grouped_fc2_shared(act, tpe, inp["w_down"], sact, inp["shared_down"])
    ones = torch.full((1,), T, dtype=torch.int32, device=DEV)
    act_ref = moe.moe_grouped_fc1_swiglu_gather(x, st, tpe, inp["w_gate"], inp["w_up"])
    sact_ref = moe.moe_grouped_fc1_swiglu(x, ones, inp["shared_gate"][None], inp["shared_up"][None])
    y_ref = moe.moe_grouped_fc2(act_ref, tpe, inp["w_down"])
    sout_ref = moe.moe_grouped_fc2(sact_ref, ones, inp["shared_down"][None])
    torch.cuda.synchronize()
    N = int(r["expert_offsets"][-1].item())
    assert torch.equal(act[:N], act_ref[:N]) and torch.equal(y[:N], y_ref[:N])
    assert torch.equal(sact, sact_ref) and torch.equal(sout, sout_ref)
    # no routed rows: the launch is the shared expert's tiles alone
    zero = torch.zeros_like(tpe)
    _, sact0 = moe.moe_grouped_fc1_swiglu_gather_shared(
        x, st[:0], zero, inp["w_gate"], inp["w_up"], inp["shared_gate"], inp["shared_up"],
        act=act[:0])
    _, sout0 = moe.moe_grouped_fc2_shared(act[:0], zero, inp["w_down"], sact0, inp["shared_down"],
                                          expert_out=y[:0])
    torch.cuda.synchronize()
    assert torch.equal(sact0, sact_ref) and torch.equal(sout0, sout_ref)


@pytest.mark.parametrize("T,E,K,f,h,fs", [(2048, 64, 5, 512, 256, 0),      # 160 rows: no queue
                                          (2048, 64, 8, 256, 512, 256),    # + shared tail
                                          (4096, 8, 2, 256, 128, 0),       # large experts
                                          (600, 64, 1, 256, 128, 0),       # 64-row launch: no queue
                                          # k-loops of 1, 3 and 6 stages of 64 in the split-ring
                                          # body (FC1 k = h, FC2 k = f); the other GEMM of each
                                          # layer has N off the tile width and takes the plain
                                          # queue body
                                          (4096, 8, 2, 256, 64, 0),
                                          (4096, 8, 2, 256, 192, 0),
                                          (4096, 8, 2, 192, 256, 0),
                                          (4096, 8, 2, 64, 256, 0),
                                          (4096, 8, 2, 128, 384, 0)])
def test_tile_queue_matches_one_tile_per_workgroup(T, E, K, f, h, fs):
    """The tile-queue launches (one workgroup per CU taking tiles from per-XCD
    counters; the 256-row tiles on the split-ring body when N is a multiple
    of the tile width) give the same bits as one workgroup per tile, on
    repeated calls with one queue, and leave the queue zeroed."""
    cfg = datagen.MoEConfig("queue", T=T, h=h, E=E, K=K, f=f, dtype="bf16", score="sigmoid",
                            expert_bias=True, shared_f=fs)
    log(f"tile queue: {cfg}")
    inp = datagen.make_inputs(cfg, seed=17, device=DEV)
    r = moe.moe_route_permute(inp["x"], inp["w_router"], K=K, score="sigmoid",
                              expert_bias=inp["expert_bias"], copy_rows=False)
    x, st, tpe = inp["x"], r["sorted_token"], r["tokens_per_expert"]
    q = moe.gemm_queue(DEV)
    N = int(r["expert_offsets"][-1].item())
    for _ in range(3):
        if fs:
            a0, s0 = moe.moe_grouped_fc1_swiglu_gather_shared(
                x, st, tpe, inp["w_gate"], inp["w_up"], inp["shared_gate"], inp["shared_up"])
            a1, s1 = moe.moe_grouped_fc1_swiglu_gather_shared(
                x, st, tpe, inp["w_gate"], inp["w_up"], inp["shared_gate"], inp["shared_up"],
                queue=q)
            y0, o0 = moe.moe_grouped_fc2_shared(a0, tpe, inp["w_down"], s0, inp["shared_down"])
            y1, o1 = moe.moe_grouped_fc2_shared(a1, tpe, inp["w_down"], s1, inp["shared_down"],
                                                queue=q)
        else:
            a0 = moe.moe_grouped_fc1_swiglu_gather(x, st, tpe, inp["w_gate"], inp["w_up"])
            a1 = moe.moe_grouped_fc1_swiglu_gather(x, st, tpe, inp["w_gate"], inp["w_up"], queue=q)
            y0 = moe.moe_grouped_fc2(a0, tpe, inp["w_down"])
            y1 = moe.moe_grouped_fc2(a1, tpe, inp["w_down"], queue=q)
        torch.cuda.synchronize()
        assert torch.equal(a0[:N], a1[:N]) and torch.equal(y0[:N], y1[:N])
        if fs:
            assert torch.equal(s0, s1) and torch.equal(o0, o1)
        assert int(q.abs().sum().item()) == 0, "the queue is left zeroed"
    if fs:
        # no routed rows: the queue holds the shared expert's tiles alone
        zero = torch.zeros_like(tpe)
        _, s2 = moe.moe_grouped_fc1_swiglu_gather_shared(
            x, st, zero, inp["w_gate"], inp["w_up"], inp["shared_gate"], inp["shared_up"], queue=q)
        _, o2 = moe.moe_grouped_fc2_shared(a1, zero, inp["w_down"], s2, inp["shared_down"], queue=q)
        torch.cuda.synchronize()
        assert torch.equal(s2, s0) and torch.equal(o2, o0)
        assert int(q.abs().sum().item()) == 0, "the queue is left zeroed"


# every expert empty; every row in one expert; one row against the rest;
# two halves; counts summing past max_rows (the second expert is clamped
# to the rows left)
DEGENERATE_COUNTS = [[0] * 8, [4096] + [0] * 7, [1] + [0] * 6 + [4095], [0, 0, 0, 2048, 0, 0, 0, 2048],
                     [3000, 3000] + [0] * 6]


@pytest.mark.parametrize("counts", DEGENERATE_COUNTS)
def test_tile_queue_degenerate_counts(counts):
    """Queue launches (max_rows / E = 512) over degenerate counts give the
    bits of one workgroup per tile on every row the counts cover, on
    repeated calls, and leave the counters zeroed."""
    E, h, f, rows = 8, 256, 512, 4096
    g = torch.Generator(device="cpu").manual_seed(3)
    x = torch.randn(rows, h, generator=g).to(DEV, torch.bfloat16)
    wg = (torch.randn(E, f, h, generator=g) * h ** -0.5).to(DEV, torch.bfloat16)
    wu = (torch.randn(E, f, h, generator=g) * h ** -0.5).to(DEV, torch.bfloat16)
    wd = (torch.randn(E, h, f, generator=g) * f ** -0.5).to(DEV, torch.bfloat16)
    tpe = torch.tensor(counts, dtype=torch.int32, device=DEV)
    N = min(sum(counts), rows)
    log(f"tile queue, degenerate counts {counts}")
    q = moe.gemm_queue(DEV)
    for _ in range(2):
        a0 = moe.moe_grouped_fc1_swiglu(x, tpe, wg, wu)
        a1 = moe.moe_grouped_fc1_swiglu(x, tpe, wg, wu, queue=q)
        y0 = moe.moe_grouped_fc2(a0, tpe, wd)
        y1 = moe.moe_grouped_fc2(a0, tpe, wd, queue=q)
        torch.cuda.synchronize()
        assert torch.equal(a0[:N], a1[:N]) and torch.equal(y0[:N], y1[:N])
        assert int(torch.count_nonzero(q).item()) == 0


def test_layer_with_and_without_tile_queue():
    cfg = datagen.CONFIGS["dsv3"].replace(T=2048)
    inp = datagen.make_inputs(cfg, seed=0, device=DEV)
    kw = dict(K=cfg.K, score=cfg.score, gather=True)
    a = MoELayerForward(inp, tile_queue=True, **kw)
    b = MoELayerForward(inp, tile_queue=False, **kw)
    outs = []
    for layer in (a, b, a):
        outs.append(layer.forward().clone())
        torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
