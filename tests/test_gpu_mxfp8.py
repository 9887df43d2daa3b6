"""GPU parity of the MXFP8 path (quantisation, FC1 + SwiGLU with fused act
quantisation, FC2) against the oracle's MXFP8 definitions (oracle/mx.py).

Quantisation from bf16/fp32 inputs is bit-exact.  The GEMMs take exact
inputs (the GPU's own codes, whose values the oracle decodes).  The scaled
fp8 MFMA does not accumulate exactly in fp32: its result is within a few
1e-5 of the sum of |products| (measured on the hardware with random
operands), so the bound used here is EPS = 2^-12 times that sum.  FC2's
bf16 output is compared within the bf16 tolerance.  FC1's act codes are a
quantisation of the GPU's act: every dequantised value must be within half
an E4M3 step of the exact act (or its saturation error), plus EPS times the
act's sensitivity to the two dot products; and almost all codes agree.
"""
import numpy as np
import pytest
import torch

import combine_router_gating_amd as moe
from gpu_helpers import assert_close, log, mx_dequantize_tiled as _dq, untile
from oracle import mx

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_bit_exact(dtype):
    rng = np.random.default_rng(0)
    rows, cols = 300, 256
    v = rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((rows, 1)) * 4)
    v[0] = 0.0                                            # all-zero blocks
    v[1, :32] = 448.0 * 2.0 ** -20 * np.arange(32) / 31   # saturation / ties region
    v[2, :32] = 1e-40                                      # subnormal-magnitude block
    v[3, 5] = 1e30
    v[4, :32] = (np.arange(32) - 16) * 2.0 ** -12          # exact values
    # midpoints between E4M3 neighbours at scale 2^-8 (ties to even)
    v[5, :32] = (np.arange(32) + 0.5) * 2.0 ** -9 * 8 * 2 ** -8
    v[5, 31] = 1.0
    t = torch.from_numpy(v).to(dtype).to(DEV)
    codes, scales = moe.moe_mxfp8_quantize(t)
    torch.cuda.synchronize()
    ref_c, ref_s = mx.mx_quantize(t.float().cpu().double().numpy())
    np.testing.assert_array_equal(_np(scales), ref_s)
    np.testing.assert_array_equal(_np(codes), ref_c)


@pytest.mark.parametrize("tile_rows", [1, 8, 96])
def test_quantize_tiled_layout(tile_rows):
    rng = np.random.default_rng(tile_rows)
    rows, cols = 192, 384
    t = torch.from_numpy(rng.standard_normal((rows, cols)) * 3).to(torch.bfloat16).to(DEV)
    c0, s0 = moe.moe_mxfp8_quantize(t)
    c1, s1 = moe.moe_mxfp8_quantize(t, tile_rows=tile_rows)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)
    assert s1.shape == (rows // tile_rows, cols // 128, tile_rows, 4)
    np.testing.assert_array_equal(untile(s1).reshape(rows, cols // 32), _np(s0))


def _weights(rng, E, n, k, std):
    w = torch.from_numpy(rng.standard_normal((E, n, k)) * std).to(torch.bfloat16).to(DEV)
    return moe.moe_mxfp8_quantize_weight(w)


CASES = [  # E, h, f, counts
    (4, 128, 256, [100, 0, 37, 200]),
    (8, 256, 384, [64, 65, 1, 128, 129, 0, 255, 300]),
    (3, 512, 128, [300, 20, 513]),
    (64, 256, 256, [80 + (i * 7) % 60 for i in range(64)]),
]


@pytest.mark.parametrize("E,h,f,counts", CASES)
@pytest.mark.parametrize("gather", [False, True])
def test_fc1_fc2_mxfp8(E, h, f, counts, gather):
    log(f"mxfp8 E={E} h={h} f={f} rows={sum(counts)} gather={gather}")
    rng = np.random.default_rng(E * 31 + h)
    N = sum(counts)
    T = N + 17 if gather else N
    x = torch.from_numpy(rng.standard_normal((T, h))).to(torch.bfloat16).to(DEV)
    xc, xs = moe.moe_mxfp8_quantize(x)
    if gather:
        st = torch.from_numpy(rng.permutation(T)[:N].astype(np.int32)).to(DEV)
    else:
        st = None
    wg = _weights(rng, E, f, h, 0.05)
    wu = _weights(rng, E, f, h, 0.05)
    wd = _weights(rng, E, h, f, 0.05)
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    ac, asc = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, st, cnt, wg, wu, N)
    y = moe.moe_grouped_fc2_mxfp8(ac, asc, cnt, wd)
    torch.cuda.synchronize()
    xq = mx.mx_dequantize(_np(xc), _np(xs))
    rows = _np(st) if gather else np.arange(N)
    xq = xq[rows]
    wgq, wuq, wdq = (_dq(c, s) for c, s in (wg, wu, wd))
    off = np.concatenate([[0], np.cumsum(counts)])
    act_exact = np.zeros((N, f))
    sens = np.zeros((N, f))  # |d act| per unit of |dg| = EPS * sum|x wg| (and likewise for u)
    for e in range(E):
        r = slice(off[e], off[e + 1])
        g = xq[r] @ wgq[e].T
        u = xq[r] @ wuq[e].T
        sg = 1 / (1 + np.exp(-g))
        act_exact[r] = g * sg * u
        ga = np.abs(xq[r]) @ np.abs(wgq[e]).T
        ua = np.abs(xq[r]) @ np.abs(wuq[e]).T
        sens[r] = 1.1 * np.abs(u) * ga + np.abs(g * sg) * ua
    # FC1: the GPU's block scales are the oracle's except where the block's
    # largest |act| is within fp32 accumulation error of a power of two ...
    ref_c, ref_s = mx.mx_quantize(act_exact)
    got_c, got_s = _np(ac)[:N], untile(asc)[:N]
    amax = np.abs(act_exact).reshape(N, f // 32, 32).max(-1)
    near_pow2 = np.abs(amax / np.ldexp(1.0, np.round(np.log2(np.maximum(amax, 1e-300))).astype(int)) - 1) < 1e-4
    bad_s = (got_s != ref_s) & ~near_pow2
    assert not bad_s.any(), (np.argwhere(bad_s)[:5], got_s[bad_s][:5], ref_s[bad_s][:5])
    # ... and every dequantised value is the exact act rounded to E4M3 under
    # its block scale, up to the MFMA's accumulation error
    EPS = 2.0 ** -12
    X = np.repeat(np.ldexp(1.0, got_s.astype(int) - 127), 32, axis=1)
    dq = mx.e4m3_value(got_c) * X
    a = np.abs(act_exact) / X
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(a, 2.0 ** -6))).astype(int) - 3) * X
    rounding = np.where(a > 448, np.abs(act_exact) - 448 * X, 0.5 * step)
    bound = rounding + EPS * sens + step * 1e-9
    bad = np.abs(dq - act_exact) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5], dq[bad][:5], act_exact[bad][:5],
                           bound[bad][:5])
    assert (got_c == mx.mx_quantize(act_exact)[0]).mean() > 0.99
    # FC2 on the GPU's act codes: exact inputs, bf16 output
    y_ref = np.zeros((N, h))
    for e in range(E):
        r = slice(off[e], off[e + 1])
        y_ref[r] = dq[r] @ wdq[e].T
    assert_close(_np(y[:N].float()), y_ref, "bf16", "y")


def test_mxfp8_rejects_bad_sizes():
    p = None
    lib = moe.load()
    import ctypes
    q = ctypes.c_void_p(16)
    assert lib.moe_mxfp8_quantize(4, 48, 0, 1, q, q, q, p) == 2       # cols % 32
    assert lib.moe_mxfp8_quantize(4, 96, 2, 1, q, q, q, p) == 2       # tiled: cols % 128
    assert lib.moe_mxfp8_quantize(6, 128, 4, 1, q, q, q, p) == 2      # tiled: rows % R
    assert lib.moe_grouped_fc2_mxfp8(4, 192, 256, 8, q, q, q, q, q, q, None, p) == 2  # h % 128


@pytest.mark.parametrize("overlap,fold", [(False, True), (True, False), (False, False)])
def test_layer_mxfp8_against_the_oracle(overlap, fold):
    import datagen
    import oracle
    from combine_router_gating_amd.layer import MoELayerForward
    from gpu_helpers import f64
    cfg = datagen.MoEConfig("mx-layer", T=300, h=256, E=16, K=2, f=384, dtype="bf16", score="sigmoid",
                            expert_bias=True, shared_f=256, capacity_factor=0.8)
    log(f"mxfp8 layer overlap={overlap} fold={fold}: {cfg}")
    inp = datagen.make_inputs(cfg, seed=3, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, score=cfg.score, capacity_factor=cfg.capacity_factor,
                            overlap_shared=overlap, precision="mxfp8", fold_shared=fold)
    assert layer.fold_shared == fold and layer.overlap_shared == overlap
    out = layer.forward().clone()
    torch.cuda.synchronize()
    # routing is the bf16 layer's (same router kernels)
    ref_r = oracle.route(logits=layer.logits.cpu().numpy(), K=cfg.K, score=cfg.score,
                         expert_bias=inp["expert_bias"].cpu().numpy(),
                         capacity_factor=cfg.capacity_factor)
    np.testing.assert_array_equal(_np(layer.routing_map), ref_r["routing_map"])
    # x quantisation: bit-exact
    xc, xs = mx.mx_quantize(f64(inp["x"]))
    np.testing.assert_array_equal(_np(layer.xq[0]), xc)
    np.testing.assert_array_equal(_np(layer.xq[1]), xs)
    # expert outputs from the GPU's act codes (exact inputs) and the combine
    pm = oracle.permute(f64(inp["x"]), ref_r["routing_map"], ref_r["probs"], cfg.K)
    N = int(pm["expert_offsets"][-1])
    act = mx.mx_dequantize(_np(layer.actq[0])[:N], untile(layer.actq[1])[:N])
    wd = _dq(*layer.wq["w_down"])
    n = pm["tokens_per_expert"]
    off = np.concatenate([[0], np.cumsum(n)])
    y = np.zeros((N, cfg.h))
    for e in range(cfg.E):
        y[off[e]:off[e + 1]] = act[off[e]:off[e + 1]] @ wd[e].T
    y = oracle.round_bf16(y)
    sact = _dq(*layer.shared_actq)
    swd = _dq(*layer.wq["shared_down"])[0]
    shared = oracle.round_bf16(sact @ swd.T)
    ref_out = oracle.combine(y, pm["permuted_probs"], pm["row_id_map"], "bf16", shared)
    assert_close(f64(out), ref_out, "bf16", "out")
    # the same forward with the shared expert in launches of its own on one
    # stream gives the same bits
    plain = MoELayerForward(inp, K=cfg.K, score=cfg.score, capacity_factor=cfg.capacity_factor,
                            precision="mxfp8", fold_shared=False)
    o2 = plain.forward()
    torch.cuda.synchronize()
    assert torch.equal(out, o2)


@pytest.mark.parametrize("fold", [False, True])
def test_layer_mxfp8_graph_capture_replays(fold):
    """The MXFP8 forward (x quantisation, router, permute, MXFP8 GEMMs, the
    shared expert on a second stream or folded into the routed launches,
    combine) captures into a graph; replays on new inputs equal the eager
    forward bit for bit."""
    import datagen
    from combine_router_gating_amd.layer import MoELayerForward
    cfg = datagen.MoEConfig("mx-graph", T=512, h=256, E=16, K=2, f=256, dtype="bf16", shared_f=128)
    inp = datagen.make_inputs(cfg, seed=5, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, overlap_shared=not fold, precision="mxfp8",
                            fold_shared=fold)
    layer.forward()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward()
    plain = MoELayerForward(inp, K=cfg.K, precision="mxfp8", fold_shared=False)
    for seed in (6, 7, 8):
        new = datagen.make_inputs(cfg, seed=seed, device=DEV, with_experts=False)
        inp["x"].copy_(new["x"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = plain.forward()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay with seed {seed}"


def test_mxfp8_gemm_edge_cases():
    """One row in one expert of three, the smallest sizes (h = f = 128), and
    nothing to do (max_rows = 0) all behave."""
    rng = np.random.default_rng(11)
    E, h, f = 3, 128, 128
    counts = [0, 1, 0]
    x = torch.from_numpy(rng.standard_normal((1, h))).to(torch.bfloat16).to(DEV)
    xc, xs = moe.moe_mxfp8_quantize(x)
    wg, wu, wd = (_weights(rng, E, n, k, 0.1) for n, k in ((f, h), (f, h), (h, f)))
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    ac, asc = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, None, cnt, wg, wu, 1)
    y = moe.moe_grouped_fc2_mxfp8(ac, asc, cnt, wd)
    torch.cuda.synchronize()
    xq = mx.mx_dequantize(_np(xc), _np(xs))
    g, u = xq @ _dq(*wg)[1].T, xq @ _dq(*wu)[1].T
    act = mx.mx_dequantize(_np(ac), untile(asc))
    exact = g / (1 + np.exp(-g)) * u
    assert np.abs(act - exact).max() <= 0.07 * np.abs(exact).max() + 1e-6
    assert_close(_np(y.float()), act @ _dq(*wd)[1].T, "bf16", "y")
    import ctypes
    lib = moe.load()
    q = ctypes.c_void_p(16)
    assert lib.moe_grouped_fc1_swiglu_mxfp8(E, h, f, 0, 1, q, q, None, q, q, q, q, q, q, q, None,
                                            None) == 0
    assert lib.moe_grouped_fc2_mxfp8(E, h, f, 0, q, q, q, q, q, q, None, None) == 0


def test_mxfp8_gemm_counts_past_max_rows_stay_in_bounds():
    """tokens_per_expert claiming more rows than max_rows: the GEMMs clamp to
    max_rows and write nothing past it (checked with guard rows)."""
    rng = np.random.default_rng(12)
    E, h, f, R = 4, 128, 256, 200
    x = torch.from_numpy(rng.standard_normal((R, h))).to(torch.bfloat16).to(DEV)
    xc, xs = moe.moe_mxfp8_quantize(x)
    wg, wu, wd = (_weights(rng, E, n, k, 0.05) for n, k in ((f, h), (f, h), (h, f)))
    cnt = torch.tensor([100, 90, 80, 70], dtype=torch.int32, device=DEV)  # 340 > R
    guard = 64
    act_c = torch.full((R + guard, f), 0x5a, dtype=torch.uint8, device=DEV)
    act_s = torch.full((f // 128, R, 4), 0x5a, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, None, cnt, wg, wu, R, act=(act_c[:R], act_s))
    y = torch.full((R + guard, h), 7.0, dtype=torch.bfloat16, device=DEV)
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = moe.load().moe_grouped_fc2_mxfp8(E, h, f, R, p(act_c), p(act_s), p(cnt), p(wd[0]), p(wd[1]),
                                         p(y), None,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert (act_c[R:] == 0x5a).all()
    assert (y[R:] == 7.0).all()
    assert torch.isfinite(y[:R].float()).all()


FC2_COMBINE_CASES = [
    # T, h, f, E, capacity_factor, hot: the three FC2 bodies (avg rows < 80, < 192, >= 192)
    (515, 128, 256, 16, 1.0, 2.0),     # drops, ~33 rows per expert
    (2000, 256, 128, 16, 1.25, 1.0),   # ~157 rows per expert
    (3000, 128, 256, 8, 0.0, 0.0),     # dropless, 375 rows per expert
    (1, 128, 128, 4, 0.0, 0.0),
    (40, 128, 128, 4, 0.05, 3.0),      # most tokens dropped
]


@pytest.mark.parametrize("T,h,f,E,cf,hot", FC2_COMBINE_CASES)
def test_fc2_combine_mxfp8_is_bitwise_fc2_then_combine(T, h, f, E, cf, hot):
    """The top-1 combine fused into the MXFP8 FC2 writes the bits of
    moe_grouped_fc2_mxfp8 followed by moe_combine (K = 1), dropped tokens'
    rows included; twice in a row into the same buffer."""
    log(f"mxfp8 fc2+combine: T={T} h={h} f={f} E={E} cf={cf}")
    rng = np.random.default_rng(T + h + E)
    x = torch.from_numpy(rng.standard_normal((T, h))).to(torch.bfloat16).to(DEV)
    w = torch.from_numpy(rng.standard_normal((E, h)) / h ** 0.5).float().to(DEV)
    w[0] += hot / h ** 0.5
    wg, wu, wd = (_weights(rng, E, n, k, 0.05) for n, k in ((f, h), (f, h), (h, f)))
    r = moe.moe_route_permute(x, w, K=1, capacity_factor=cf, copy_rows=False)
    tpe, st = r["tokens_per_expert"], r["sorted_token"]
    R = st.shape[0]
    xc, xs = moe.moe_mxfp8_quantize(x)
    ac, asc = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, st, tpe, wg, wu, R)
    y = moe.moe_grouped_fc2_mxfp8(ac, asc, tpe, wd)
    ref = moe.moe_combine(y, r["permuted_probs"], r["row_id_map"])
    out = torch.full((T, h), float("nan"), dtype=torch.bfloat16, device=DEV)
    for _ in range(2):
        moe.moe_grouped_fc2_combine_mxfp8(ac, asc, tpe, wd, r["permuted_probs"], st,
                                          r["row_id_map"], out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        out.fill_(float("nan"))


def test_fc2_combine_mxfp8_on_an_empty_batch_and_no_rows():
    """T = 0 is a no-op; max_rows = 0 (every token dropped) writes zero rows."""
    E, h, f = 4, 128, 128
    rng = np.random.default_rng(5)
    wd = _weights(rng, E, h, f, 0.05)
    cnt = torch.zeros((E,), dtype=torch.int32, device=DEV)
    import ctypes
    lib = moe.load()
    q = ctypes.c_void_p(16)
    assert lib.moe_grouped_fc2_combine_mxfp8(E, h, f, 0, 0, None, None, None, None, None, None,
                                             None, None, None, None) == 0
    T = 70
    rid = torch.full((T,), -1, dtype=torch.int32, device=DEV)
    out = torch.full((T, h), 3.0, dtype=torch.bfloat16, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.moe_grouped_fc2_combine_mxfp8(E, h, f, 0, T, None, None, p(cnt), p(wd[0]), p(wd[1]),
                                           None, None, p(rid), p(out),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert (out == 0).all()
    assert lib.moe_grouped_fc2_combine_mxfp8(E, 192, f, 8, T, q, q, q, q, q, q, q, q, q, None) == 2


def _act_bound(act_exact, sens, scale_bytes):
    """Allowed |dq(act) - act_exact|: half an E4M3 step under the block scale
    (or the saturation error) plus the MFMA accumulation bound."""
    EPS = 2.0 ** -12
    X = np.repeat(np.ldexp(1.0, scale_bytes.astype(int) - 127), 32, axis=-1)
    a = np.abs(act_exact) / X
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(a, 2.0 ** -6))).astype(int) - 3) * X
    rounding = np.where(a > 448, np.abs(act_exact) - 448 * X, 0.5 * step)
    return rounding + EPS * sens + step * 1e-9


@pytest.mark.parametrize("name,n_tok", [("switch", 6), ("dsv3", 2)])
def test_layer_mxfp8_full_size_sampled(name, n_tok):
    """The MXFP8 layer at full size, in the configuration the bench times
    (gathering FC1, overlapped shared expert): routing bit-exact on the
    GPU's logits; x quantisation bit-exact; sampled act rows within the
    accumulation bound of the exact SwiGLU of the GPU's MXFP8 operands;
    those rows' expert outputs and sampled tokens' outputs within the bf16
    tolerance of the oracle run on the GPU's act codes."""
    import datagen
    import oracle
    from combine_router_gating_amd.layer import MoELayerForward
    from gpu_helpers import f64, routing_ref
    cfg = datagen.CONFIGS[name]
    log(f"mxfp8 layer full size: {cfg}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                            capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity,
                            gather=True, overlap_shared=True, precision="mxfp8")
    out = layer.forward()
    torch.cuda.synchronize()
    eb = inp["expert_bias"].cpu().numpy() if "expert_bias" in inp else None
    ref = routing_ref(cfg, layer.logits.cpu().numpy(), eb)
    np.testing.assert_array_equal(_np(layer.routing_map), ref["routing_map"])
    xc, xs = mx.mx_quantize(f64(inp["x"]))
    np.testing.assert_array_equal(_np(layer.xq[0]), xc)
    np.testing.assert_array_equal(_np(layer.xq[1]), xs)
    xq = mx.mx_dequantize(xc, xs)
    pm = oracle.permute(np.zeros((cfg.T, 1)), ref["routing_map"], ref["probs"], cfg.K)
    n = pm["tokens_per_expert"]
    offs = np.concatenate([[0], np.cumsum(n)])
    np.testing.assert_array_equal(_np(layer.sorted_token)[:offs[-1]], pm["sorted_token"])
    act_c, act_s = _np(layer.actq[0]), untile(layer.actq[1])
    wq = {k: layer.wq[k] for k in ("w_gate", "w_up", "w_down")}

    def expert_w(e, keys=("w_gate", "w_up", "w_down")):
        return [mx.mx_dequantize(_np(wq[k][0][e]), untile(wq[k][1][e][None])[0]) for k in keys]

    def gpu_rows(t, rows):
        return f64(t[torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(DEV)])

    def y_rows(rows, e, wd):
        return oracle.round_bf16(mx.mx_dequantize(act_c[rows], act_s[rows]) @ wd.T)

    rng = np.random.default_rng(1)
    for e in sorted({int(np.argmax(n)), int(np.nonzero(n)[0][-1])}):
        rows = rng.choice(np.arange(offs[e], offs[e + 1]), size=min(4, int(n[e])), replace=False)
        wg, wu, wd = expert_w(e)
        xr = xq[pm["sorted_token"][rows]]
        g, u = xr @ wg.T, xr @ wu.T
        sg = 1 / (1 + np.exp(-g))
        exact = g * sg * u
        sens = 1.1 * np.abs(u) * (np.abs(xr) @ np.abs(wg).T) + np.abs(g * sg) * (np.abs(xr) @ np.abs(wu).T)
        dq = mx.mx_dequantize(act_c[rows], act_s[rows])
        bad = np.abs(dq - exact) > _act_bound(exact, sens, act_s[rows])
        assert not bad.any(), (name, e, int(bad.sum()))
        if not layer.fused_combine:  # (the fused FC2 writes no expert_out)
            assert_close(gpu_rows(layer.expert_out, rows), y_rows(rows, e, wd), "bf16",
                         f"expert_out[{name}, e={e}]")
    # sampled tokens: combine of the oracle's expert outputs (from the GPU's act codes)
    toks = rng.choice(cfg.T, size=n_tok, replace=False)
    shared = None
    if "shared_gate" in inp:
        swd = mx.mx_dequantize(_np(layer.wq["shared_down"][0][0]), untile(layer.wq["shared_down"][1])[0])
        sact = mx.mx_dequantize(_np(layer.shared_actq[0])[toks], untile(layer.shared_actq[1])[toks])
        shared = oracle.round_bf16(sact @ swd.T)
    for i, t in enumerate(toks):
        acc = np.zeros(cfg.h)
        for k in range(cfg.K):
            r = int(pm["row_id_map"][t, k])
            if r < 0:
                continue
            e = int(np.searchsorted(offs, r, side="right") - 1)
            acc += pm["permuted_probs"][r] * y_rows(np.array([r]), e, expert_w(e, ("w_down",))[0])[0]
        if shared is not None:
            acc += shared[i]
        assert_close(gpu_rows(out, [t]), oracle.round_bf16(acc)[None], "bf16", f"out[{name}, t={t}]")
    if layer.fused_combine:
        # the fused FC2 + combine gives the bits of the two calls
        out = out.clone()
        plain = MoELayerForward(inp, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                                capacity_factor=cfg.capacity_factor,
                                min_capacity=cfg.min_capacity, gather=True, overlap_shared=True,
                                precision="mxfp8", fuse_combine=False)
        o2 = plain.forward()
        torch.cuda.synchronize()
        assert torch.equal(out, o2)


# (h, f): FC1 runs k = h in stages of 128 over N = f, FC2 k = f over N = h; the
# split-ring queue bodies need N a multiple of 128 (FC1) / 256 (FC2), else the
# plain queue body runs: (256, 384) splits both with 2 and 3 stages, (128, 256)
# splits FC1 with 1 stage and FC2 falls back, (512, 128) splits FC1 with 4
# stages and FC2 with 1
@pytest.mark.parametrize("h,f,fs", [(256, 384, 0), (256, 384, 256), (128, 256, 0), (128, 256, 128),
                                    (512, 128, 0), (512, 128, 256)])
def test_mxfp8_tile_queue_and_folded_shared_expert_match_plain_launches(h, f, fs):
    """The MXFP8 GEMMs with a tile queue (experts of >= 192 rows on average)
    give the bits of one workgroup per tile, and with the shared expert's
    tiles folded into the routed launches the shared act and output are the
    bits of separate E = 1 launches; on repeated calls with one queue, which
    is zero again afterwards."""
    import datagen
    cfg = datagen.MoEConfig("mx-queue", T=2048, h=h, E=16, K=2, f=f, dtype="bf16",
                            score="sigmoid", expert_bias=True, shared_f=fs)
    log(f"mxfp8 tile queue / fold: {cfg}")
    inp = datagen.make_inputs(cfg, seed=21, device=DEV)
    r = moe.moe_route_permute(inp["x"], inp["w_router"], K=cfg.K, score="sigmoid",
                              expert_bias=inp["expert_bias"], copy_rows=False)
    st, tpe = r["sorted_token"], r["tokens_per_expert"]
    rows = st.shape[0]
    N = int(r["expert_offsets"][-1].item())
    assert rows // cfg.E >= 192  # the queue is used
    xc, xs = moe.moe_mxfp8_quantize(inp["x"])
    wg, wu, wd = (moe.moe_mxfp8_quantize_weight(inp[k]) for k in ("w_gate", "w_up", "w_down"))
    q = moe.gemm_queue(DEV)
    if fs:
        sg, su, sd = (moe.moe_mxfp8_quantize_weight(inp[k][None])
                      for k in ("shared_gate", "shared_up", "shared_down"))
        allrows = torch.tensor([cfg.T], dtype=torch.int32, device=DEV)
    for _ in range(3):
        a0 = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, st, tpe, wg, wu, rows)
        a1 = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, st, tpe, wg, wu, rows, queue=q)
        y0 = moe.moe_grouped_fc2_mxfp8(a0[0], a0[1], tpe, wd)
        y1 = moe.moe_grouped_fc2_mxfp8(a1[0], a1[1], tpe, wd, queue=q)
        torch.cuda.synchronize()
        assert torch.equal(a0[0][:N], a1[0][:N]) and torch.equal(a0[1][:, :N], a1[1][:, :N])
        assert torch.equal(y0[:N], y1[:N])
        if fs:
            s0 = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, None, allrows, sg, su, cfg.T)
            o0 = moe.moe_grouped_fc2_mxfp8(s0[0], s0[1], allrows, sd)
            for queue in (None, q):
                a2, s2 = moe.moe_grouped_fc1_swiglu_mxfp8_shared(xc, xs, st, tpe, wg, wu, rows, sg,
                                                                 su, queue=queue)
                y2, o2 = moe.moe_grouped_fc2_mxfp8_shared(a2[0], a2[1], tpe, wd, s2, sd,
                                                          queue=queue)
                torch.cuda.synchronize()
                assert torch.equal(a2[0][:N], a0[0][:N]) and torch.equal(a2[1][:, :N], a0[1][:, :N])
                assert torch.equal(y2[:N], y0[:N])
                assert torch.equal(s2[0], s0[0]) and torch.equal(s2[1], s0[1])
                assert torch.equal(o2, o0)
        assert int(torch.count_nonzero(q).item()) == 0


@pytest.mark.parametrize("counts", [[0] * 8, [4096] + [0] * 7, [1] + [0] * 6 + [4095],
                                    [3000, 3000] + [0] * 6])
def test_mxfp8_tile_queue_degenerate_counts(counts):
    """MXFP8 queue launches (max_rows / E = 512) over degenerate counts (all
    empty, one expert, one row against the rest, counts past max_rows) give
    the bits of one workgroup per tile and leave the counters zeroed."""
    rng = np.random.default_rng(4)
    E, h, f, rows = 8, 256, 512, 4096
    x = torch.from_numpy(rng.standard_normal((rows, h))).to(torch.bfloat16).to(DEV)
    xc, xs = moe.moe_mxfp8_quantize(x)
    wg, wu = _weights(rng, E, f, h, h ** -0.5), _weights(rng, E, f, h, h ** -0.5)
    wd = _weights(rng, E, h, f, f ** -0.5)
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    N = min(sum(counts), rows)
    log(f"mxfp8 tile queue, degenerate counts {counts}")
    q = moe.gemm_queue(DEV)
    for _ in range(2):
        a0 = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, None, cnt, wg, wu, rows)
        a1 = moe.moe_grouped_fc1_swiglu_mxfp8(xc, xs, None, cnt, wg, wu, rows, queue=q)
        y0 = moe.moe_grouped_fc2_mxfp8(a0[0], a0[1], cnt, wd)
        y1 = moe.moe_grouped_fc2_mxfp8(a0[0], a0[1], cnt, wd, queue=q)
        torch.cuda.synchronize()
        assert torch.equal(a0[0][:N], a1[0][:N]) and torch.equal(a0[1][:, :N], a1[1][:, :N])
        assert torch.equal(y0[:N], y1[:N])
        assert int(torch.count_nonzero(q).item()) == 0


@pytest.mark.parametrize("name", ["dsv3", "mixtral", "qwen3"])
def test_mxfp8_bench_layer_whole_experts(name):
    """The MXFP8 layer at full size in the benchmark's launch configuration
    (gathering FC1, tile queue, shared expert folded into the routed
    launches): every row and column of act and expert_out for the busiest
    expert, for one whose last 128-row m-tile is ragged and (DeepSeek-V3-
    shaped) for the smallest; the folded shared expert on a whole 128-row
    m-tile; and 256 tokens of the output as the combine of the checked
    expert and shared outputs.  act within the accumulation bound of the
    exact SwiGLU of the GPU's MXFP8 operands, expert_out and out within the
    bf16 tolerance of the oracle run on the GPU's act codes."""
    import datagen
    import oracle
    from combine_router_gating_amd.layer import MoELayerForward
    from gpu_helpers import f64, routing_ref
    cfg = datagen.CONFIGS[name]
    log(f"mxfp8 full-size whole experts: {cfg}")
    inp = datagen.make_inputs(cfg, seed=0, device=DEV)
    layer = MoELayerForward(inp, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                            capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity,
                            gather=True, precision="mxfp8")
    assert layer.fold_shared == ("shared_gate" in inp) and layer.queue is not None
    out = layer.forward()
    torch.cuda.synchronize()
    eb = inp["expert_bias"].cpu().numpy() if "expert_bias" in inp else None
    ref = routing_ref(cfg, layer.logits.cpu().numpy(), eb)
    np.testing.assert_array_equal(_np(layer.routing_map), ref["routing_map"])
    xc, xs = mx.mx_quantize(f64(inp["x"]))
    np.testing.assert_array_equal(_np(layer.xq[0]), xc)
    np.testing.assert_array_equal(_np(layer.xq[1]), xs)
    xq = mx.mx_dequantize(xc, xs)
    pm = oracle.permute(np.zeros((cfg.T, 1)), ref["routing_map"], ref["probs"], cfg.K)
    n = pm["tokens_per_expert"]
    offs = np.concatenate([[0], np.cumsum(n)])
    st = pm["sorted_token"]
    np.testing.assert_array_equal(_np(layer.sorted_token)[:offs[-1]], st)
    act_s_all = layer.actq[1]

    def check_rows(xr, wg, wu, wd, act_c, act_s, y_gpu, what):
        g, u = xr @ wg.T, xr @ wu.T
        sg = 1 / (1 + np.exp(-g))
        exact = g * sg * u
        sens = 1.1 * np.abs(u) * (np.abs(xr) @ np.abs(wg).T) + \
            np.abs(g * sg) * (np.abs(xr) @ np.abs(wu).T)
        dq = mx.mx_dequantize(act_c, act_s)
        bad = np.abs(dq - exact) > _act_bound(exact, sens, act_s)
        assert not bad.any(), (what, int(bad.sum()))
        assert_close(y_gpu, oracle.round_bf16(dq @ wd.T), "bf16", what)

    def expert_w(key, e):
        c, s = layer.wq[key]
        return mx.mx_dequantize(_np(c[e]), untile(s[e][None])[0])

    busiest = int(np.argmax(n))
    ragged = [int(e) for e in np.argsort(-n) if n[e] > 128 and n[e] % 128 and e != busiest]
    experts = [busiest] + ragged[:1]
    nz = np.nonzero(n)[0]
    smallest = int(nz[np.argmin(n[nz])])
    if n[smallest] < 64 and smallest not in experts:
        experts.append(smallest)
    act_rows_c = layer.actq[0]
    for e in experts:
        rows = np.arange(offs[e], offs[e + 1])
        log(f"  expert {e}: {len(rows)} rows")
        idx = torch.from_numpy(rows).to(DEV)
        act_c = _np(act_rows_c[idx])
        act_s = untile(act_s_all[:, idx])
        check_rows(xq[st[rows]], expert_w("w_gate", e), expert_w("w_up", e),
                   expert_w("w_down", e), act_c, act_s, f64(layer.expert_out[idx]),
                   f"{name} expert {e}")
    if layer.shared:
        t0 = 1024
        tok = np.arange(t0, t0 + 128)
        sact_s = untile(layer.shared_actq[1][:, t0:t0 + 128])
        check_rows(xq[tok], expert_w("shared_gate", 0), expert_w("shared_up", 0),
                   expert_w("shared_down", 0), _np(layer.shared_actq[0][t0:t0 + 128]), sact_s,
                   f64(layer.shared_out[t0:t0 + 128]), f"{name} shared expert")
    # 256 tokens: combine of the GPU's expert rows (and shared rows), in the oracle's order
    toks = np.sort(np.random.default_rng(7).choice(cfg.T, size=256, replace=False))
    rid = pm["row_id_map"][toks]
    rows_needed = np.unique(rid[rid >= 0])
    y = np.zeros((int(offs[-1]), cfg.h))
    y[rows_needed] = f64(layer.expert_out[torch.from_numpy(rows_needed).to(DEV)])
    shared = f64(layer.shared_out)[toks] if layer.shared else None
    sub_rid = np.where(rid >= 0, rid, -1)
    exp = oracle.combine(y, pm["permuted_probs"], sub_rid, "bf16", shared)
    assert_close(f64(out)[toks], exp, "bf16", f"out[{name}, 256 tokens]")
