"""GPU parity of the grouped SwiGLU expert MLP.

Small shapes are compared in full against the oracle; each case spans
several tiles and ragged tails, including experts with no rows.  Counts are
set directly, so every tile-height variant of the kernel is exercised.
"""
import numpy as np
import pytest
import torch

import combine_router_gating_amd as moe
import oracle
from gpu_helpers import assert_close, f64, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(counts, h, f, dt, seed, extra_rows=0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    E = len(counts)
    N = int(sum(counts))
    rows = N + extra_rows
    x = torch.randn((rows, h), device=DEV, generator=g).to(dt)
    wg = (torch.randn((E, f, h), device=DEV, generator=g) * 0.05).to(dt)
    wu = (torch.randn((E, f, h), device=DEV, generator=g) * 0.05).to(dt)
    wd = (torch.randn((E, h, f), device=DEV, generator=g) * 0.05).to(dt)
    tpe = torch.tensor(counts, dtype=torch.int32, device=DEV)
    return x, wg, wu, wd, tpe, N


CASES = [
    # counts, h, f, dtype
    ([60, 0, 13, 100], 64, 128, torch.bfloat16),
    ([130, 1, 0, 64, 200], 128, 192, torch.bfloat16),
    ([100, 90, 150, 0, 97], 128, 192, torch.bfloat16),  # 128-row tiles (80 <= avg < 128)
    # 256-row tiles of 128 columns in FC2 (128 <= avg < 192): 256-, 128- and 64-row bodies
    ([150, 129, 100, 60, 270, 90], 128, 192, torch.bfloat16),
    ([300, 250], 128, 256, torch.bfloat16),          # 256-row tiles (avg >= 192)
    ([700, 513, 1], 192, 384, torch.bfloat16),       # tallest tiles (avg >= 512)
    ([0, 0, 5], 64, 64, torch.bfloat16),
    ([33, 7, 90], 40, 72, torch.float32),            # fp32 path, odd sizes
    ([256], 128, 256, torch.float32),
    ([70, 0, 129, 64], 200, 136, torch.float32),    # fp32: ragged k-slabs and column tiles
]


@pytest.mark.parametrize("counts,h,f,dt", CASES)
def test_grouped_mlp_matches_oracle(counts, h, f, dt):
    log(f"grouped mlp: counts={counts} h={h} f={f} {dt}")
    x, wg, wu, wd, tpe, N = _case(counts, h, f, dt, seed=sum(counts) + h)
    act, y = moe.moe_grouped_mlp(x, tpe, wg, wu, wd)
    torch.cuda.synchronize()
    dts = "bf16" if dt == torch.bfloat16 else "f32"
    ref_act, ref_y = oracle.grouped_experts(f64(x), np.array(counts), (f64(wg), f64(wu), f64(wd)), dts)
    assert_close(f64(act[:N]), ref_act, dts, "act")
    assert_close(f64(y[:N]), ref_y, dts, "expert_out")


def test_grouped_mlp_rows_beyond_max_rows_are_never_touched():
    """Counts summing past max_rows are clamped; rows past sum(counts) stay untouched."""
    counts = [50, 50, 50]
    x, wg, wu, wd, tpe, N = _case(counts, 64, 128, torch.bfloat16, seed=3, extra_rows=20)
    act = torch.full((N + 20, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    y = torch.full((N + 20, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_fc1_swiglu(x, tpe, wg, wu, act)
    moe.moe_grouped_fc2(act, tpe, wd, y)
    torch.cuda.synchronize()
    assert torch.all(act[N:] == 7.0) and torch.all(y[N:] == 7.0)
    # counts claiming more rows than exist: only the first max_rows rows are written
    big = torch.tensor([100, 100, 100], dtype=torch.int32, device=DEV)
    act2 = moe.moe_grouped_fc1_swiglu(x[:N], big, wg, wu)
    torch.cuda.synchronize()
    assert act2.shape[0] == N


def test_grouped_mlp_all_experts_share_weights():
    """All experts with one weight set: the grouped result equals one dense
    SwiGLU over all rows (computed by the same kernel with E=1)."""
    counts = [17, 0, 90, 33, 1]
    E, h, f = len(counts), 128, 256
    x, wg, wu, wd, tpe, N = _case(counts, h, f, torch.bfloat16, seed=9)
    wg_s, wu_s, wd_s = (w[:1].expand(E, -1, -1).contiguous() for w in (wg, wu, wd))
    _, y = moe.moe_grouped_mlp(x, tpe, wg_s, wu_s, wd_s)
    one = torch.tensor([N], dtype=torch.int32, device=DEV)
    _, y1 = moe.moe_grouped_mlp(x, one, wg[:1].contiguous(), wu[:1].contiguous(), wd[:1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y[:N], y1[:N])


def test_weight_streaming_tiles_over_several_rounds():
    """128-row tiles (80 <= rows per expert < 128), more tiles than the chip
    runs at once, an empty expert; the gathering FC1 reads the same rows
    through sorted_token and must give bitwise the same act."""
    rng = np.random.default_rng(11)
    counts = [int(c) for c in rng.integers(80, 140, size=80)]
    counts[3] = 0
    h, f = 256, 512
    log(f"several rounds of 128-row tiles: E={len(counts)} N={sum(counts)} h={h} f={f}")
    x, wg, wu, wd, tpe, N = _case(counts, h, f, torch.bfloat16, seed=12)
    act, y = moe.moe_grouped_mlp(x, tpe, wg, wu, wd)
    T = N + 9
    perm = torch.randperm(T, device=DEV)[:N].to(torch.int32)
    xt = torch.zeros((T, h), dtype=x.dtype, device=DEV)
    xt[perm.long()] = x[:N]
    a2 = moe.moe_grouped_fc1_swiglu_gather(xt, perm, tpe, wg, wu)
    torch.cuda.synchronize()
    assert torch.equal(act[:N], a2[:N])
    ref_act, ref_y = oracle.grouped_experts(f64(x), np.array(counts), (f64(wg), f64(wu), f64(wd)), "bf16")
    assert_close(f64(act[:N]), ref_act, "bf16", "act")
    assert_close(f64(y[:N]), ref_y, "bf16", "expert_out")


def test_grouped_mlp_many_experts_mostly_empty():
    """700 experts (the tile decode's counts span eleven 64-expert steps),
    most of them empty, a few with rows."""
    counts = [0] * 700
    for e, c in ((0, 5), (63, 70), (64, 1), (250, 130), (511, 3), (699, 40)):
        counts[e] = c
    log(f"many experts: E={len(counts)} N={sum(counts)}")
    x, wg, wu, wd, tpe, N = _case(counts, 64, 128, torch.bfloat16, seed=21)
    act, y = moe.moe_grouped_mlp(x, tpe, wg, wu, wd)
    torch.cuda.synchronize()
    ref_act, ref_y = oracle.grouped_experts(f64(x), np.array(counts), (f64(wg), f64(wu), f64(wd)), "bf16")
    assert_close(f64(act[:N]), ref_act, "bf16", "act")
    assert_close(f64(y[:N]), ref_y, "bf16", "expert_out")
