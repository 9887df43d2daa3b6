"""Shared helpers of the GPU parity tests: tolerances and runners."""
from __future__ import annotations

import sys

import numpy as np
import torch

import datagen
import oracle

f64 = datagen.to_f64


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# fp32 outputs: |d| <= 1e-4 |ref| + FP32_FLOOR max|ref|.  The floor covers
# elements near zero, where a relative bound alone would ask for more than
# fp32 accumulation gives (cancellation); at 1e-6 of the largest element it
# is well below the 1e-4 relative bound of every element larger than 1% of
# the largest.  Outputs of a length-n reduction whose rounding grows with n
# (the gating linear's logits) pass floor=logits_floor(n).
FP32_FLOOR = 1e-6


def logits_floor(n: int) -> float:
    """Absolute floor (as a fraction of max|ref|) for fp32 dot products of
    length n: summing n products in fp32 in some order leaves an error that
    grows like sqrt(n) unit roundoffs of the partial-sum magnitude (bounded
    by max|ref| here); 2^-23 sqrt(n) is that with a factor 2 of margin,
    and never below FP32_FLOOR."""
    return max(FP32_FLOOR, 2.0 ** -23 * float(n) ** 0.5)


def assert_close(got, ref, dtype: str, what: str = "", floor: float = None) -> None:
    """The layer's tolerance: fp32 |d| <= 1e-4 |ref| + floor max|ref|
    (floor = FP32_FLOOR unless given); bf16 |d| <= 1e-2 + 2e-2 |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return
    d = np.abs(got - ref)
    if dtype == "f32":
        fl = FP32_FLOOR if floor is None else floor
        bound = 1e-4 * np.abs(ref) + fl * np.abs(ref).max()
    else:
        bound = 1e-2 + 2e-2 * np.abs(ref)
    bad = d > bound
    if bad.any():
        i = np.unravel_index(np.argmax(d - bound), d.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {d.size} out of tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")


def routing_ref(cfg, logits_np, expert_bias=None):
    """Oracle routing from given fp32 logits."""
    return oracle.route(logits=logits_np, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                        expert_bias=expert_bias, capacity_factor=cfg.capacity_factor,
                        min_capacity=cfg.min_capacity)


def expert_weights_from(inp):
    """Callable e -> float64 (w_gate[e], w_up[e], w_down[e]) copied from the
    device inputs (regenerating nothing, transferring one expert at a time)."""
    def get(e):
        return f64(inp["w_gate"][e]), f64(inp["w_up"][e]), f64(inp["w_down"][e])
    return get


def shared_weights_from(inp):
    if "shared_gate" not in inp:
        return None
    return f64(inp["shared_gate"]), f64(inp["shared_up"]), f64(inp["shared_down"])


def untile(scales):
    """k-tiled MXFP8 scales [G, cols/128, R, 4] (or [cols/128, R, 4]) ->
    row-major [G, R, cols/32] (or [R, cols/32])."""
    s = scales.cpu().numpy() if hasattr(scales, "cpu") else np.asarray(scales)
    s = np.swapaxes(s, -3, -2)
    return s.reshape(s.shape[:-2] + (-1,))


def mx_dequantize_tiled(codes, scales):
    """MXFP8 codes with k-tiled scales, dequantised by the oracle."""
    from oracle import mx
    c = codes.cpu().numpy() if hasattr(codes, "cpu") else np.asarray(codes)
    return mx.mx_dequantize(c, untile(scales))
