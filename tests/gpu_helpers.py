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


def assert_close(got, ref, dtype: str, what: str = "") -> None:
    """The layer's tolerance: fp32 |d| <= 1e-4 |ref| + 1e-4 max|ref|;
    bf16 |d| <= 1e-2 + 2e-2 |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return
    d = np.abs(got - ref)
    if dtype == "f32":
        bound = 1e-4 * np.abs(ref) + 1e-4 * np.abs(ref).max()
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
