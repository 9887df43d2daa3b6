"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random numbers and stores them in the dtypes a
workload asks for.  It holds none of the layer's arithmetic (no routing,
no softmax, no matmul), so both the CPU oracle and the GPU path can take
their inputs from here without sharing any computation.

Workloads (the five layer shapes and their value distributions):

  tiny     T=256  h=128  E=8   K=2 f=256   fp32 everywhere, softmax top-2
  switch   T=8192 h=2048 E=64  K=1 f=4096  bf16, fp32 router, capacity 1.25,
           Zipf(s=1.1) per-expert gate bias with maximum 2.0
  mixtral  T=4096 h=4096 E=8   K=2 f=14336 bf16, fp32 router, softmax top-2
  qwen3    T=8192 h=4096 E=128 K=8 f=1536  bf16, fp32 router, softmax top-8
           with the top-k probabilities renormalised
  dsv3     T=8192 h=7168 E=256 K=8 f=2048  bf16, fp32 router, sigmoid top-8
           with a selection-only expert bias ~U(-0.1, 0.1), plus one shared
           expert with ffn 2048

Value recipe: hidden ~ N(0, 1); gate weight ~ N(0, 1/h) (variance 1/h, so
logits are ~N(0, 1)); expert and shared weights ~ N(0, 0.02^2) (std 0.02).
bf16 tensors are drawn in fp32 and rounded to nearest-even.

Every tensor has its own seed derived from (seed, tensor name), so a tensor
can be regenerated alone.  Random draws use torch generators on the device
the tensors are made for; the same seed gives the same values on the same
device type.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Shape and routing options of one MoE layer forward."""

    name: str
    T: int            # tokens (sequence x batch, flattened)
    h: int            # hidden size
    E: int            # routed experts
    K: int            # experts per token (top-k)
    f: int            # expert ffn size
    dtype: str        # "f32" or "bf16": hidden, expert weights, outputs
    score: str = "softmax"        # "softmax" or "sigmoid"
    pre_softmax: bool = True      # softmax over E then top-k; False: renormalise over the k
    capacity_factor: float = 0.0  # <= 0: dropless
    min_capacity: int = 0
    gate_bias: Optional[str] = None   # "zipf": per-expert logit bias of the gating linear
    expert_bias: bool = False         # selection-only bias (sigmoid scoring)
    shared_f: int = 0                 # ffn size of the shared expert (0: none)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", T=256, h=128, E=8, K=2, f=256, dtype="f32"),
    "switch": MoEConfig("switch", T=8192, h=2048, E=64, K=1, f=4096, dtype="bf16",
                        capacity_factor=1.25, gate_bias="zipf"),
    "mixtral": MoEConfig("mixtral", T=4096, h=4096, E=8, K=2, f=14336, dtype="bf16"),
    "qwen3": MoEConfig("qwen3", T=8192, h=4096, E=128, K=8, f=1536, dtype="bf16",
                       pre_softmax=False),
    "dsv3": MoEConfig("dsv3", T=8192, h=7168, E=256, K=8, f=2048, dtype="bf16",
                      score="sigmoid", expert_bias=True, shared_f=2048),
}

EXPERT_STD = 0.02
ZIPF_S = 1.1
ZIPF_MAX = 2.0
EXPERT_BIAS_RANGE = 0.1


def tensor_seed(seed: int, name: str) -> int:
    """A 63-bit seed for one named tensor, stable across processes."""
    digest = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    return int.from_bytes(digest[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, name))
    return g


def _normal(shape, std, dtype, seed, name, device) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(seed, name, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)  # fp32 -> bf16 conversion rounds to nearest-even


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu",
                with_experts: bool = True) -> Dict[str, torch.Tensor]:
    """All inputs of one layer forward, on ``device``.

    Keys: x [T,h]; w_router [E,h] fp32; b_router [E] fp32 or absent;
    expert_bias [E] fp32 or absent; w_gate, w_up [E,f,h]; w_down [E,h,f];
    shared_gate, shared_up [shared_f,h]; shared_down [h,shared_f] when the
    layer has a shared expert.  Expert tensors are skipped when
    ``with_experts`` is False (routing-only tests).
    """
    dt = cfg.torch_dtype
    out: Dict[str, torch.Tensor] = {}
    out["x"] = _normal((cfg.T, cfg.h), 1.0, dt, seed, "x", device)
    out["w_router"] = _normal((cfg.E, cfg.h), cfg.h ** -0.5, torch.float32, seed,
                              "w_router", device)
    if cfg.gate_bias == "zipf":
        perm = torch.randperm(cfg.E, generator=_gen(seed, "b_router", "cpu"))
        rank = perm.to(torch.float64) + 1.0
        out["b_router"] = (ZIPF_MAX * rank.pow(-ZIPF_S)).to(torch.float32).to(device)
    if cfg.expert_bias:
        u = torch.rand((cfg.E,), generator=_gen(seed, "expert_bias", device),
                       device=device, dtype=torch.float32)
        out["expert_bias"] = (u * 2.0 - 1.0) * EXPERT_BIAS_RANGE
    if with_experts:
        out["w_gate"] = _normal((cfg.E, cfg.f, cfg.h), EXPERT_STD, dt, seed, "w_gate", device)
        out["w_up"] = _normal((cfg.E, cfg.f, cfg.h), EXPERT_STD, dt, seed, "w_up", device)
        out["w_down"] = _normal((cfg.E, cfg.h, cfg.f), EXPERT_STD, dt, seed, "w_down", device)
        if cfg.shared_f:
            fs = cfg.shared_f
            out["shared_gate"] = _normal((fs, cfg.h), EXPERT_STD, dt, seed, "shared_gate", device)
            out["shared_up"] = _normal((fs, cfg.h), EXPERT_STD, dt, seed, "shared_up", device)
            out["shared_down"] = _normal((cfg.h, fs), EXPERT_STD, dt, seed, "shared_down", device)
    return out


def to_f64(t: torch.Tensor):
    """A tensor as a float64 numpy array (exact for bf16 and fp32 values)."""
    return t.detach().to("cpu", torch.float64).numpy()
