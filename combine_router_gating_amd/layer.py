"""A preallocated MoE layer forward: buffers are allocated once (torch), the
C arguments are built once, and each forward is a fixed sequence of libmoe
calls on the current stream — no allocation and no host sync per call, so
it can also be captured into a graph.

Options: `gather` skips the permuted copy of x (the permute writes indices
and probs only, and FC1 reads token rows through sorted_token);
`overlap_shared` runs the shared expert on a second stream (default
priority) from the start of the forward, joined before the combine;
`fuse_combine` (on by default; top-1 bf16 layers without a shared expert)
runs FC2 with the combine as its epilogue (moe_grouped_fc2_combine, or
moe_grouped_fc2_combine_mxfp8 for MXFP8 experts; one "fc2_combine" stage):
no expert_out round trip, bitwise the same output.
`fold_shared` (on by default; layers with a shared expert and the
gathering FC1) runs the shared expert's FC1 and FC2 as the last tiles of
the routed experts' FC1 and FC2 launches (moe_grouped_fc1_swiglu_gather_shared,
moe_grouped_fc2_shared; the _mxfp8_shared pair for MXFP8 experts): one
stream, bitwise the same output.  `tile_queue` (on by default) gives the
grouped GEMMs a tile queue (used where experts average >= 192 rows).
`fuse_route_permute` (on by default) runs route and permute as one library
call (moe_route_permute, one "route_permute" stage), which reuses the
router's per-block counts for the permute; the outputs are bitwise those of
the two calls.  `precision="mxfp8"` runs the expert GEMMs (routed and shared) on MXFP8
operands: the weights are quantised once here, x once per forward (the
router still reads the bf16 x), FC1 writes MXFP8 act, FC2 bf16 outputs."""
from __future__ import annotations

import ctypes
from typing import Callable, Dict, Optional

import torch

from . import _lib
from ._lib import check
from .moe import _dtype_code, _need, route_desc


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class MoELayerForward:
    """route -> permute -> FC1+SwiGLU -> FC2 (-> shared expert) -> combine."""

    STAGES = ("quantize", "route", "permute", "route_permute", "fc1", "fc2", "shared", "combine",
              "fc2_combine")

    def __init__(self, inp: Dict[str, torch.Tensor], *, K: int, score: str = "softmax",
                 pre_softmax: bool = True, capacity_factor: float = 0.0, min_capacity: int = 0,
                 drop_policy: str = "position", pad_to_capacity: bool = False,
                 gather: bool = False, overlap_shared: bool = False, precision: str = "bf16",
                 fuse_route_permute: bool = True, fuse_combine: bool = True,
                 fold_shared: bool = True, tile_queue: bool = True):
        self.lib = _lib.load()
        self.inp = inp
        x = _need(inp["x"], "x")
        self.T, self.h = x.shape
        self.E = inp["w_router"].shape[0]
        self.f = inp["w_gate"].shape[1]
        self.K = K
        self.dt = _dtype_code(x, "x")
        dev = x.device
        self.desc = route_desc(self.T, self.h, self.E, K, x.dtype, score, pre_softmax,
                               capacity_factor, min_capacity, drop_policy, pad_to_capacity)
        self.max_rows = int(self.lib.moe_max_rows(ctypes.byref(self.desc)))
        T, h, E, f, R = self.T, self.h, self.E, self.f, self.max_rows
        e = torch.empty
        self.probs = e((T, E), dtype=torch.float32, device=dev)
        self.routing_map = e((T, E), dtype=torch.uint8, device=dev)
        self.tokens_per_expert = e((E,), dtype=torch.int32, device=dev)
        self.logits = e((T, E), dtype=torch.float32, device=dev)
        self.fused = bool(fuse_route_permute)
        ws_fn = (self.lib.moe_route_permute_workspace_size if self.fused
                 else self.lib.moe_route_workspace_size)
        self.route_ws_bytes = int(ws_fn(ctypes.byref(self.desc)))
        self.route_ws = e((max(self.route_ws_bytes, 1),), dtype=torch.uint8, device=dev)
        if precision not in ("bf16", "mxfp8"):
            raise ValueError(f"unknown precision {precision!r}")
        self.mx = precision == "mxfp8"
        if self.mx and x.dtype != torch.bfloat16:
            raise ValueError("the MXFP8 experts take a bf16 layer")
        self.gather = gather or self.mx
        self.permuted_x = None if self.gather else e((R, h), dtype=x.dtype, device=dev)
        self.permuted_probs = e((R,), dtype=torch.float32, device=dev)
        self.sorted_token = e((R,), dtype=torch.int32, device=dev)
        self.row_id_map = e((T, K), dtype=torch.int32, device=dev)
        self.expert_offsets = e((E + 1,), dtype=torch.int32, device=dev)
        self.perm_ws_bytes = int(self.lib.moe_permute_workspace_size(T, E))
        self.perm_ws = e((max(self.perm_ws_bytes, 1),), dtype=torch.uint8, device=dev)
        self.act = None if self.mx else e((R, f), dtype=x.dtype, device=dev)
        self.expert_out = e((R, h), dtype=x.dtype, device=dev)
        self.out = e((T, h), dtype=x.dtype, device=dev)
        self.shared = "shared_gate" in inp
        if self.shared:
            self.fs = inp["shared_gate"].shape[0]
            self.shared_count = torch.full((1,), T, dtype=torch.int32, device=dev)
            self.shared_act = None if self.mx else e((T, self.fs), dtype=x.dtype, device=dev)
            self.shared_out = e((T, h), dtype=x.dtype, device=dev)
        else:
            self.shared_out = None
        if self.mx:
            u8 = torch.uint8
            q = self._quantize_weight
            self.wq = {k: q(inp[k]) for k in ("w_gate", "w_up", "w_down")}
            self.xq = (e((T, h), dtype=u8, device=dev), e((T, h // 32), dtype=u8, device=dev))
            self.actq = (e((R, f), dtype=u8, device=dev), e((f // 128, R, 4), dtype=u8, device=dev))
            if self.shared:
                self.wq.update({k: q(inp[k][None]) for k in ("shared_gate", "shared_up",
                                                              "shared_down")})
                fs = self.fs
                self.shared_actq = (e((T, fs), dtype=u8, device=dev),
                                    e((fs // 128, T, 4), dtype=u8, device=dev))
        # layers with a shared expert and the gathering FC1 (bf16 or MXFP8
        # experts) run the shared expert's GEMMs as the last tiles of the
        # routed launches
        self.fold_shared = bool(fold_shared and self.shared and self.gather
                                and x.dtype == torch.bfloat16)
        self.overlap_shared = bool(overlap_shared and self.shared and not self.fold_shared)
        # the grouped GEMMs' tile queue (zeroed once; every call leaves it zeroed)
        self.queue = (torch.zeros((_lib.MOE_GEMM_QUEUE_BYTES // 4,), dtype=torch.int32, device=dev)
                      if tile_queue else None)
        self.fused_combine = bool(fuse_combine and K == 1 and not self.shared
                                  and x.dtype == torch.bfloat16)
        if self.overlap_shared:
            self.side = torch.cuda.Stream(device=dev)  # default priority
            self.ev_fork = torch.cuda.Event()
            self.ev_join = torch.cuda.Event()

    def _stream(self):
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def _quantize_weight(self, w: torch.Tensor):
        """MXFP8 codes and k-tiled scales of a [E, n, k] weight along k (done once)."""
        E, n, k = w.shape
        codes = torch.empty((E, n, k), dtype=torch.uint8, device=w.device)
        scales = torch.empty((E, k // 128, n, 4), dtype=torch.uint8, device=w.device)
        check("moe_mxfp8_quantize", self.lib.moe_mxfp8_quantize(
            E * n, k, n, self.dt, _p(w), _p(codes), _p(scales), self._stream()))
        return codes, scales

    def quantize(self):
        check("moe_mxfp8_quantize", self.lib.moe_mxfp8_quantize(
            self.T, self.h, 0, self.dt, _p(self.inp["x"]), _p(self.xq[0]), _p(self.xq[1]),
            self._stream()))

    def route(self):
        i = self.inp
        check("moe_route", self.lib.moe_route(
            ctypes.byref(self.desc), _p(i["x"]), _p(i["w_router"]), _p(i.get("b_router")),
            _p(i.get("expert_bias")), None, _p(self.logits), None, _p(self.probs),
            _p(self.routing_map), _p(self.tokens_per_expert), _p(self.route_ws),
            self.route_ws_bytes, self._stream()))

    def route_permute(self):
        i = self.inp
        check("moe_route_permute", self.lib.moe_route_permute(
            ctypes.byref(self.desc), _p(i["x"]), _p(i["w_router"]), _p(i.get("b_router")),
            _p(i.get("expert_bias")), None, _p(self.logits), None, _p(self.probs),
            _p(self.routing_map), _p(self.tokens_per_expert), self.max_rows,
            _p(self.permuted_x), _p(self.permuted_probs), _p(self.sorted_token),
            _p(self.row_id_map), _p(self.expert_offsets), _p(self.route_ws),
            self.route_ws_bytes, self._stream()))

    def permute(self):
        check("moe_permute", self.lib.moe_permute(
            self.T, self.h, self.E, self.K, self.dt, None if self.gather else _p(self.inp["x"]),
            _p(self.routing_map),
            _p(self.probs), self.max_rows, _p(self.permuted_x), _p(self.permuted_probs),
            _p(self.sorted_token), _p(self.row_id_map), _p(self.expert_offsets), _p(self.perm_ws),
            self.perm_ws_bytes, self._stream()))

    def fc1(self):
        i = self.inp
        if self.mx:
            wg, wu = self.wq["w_gate"], self.wq["w_up"]
            if self.fold_shared:
                sg, su = self.wq["shared_gate"], self.wq["shared_up"]
                check("moe_grouped_fc1_swiglu_mxfp8_shared",
                      self.lib.moe_grouped_fc1_swiglu_mxfp8_shared(
                          self.E, self.h, self.f, self.max_rows, self.T, _p(self.xq[0]),
                          _p(self.xq[1]), _p(self.sorted_token), _p(self.tokens_per_expert),
                          _p(wg[0]), _p(wg[1]), _p(wu[0]), _p(wu[1]), _p(self.actq[0]),
                          _p(self.actq[1]), self.fs, _p(sg[0]), _p(sg[1]), _p(su[0]), _p(su[1]),
                          _p(self.shared_actq[0]), _p(self.shared_actq[1]), _p(self.queue),
                          self._stream()))
                return
            check("moe_grouped_fc1_swiglu_mxfp8", self.lib.moe_grouped_fc1_swiglu_mxfp8(
                self.E, self.h, self.f, self.max_rows, self.T, _p(self.xq[0]), _p(self.xq[1]),
                _p(self.sorted_token), _p(self.tokens_per_expert), _p(wg[0]), _p(wg[1]),
                _p(wu[0]), _p(wu[1]), _p(self.actq[0]), _p(self.actq[1]), _p(self.queue),
                self._stream()))
            return
        if self.fold_shared:
            check("moe_grouped_fc1_swiglu_gather_shared",
                  self.lib.moe_grouped_fc1_swiglu_gather_shared(
                      self.E, self.h, self.f, self.max_rows, self.dt, self.T, _p(i["x"]),
                      _p(self.sorted_token), _p(self.tokens_per_expert), _p(i["w_gate"]),
                      _p(i["w_up"]), _p(self.act), self.fs, _p(i["shared_gate"]),
                      _p(i["shared_up"]), _p(self.shared_act), _p(self.queue), self._stream()))
            return
        if self.gather:
            check("moe_grouped_fc1_swiglu_gather", self.lib.moe_grouped_fc1_swiglu_gather(
                self.E, self.h, self.f, self.max_rows, self.dt, self.T, _p(i["x"]),
                _p(self.sorted_token), _p(self.tokens_per_expert), _p(i["w_gate"]), _p(i["w_up"]),
                _p(self.act), _p(self.queue), self._stream()))
            return
        check("moe_grouped_fc1_swiglu", self.lib.moe_grouped_fc1_swiglu(
            self.E, self.h, self.f, self.max_rows, self.dt, _p(self.permuted_x),
            _p(self.tokens_per_expert), _p(i["w_gate"]), _p(i["w_up"]), _p(self.act),
            _p(self.queue), self._stream()))

    def fc2(self):
        if self.mx:
            wd = self.wq["w_down"]
            if self.fold_shared:
                sd = self.wq["shared_down"]
                check("moe_grouped_fc2_mxfp8_shared", self.lib.moe_grouped_fc2_mxfp8_shared(
                    self.E, self.h, self.f, self.max_rows, _p(self.actq[0]), _p(self.actq[1]),
                    _p(self.tokens_per_expert), _p(wd[0]), _p(wd[1]), _p(self.expert_out),
                    self.T, self.fs, _p(self.shared_actq[0]), _p(self.shared_actq[1]),
                    _p(sd[0]), _p(sd[1]), _p(self.shared_out), _p(self.queue), self._stream()))
                return
            check("moe_grouped_fc2_mxfp8", self.lib.moe_grouped_fc2_mxfp8(
                self.E, self.h, self.f, self.max_rows, _p(self.actq[0]), _p(self.actq[1]),
                _p(self.tokens_per_expert), _p(wd[0]), _p(wd[1]), _p(self.expert_out),
                _p(self.queue), self._stream()))
            return
        if self.fold_shared:
            i = self.inp
            check("moe_grouped_fc2_shared", self.lib.moe_grouped_fc2_shared(
                self.E, self.h, self.f, self.max_rows, self.dt, _p(self.act),
                _p(self.tokens_per_expert), _p(i["w_down"]), _p(self.expert_out), self.T,
                self.fs, _p(self.shared_act), _p(i["shared_down"]), _p(self.shared_out),
                _p(self.queue), self._stream()))
            return
        check("moe_grouped_fc2", self.lib.moe_grouped_fc2(
            self.E, self.h, self.f, self.max_rows, self.dt, _p(self.act),
            _p(self.tokens_per_expert), _p(self.inp["w_down"]), _p(self.expert_out),
            _p(self.queue), self._stream()))

    def shared_expert(self):
        if not self.shared:
            return
        i = self.inp
        if self.mx:
            wg, wu, wd = (self.wq[k] for k in ("shared_gate", "shared_up", "shared_down"))
            check("moe_grouped_fc1_swiglu_mxfp8", self.lib.moe_grouped_fc1_swiglu_mxfp8(
                1, self.h, self.fs, self.T, self.T, _p(self.xq[0]), _p(self.xq[1]), None,
                _p(self.shared_count), _p(wg[0]), _p(wg[1]), _p(wu[0]), _p(wu[1]),
                _p(self.shared_actq[0]), _p(self.shared_actq[1]), None, self._stream()))
            check("moe_grouped_fc2_mxfp8", self.lib.moe_grouped_fc2_mxfp8(
                1, self.h, self.fs, self.T, _p(self.shared_actq[0]), _p(self.shared_actq[1]),
                _p(self.shared_count), _p(wd[0]), _p(wd[1]), _p(self.shared_out), None,
                self._stream()))
            return
        check("moe_grouped_fc1_swiglu", self.lib.moe_grouped_fc1_swiglu(
            1, self.h, self.fs, self.T, self.dt, _p(i["x"]), _p(self.shared_count),
            _p(i["shared_gate"]), _p(i["shared_up"]), _p(self.shared_act), None, self._stream()))
        check("moe_grouped_fc2", self.lib.moe_grouped_fc2(
            1, self.h, self.fs, self.T, self.dt, _p(self.shared_act), _p(self.shared_count),
            _p(i["shared_down"]), _p(self.shared_out), None, self._stream()))

    def fc2_combine(self):
        if self.mx:
            wd = self.wq["w_down"]
            check("moe_grouped_fc2_combine_mxfp8", self.lib.moe_grouped_fc2_combine_mxfp8(
                self.E, self.h, self.f, self.max_rows, self.T, _p(self.actq[0]),
                _p(self.actq[1]), _p(self.tokens_per_expert), _p(wd[0]), _p(wd[1]),
                _p(self.permuted_probs), _p(self.sorted_token), _p(self.row_id_map),
                _p(self.out), self._stream()))
            return
        check("moe_grouped_fc2_combine", self.lib.moe_grouped_fc2_combine(
            self.E, self.h, self.f, self.max_rows, self.dt, self.T, _p(self.act),
            _p(self.tokens_per_expert), _p(self.inp["w_down"]), _p(self.permuted_probs),
            _p(self.sorted_token), _p(self.row_id_map), _p(self.out), self._stream()))

    def combine(self):
        check("moe_combine", self.lib.moe_combine(
            self.T, self.h, self.K, self.dt, _p(self.expert_out), _p(self.permuted_probs),
            _p(self.row_id_map), self.max_rows, _p(self.shared_out), _p(self.out),
            self._stream()))

    def stages(self):
        """Stage names in launch order on the main stream."""
        keep = []
        for n in self.STAGES:
            if n == "quantize" and not self.mx:
                continue
            if n == "shared" and (not self.shared or self.overlap_shared or self.fold_shared):
                continue
            if n in ("route", "permute") and self.fused:
                continue
            if n == "route_permute" and not self.fused:
                continue
            if n in ("fc2", "combine") and self.fused_combine:
                continue
            if n == "fc2_combine" and not self.fused_combine:
                continue
            keep.append(n)
        return keep

    def _fork_shared(self):
        main = torch.cuda.current_stream()
        self.ev_fork.record(main)
        self.side.wait_event(self.ev_fork)
        with torch.cuda.stream(self.side):
            self.shared_expert()
            self.ev_join.record(self.side)

    def forward(self, mark: Optional[Callable[[str], None]] = None) -> torch.Tensor:
        """One layer forward.  `mark(name)` is called before each main-stream
        stage and once more with "end" (used to record timing events)."""
        forked = not self.overlap_shared
        for name in self.stages():
            if not forked and name != "quantize":  # the shared expert reads the quantised x
                self._fork_shared()
                forked = True
            if name == "combine" and self.overlap_shared:
                torch.cuda.current_stream().wait_event(self.ev_join)
            if mark:
                mark(name)
            getattr(self, "shared_expert" if name == "shared" else name)()
        if mark:
            mark("end")
        return self.out
