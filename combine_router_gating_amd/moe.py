"""Python binding of libmoe: same entry points as include/moe.h.

Argument marshalling only.  Tensors are torch CUDA (HIP) tensors; outputs
and workspaces are allocated with torch, every step of the layer runs in
the library's HIP kernels, enqueued on torch's current stream.  There is
no fallback: a missing library or a CPU tensor raises.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_DROP_POSITION, MOE_DROP_PROBS, MOE_F32, MOE_SCORE_SIGMOID,
                   MOE_SCORE_SOFTMAX, MOE_SCORE_SQRTSOFTPLUS, RouteDesc, check)

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}
_SCORE = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID,
          "sqrtsoftplus": MOE_SCORE_SQRTSOFTPLUS}
_DROP = {"position": MOE_DROP_POSITION, "probs": MOE_DROP_PROBS}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def route_desc(T: int, h: int, E: int, K: int, x_dtype: torch.dtype, score: str = "softmax",
               pre_softmax: bool = True, capacity_factor: float = 0.0,
               min_capacity: int = 0, drop_policy: str = "position",
               pad_to_capacity: bool = False) -> RouteDesc:
    if score not in _SCORE:
        raise ValueError(f"unknown score function {score!r}")
    if drop_policy not in _DROP:
        raise ValueError(f"unknown drop policy {drop_policy!r}")
    return RouteDesc(T, h, E, K, _DT[x_dtype], _SCORE[score], 1 if pre_softmax else 0,
                     float(capacity_factor), int(min_capacity), _DROP[drop_policy],
                     1 if pad_to_capacity else 0)


def moe_max_rows(desc: RouteDesc) -> int:
    return int(_lib.load().moe_max_rows(ctypes.byref(desc)))


def moe_route_capacity(desc: RouteDesc) -> int:
    return int(_lib.load().moe_route_capacity(ctypes.byref(desc)))


def moe_route(x: Optional[torch.Tensor], w_router: Optional[torch.Tensor], *, K: int,
              b_router: Optional[torch.Tensor] = None, expert_bias: Optional[torch.Tensor] = None,
              score: str = "softmax", pre_softmax: bool = True, capacity_factor: float = 0.0,
              min_capacity: int = 0, drop_policy: str = "position", pad_to_capacity: bool = False,
              logits_in: Optional[torch.Tensor] = None,
              want_logits: bool = False, want_scores: bool = False,
              T: Optional[int] = None, h: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Router forward (gating, score, top-k, capacity drop)."""
    lib = _lib.load()
    if logits_in is not None:
        _need(logits_in, "logits_in", torch.float32)
        T_, E = logits_in.shape
        dev = logits_in.device
        h_ = h if h is not None else (x.shape[1] if x is not None else 8)
        xdt = x.dtype if x is not None else torch.float32
    else:
        _need(x, "x")
        _need(w_router, "w_router", torch.float32)
        T_, h_ = x.shape
        E = w_router.shape[0]
        _need(w_router, "w_router", torch.float32, (E, h_))
        dev = x.device
        xdt = x.dtype
    if b_router is not None:
        _need(b_router, "b_router", torch.float32, (E,))
    if expert_bias is not None:
        _need(expert_bias, "expert_bias", torch.float32, (E,))
    desc = route_desc(T_, h_, E, K, xdt, score, pre_softmax, capacity_factor, min_capacity,
                      drop_policy, pad_to_capacity)
    probs = torch.empty((T_, E), dtype=torch.float32, device=dev)
    rmap = torch.empty((T_, E), dtype=torch.uint8, device=dev)
    tpe = torch.empty((E,), dtype=torch.int32, device=dev)
    logits = torch.empty((T_, E), dtype=torch.float32, device=dev) if want_logits else None
    scores = torch.empty((T_, E), dtype=torch.float32, device=dev) if want_scores else None
    ws_bytes = int(lib.moe_route_workspace_size(ctypes.byref(desc)))
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    st = lib.moe_route(ctypes.byref(desc), _ptr(x) if logits_in is None else None,
                       _ptr(w_router) if logits_in is None else None, _ptr(b_router),
                       _ptr(expert_bias), _ptr(logits_in), _ptr(logits), _ptr(scores),
                       _ptr(probs), _ptr(rmap), _ptr(tpe), _ptr(ws), ws_bytes, _stream())
    check("moe_route", st)
    out = {"probs": probs, "routing_map": rmap, "tokens_per_expert": tpe,
           "max_rows": moe_max_rows(desc), "capacity": moe_route_capacity(desc)}
    if logits is not None:
        out["logits"] = logits
    if scores is not None:
        out["scores"] = scores
    return out


def moe_route_permute(x: Optional[torch.Tensor], w_router: Optional[torch.Tensor], *, K: int,
                      b_router: Optional[torch.Tensor] = None,
                      expert_bias: Optional[torch.Tensor] = None, score: str = "softmax",
                      pre_softmax: bool = True, capacity_factor: float = 0.0, min_capacity: int = 0,
                      drop_policy: str = "position", pad_to_capacity: bool = False,
                      logits_in: Optional[torch.Tensor] = None, want_logits: bool = False,
                      want_scores: bool = False, copy_rows: bool = True,
                      h: Optional[int] = None, noalloc: bool = False) -> Dict[str, torch.Tensor]:
    """moe_route then moe_permute of its outputs in one library call (the
    permute reuses the router's counting); the union of both results.  With
    noalloc=True the call is moe_route_permute_noalloc (workspace in the
    library's static scratch; the outputs are still allocated here)."""
    lib = _lib.load()
    if logits_in is not None:
        _need(logits_in, "logits_in", torch.float32)
        T_, E = logits_in.shape
        dev = logits_in.device
        h_ = h if h is not None else (x.shape[1] if x is not None else 8)
        xdt = x.dtype if x is not None else torch.float32
    else:
        _need(x, "x")
        _need(w_router, "w_router", torch.float32)
        T_, h_ = x.shape
        E = w_router.shape[0]
        _need(w_router, "w_router", torch.float32, (E, h_))
        dev = x.device
        xdt = x.dtype
    if copy_rows:
        _need(x, "x")
    if b_router is not None:
        _need(b_router, "b_router", torch.float32, (E,))
    if expert_bias is not None:
        _need(expert_bias, "expert_bias", torch.float32, (E,))
    desc = route_desc(T_, h_, E, K, xdt, score, pre_softmax, capacity_factor, min_capacity,
                      drop_policy, pad_to_capacity)
    rows = max(moe_max_rows(desc), 0)
    e = torch.empty
    out = {"probs": e((T_, E), dtype=torch.float32, device=dev),
           "routing_map": e((T_, E), dtype=torch.uint8, device=dev),
           "tokens_per_expert": e((E,), dtype=torch.int32, device=dev),
           "permuted_x": e((rows, h_), dtype=xdt, device=dev) if copy_rows else None,
           "permuted_probs": e((rows,), dtype=torch.float32, device=dev),
           "sorted_token": e((rows,), dtype=torch.int32, device=dev),
           "row_id_map": e((T_, K), dtype=torch.int32, device=dev),
           "expert_offsets": e((E + 1,), dtype=torch.int32, device=dev),
           "max_rows": rows, "capacity": moe_route_capacity(desc)}
    logits = e((T_, E), dtype=torch.float32, device=dev) if want_logits else None
    scores = e((T_, E), dtype=torch.float32, device=dev) if want_scores else None
    args = (ctypes.byref(desc), _ptr(x) if (logits_in is None or copy_rows) else None,
            _ptr(w_router) if logits_in is None else None, _ptr(b_router), _ptr(expert_bias),
            _ptr(logits_in), _ptr(logits), _ptr(scores), _ptr(out["probs"]),
            _ptr(out["routing_map"]), _ptr(out["tokens_per_expert"]), rows,
            _ptr(out["permuted_x"]), _ptr(out["permuted_probs"]), _ptr(out["sorted_token"]),
            _ptr(out["row_id_map"]), _ptr(out["expert_offsets"]))
    if noalloc:
        # the library's static scratch: no workspace is allocated here
        check("moe_route_permute_noalloc", lib.moe_route_permute_noalloc(*args, _stream()))
    else:
        ws_bytes = int(lib.moe_route_permute_workspace_size(ctypes.byref(desc)))
        ws = e((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
        check("moe_route_permute", lib.moe_route_permute(*args, _ptr(ws), ws_bytes, _stream()))
    if logits is not None:
        out["logits"] = logits
    if scores is not None:
        out["scores"] = scores
    return out


def moe_router_aux_loss(scores: torch.Tensor, tokens_per_expert: torch.Tensor, *, K: int,
                        score: str = "softmax") -> torch.Tensor:
    """Forward value of the load-balancing loss, E * sum_e f_e * P_e (fp32 [1])."""
    lib = _lib.load()
    _need(scores, "scores", torch.float32)
    T, E = scores.shape
    _need(tokens_per_expert, "tokens_per_expert", torch.int32, (E,))
    loss = torch.empty((1,), dtype=torch.float32, device=scores.device)
    ws_bytes = int(lib.moe_aux_loss_workspace_size(T, E))
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=scores.device)
    st = lib.moe_router_aux_loss(T, E, K, _SCORE[score], _ptr(scores), _ptr(tokens_per_expert),
                                 _ptr(loss), _ptr(ws), ws_bytes, _stream())
    check("moe_router_aux_loss", st)
    return loss


def moe_accumulate_tokens_per_expert(tokens_per_expert: torch.Tensor,
                                     local_tokens_per_expert: torch.Tensor) -> torch.Tensor:
    """local_tokens_per_expert += tokens_per_expert (int64, in place)."""
    E = tokens_per_expert.shape[0]
    _need(tokens_per_expert, "tokens_per_expert", torch.int32, (E,))
    _need(local_tokens_per_expert, "local_tokens_per_expert", torch.int64, (E,))
    st = _lib.load().moe_accumulate_tokens_per_expert(E, _ptr(tokens_per_expert),
                                                      _ptr(local_tokens_per_expert), _stream())
    check("moe_accumulate_tokens_per_expert", st)
    return local_tokens_per_expert


def moe_update_expert_bias(local_tokens_per_expert: torch.Tensor, expert_bias: torch.Tensor,
                           update_rate: float, reset: bool = True) -> torch.Tensor:
    """expert_bias += sign(mean - count) * update_rate (in place); optionally
    zero the running counts."""
    E = expert_bias.shape[0]
    _need(local_tokens_per_expert, "local_tokens_per_expert", torch.int64, (E,))
    _need(expert_bias, "expert_bias", torch.float32, (E,))
    st = _lib.load().moe_update_expert_bias(E, _ptr(local_tokens_per_expert), _ptr(expert_bias),
                                            float(update_rate), 1 if reset else 0, _stream())
    check("moe_update_expert_bias", st)
    return expert_bias


def moe_permute(x: torch.Tensor, routing_map: torch.Tensor, probs: torch.Tensor, K: int,
                max_rows: int, copy_rows: bool = True) -> Dict[str, torch.Tensor]:
    """Expert-major permute of token rows (copy_rows=False: indices and probs
    only, for the gathering FC1)."""
    lib = _lib.load()
    _need(x, "x")
    T, h = x.shape
    E = routing_map.shape[1]
    _need(routing_map, "routing_map", torch.uint8, (T, E))
    _need(probs, "probs", torch.float32, (T, E))
    dev = x.device
    rows = max(int(max_rows), 0)
    px = torch.empty((rows, h), dtype=x.dtype, device=dev) if copy_rows else None
    pp = torch.empty((rows,), dtype=torch.float32, device=dev)
    st_tok = torch.empty((rows,), dtype=torch.int32, device=dev)
    rid = torch.empty((T, K), dtype=torch.int32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    ws_bytes = int(lib.moe_permute_workspace_size(T, E))
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    st = lib.moe_permute(T, h, E, K, _dtype_code(x, "x"), _ptr(x) if copy_rows else None,
                         _ptr(routing_map), _ptr(probs),
                         rows, _ptr(px), _ptr(pp), _ptr(st_tok), _ptr(rid), _ptr(offs), _ptr(ws),
                         ws_bytes, _stream())
    check("moe_permute", st)
    return {"permuted_x": px, "permuted_probs": pp, "sorted_token": st_tok, "row_id_map": rid,
            "expert_offsets": offs}


def moe_clock_probe(out: torch.Tensor, spin_us: int) -> torch.Tensor:
    """Queue one clock probe on the current stream: after spin_us
    microseconds, out (int64[2] on the GPU) holds the shader-clock cycles and
    the 100 MHz ticks that elapsed (clock MHz = 100 * out[0] / out[1])."""
    _need(out, "out", torch.int64, (2,))
    check("moe_clock_probe", _lib.load().moe_clock_probe(_ptr(out), int(spin_us), _stream()))
    return out


def gemm_queue(device) -> torch.Tensor:
    """A zeroed tile-queue buffer for the grouped GEMM entry points
    (MOE_GEMM_QUEUE_BYTES; the calls leave it zeroed)."""
    return torch.zeros((_lib.MOE_GEMM_QUEUE_BYTES // 4,), dtype=torch.int32, device=device)


def _mlp_args(permuted_x, tokens_per_expert, w_a, w_b=None):
    _need(permuted_x, "rows")
    _need(tokens_per_expert, "tokens_per_expert", torch.int32)
    E = tokens_per_expert.shape[0]
    _need(w_a, "weight", permuted_x.dtype)
    if w_b is not None:
        _need(w_b, "weight", permuted_x.dtype, w_a.shape)
    if w_a.shape[0] != E:
        raise ValueError("weights and tokens_per_expert disagree on E")
    return E


def moe_grouped_fc1_swiglu(permuted_x: torch.Tensor, tokens_per_expert: torch.Tensor,
                           w_gate: torch.Tensor, w_up: torch.Tensor,
                           act: Optional[torch.Tensor] = None,
                           queue: Optional[torch.Tensor] = None) -> torch.Tensor:
    """act = silu(x W_gate^T) * (x W_up^T), per expert row range."""
    E = _mlp_args(permuted_x, tokens_per_expert, w_gate, w_up)
    rows, h = permuted_x.shape
    f = w_gate.shape[1]
    _need(w_gate, "w_gate", permuted_x.dtype, (E, f, h))
    if act is None:
        act = torch.empty((rows, f), dtype=permuted_x.dtype, device=permuted_x.device)
    _need(act, "act", permuted_x.dtype, (rows, f))
    st = _lib.load().moe_grouped_fc1_swiglu(E, h, f, rows, _dtype_code(permuted_x, "x"),
                                            _ptr(permuted_x), _ptr(tokens_per_expert),
                                            _ptr(w_gate), _ptr(w_up), _ptr(act), _ptr(queue),
                                            _stream())
    check("moe_grouped_fc1_swiglu", st)
    return act


def moe_grouped_fc1_swiglu_gather(x: torch.Tensor, sorted_token: torch.Tensor,
                                  tokens_per_expert: torch.Tensor, w_gate: torch.Tensor,
                                  w_up: torch.Tensor, act: Optional[torch.Tensor] = None,
                                  queue: Optional[torch.Tensor] = None) -> torch.Tensor:
    """act = silu(x[sorted_token] W_gate^T) * (x[sorted_token] W_up^T), per expert row range."""
    E = _mlp_args(x, tokens_per_expert, w_gate, w_up)
    T, h = x.shape
    rows = sorted_token.shape[0]
    _need(sorted_token, "sorted_token", torch.int32, (rows,))
    f = w_gate.shape[1]
    _need(w_gate, "w_gate", x.dtype, (E, f, h))
    if act is None:
        act = torch.empty((rows, f), dtype=x.dtype, device=x.device)
    _need(act, "act", x.dtype, (rows, f))
    st = _lib.load().moe_grouped_fc1_swiglu_gather(E, h, f, rows, _dtype_code(x, "x"), T, _ptr(x),
                                                   _ptr(sorted_token), _ptr(tokens_per_expert),
                                                   _ptr(w_gate), _ptr(w_up), _ptr(act), _ptr(queue),
                                                   _stream())
    check("moe_grouped_fc1_swiglu_gather", st)
    return act


def moe_grouped_fc1_swiglu_gather_shared(x: torch.Tensor, sorted_token: torch.Tensor,
                                         tokens_per_expert: torch.Tensor, w_gate: torch.Tensor,
                                         w_up: torch.Tensor, shared_gate: torch.Tensor,
                                         shared_up: torch.Tensor, act: Optional[torch.Tensor] = None,
                                         shared_act: Optional[torch.Tensor] = None,
                                         queue: Optional[torch.Tensor] = None):
    """The gathering FC1 of the routed experts and the shared expert's FC1
    over all tokens in one launch; returns (act, shared_act)."""
    E = _mlp_args(x, tokens_per_expert, w_gate, w_up)
    T, h = x.shape
    rows = sorted_token.shape[0]
    _need(sorted_token, "sorted_token", torch.int32, (rows,))
    f = w_gate.shape[1]
    _need(w_gate, "w_gate", x.dtype, (E, f, h))
    fs = shared_gate.shape[0]
    _need(shared_gate, "shared_gate", x.dtype, (fs, h))
    _need(shared_up, "shared_up", x.dtype, (fs, h))
    if act is None:
        act = torch.empty((rows, f), dtype=x.dtype, device=x.device)
    if shared_act is None:
        shared_act = torch.empty((T, fs), dtype=x.dtype, device=x.device)
    _need(act, "act", x.dtype, (rows, f))
    _need(shared_act, "shared_act", x.dtype, (T, fs))
    st = _lib.load().moe_grouped_fc1_swiglu_gather_shared(
        E, h, f, rows, _dtype_code(x, "x"), T, _ptr(x), _ptr(sorted_token),
        _ptr(tokens_per_expert), _ptr(w_gate), _ptr(w_up), _ptr(act), fs, _ptr(shared_gate),
        _ptr(shared_up), _ptr(shared_act), _ptr(queue), _stream())
    check("moe_grouped_fc1_swiglu_gather_shared", st)
    return act, shared_act


def moe_grouped_fc2_shared(act: torch.Tensor, tokens_per_expert: torch.Tensor,
                           w_down: torch.Tensor, shared_act: torch.Tensor,
                           shared_down: torch.Tensor, expert_out: Optional[torch.Tensor] = None,
                           shared_out: Optional[torch.Tensor] = None,
                           queue: Optional[torch.Tensor] = None):
    """The routed experts' FC2 and the shared expert's FC2 in one launch;
    returns (expert_out, shared_out)."""
    E = _mlp_args(act, tokens_per_expert, w_down)
    rows, f = act.shape
    h = w_down.shape[1]
    _need(w_down, "w_down", act.dtype, (E, h, f))
    T, fs = shared_act.shape
    _need(shared_act, "shared_act", act.dtype, (T, fs))
    _need(shared_down, "shared_down", act.dtype, (h, fs))
    if expert_out is None:
        expert_out = torch.empty((rows, h), dtype=act.dtype, device=act.device)
    if shared_out is None:
        shared_out = torch.empty((T, h), dtype=act.dtype, device=act.device)
    _need(expert_out, "expert_out", act.dtype, (rows, h))
    _need(shared_out, "shared_out", act.dtype, (T, h))
    st = _lib.load().moe_grouped_fc2_shared(
        E, h, f, rows, _dtype_code(act, "act"), _ptr(act), _ptr(tokens_per_expert), _ptr(w_down),
        _ptr(expert_out), T, fs, _ptr(shared_act), _ptr(shared_down), _ptr(shared_out), _ptr(queue), _stream())
    check("moe_grouped_fc2_shared", st)
    return expert_out, shared_out


def moe_grouped_fc2(act: torch.Tensor, tokens_per_expert: torch.Tensor, w_down: torch.Tensor,
                    expert_out: Optional[torch.Tensor] = None,
                    queue: Optional[torch.Tensor] = None) -> torch.Tensor:
    """expert_out = act W_down^T, per expert row range."""
    E = _mlp_args(act, tokens_per_expert, w_down)
    rows, f = act.shape
    h = w_down.shape[1]
    _need(w_down, "w_down", act.dtype, (E, h, f))
    if expert_out is None:
        expert_out = torch.empty((rows, h), dtype=act.dtype, device=act.device)
    _need(expert_out, "expert_out", act.dtype, (rows, h))
    st = _lib.load().moe_grouped_fc2(E, h, f, rows, _dtype_code(act, "act"), _ptr(act),
                                     _ptr(tokens_per_expert), _ptr(w_down), _ptr(expert_out),
                                     _ptr(queue), _stream())
    check("moe_grouped_fc2", st)
    return expert_out


def moe_grouped_fc2_combine(act: torch.Tensor, tokens_per_expert: torch.Tensor,
                            w_down: torch.Tensor, permuted_probs: torch.Tensor,
                            sorted_token: torch.Tensor, row_id_map: torch.Tensor,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-1 combine fused into FC2: out[t] = p * (act W_down^T)[row of t],
    zero for dropped tokens; bitwise moe_grouped_fc2 then moe_combine (K=1)."""
    E = _mlp_args(act, tokens_per_expert, w_down)
    rows, f = act.shape
    h = w_down.shape[1]
    _need(w_down, "w_down", act.dtype, (E, h, f))
    T = row_id_map.shape[0]
    if row_id_map.dim() == 2:
        if row_id_map.shape[1] != 1:
            raise ValueError("moe_grouped_fc2_combine is for top-1 routing (row_id_map [T, 1])")
    _need(row_id_map, "row_id_map", torch.int32)
    _need(permuted_probs, "permuted_probs", torch.float32, (rows,))
    _need(sorted_token, "sorted_token", torch.int32, (rows,))
    if out is None:
        out = torch.empty((T, h), dtype=act.dtype, device=act.device)
    _need(out, "out", act.dtype, (T, h))
    st = _lib.load().moe_grouped_fc2_combine(E, h, f, rows, _dtype_code(act, "act"), T, _ptr(act),
                                             _ptr(tokens_per_expert), _ptr(w_down),
                                             _ptr(permuted_probs), _ptr(sorted_token),
                                             _ptr(row_id_map), _ptr(out), _stream())
    check("moe_grouped_fc2_combine", st)
    return out


def moe_grouped_mlp(permuted_x: torch.Tensor, tokens_per_expert: torch.Tensor,
                    w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                    queue: Optional[torch.Tensor] = None):
    """SwiGLU MLP of every expert over its row range; returns (act, expert_out)."""
    E = _mlp_args(permuted_x, tokens_per_expert, w_gate, w_up)
    rows, h = permuted_x.shape
    f = w_gate.shape[1]
    _need(w_gate, "w_gate", permuted_x.dtype, (E, f, h))
    _need(w_down, "w_down", permuted_x.dtype, (E, h, f))
    act = torch.empty((rows, f), dtype=permuted_x.dtype, device=permuted_x.device)
    out = torch.empty((rows, h), dtype=permuted_x.dtype, device=permuted_x.device)
    st = _lib.load().moe_grouped_mlp(E, h, f, rows, _dtype_code(permuted_x, "x"), _ptr(permuted_x),
                                     _ptr(tokens_per_expert), _ptr(w_gate), _ptr(w_up),
                                     _ptr(w_down), _ptr(act), _ptr(out), _ptr(queue),
                                     _stream())
    check("moe_grouped_mlp", st)
    return act, out


def moe_mxfp8_quantize(src: torch.Tensor, tile_rows: int = 0):
    """MXFP8-E4M3 of a 2-D tensor along its last dim: (codes uint8 [rows, cols],
    scales uint8): row-major [rows, cols/32] when tile_rows = 0, else k-tiled
    [rows/R, cols/128, R, 4] with R = tile_rows."""
    _need(src, "src")
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    if tile_rows:
        scales = torch.empty((rows // tile_rows, cols // 128, tile_rows, 4), dtype=torch.uint8,
                             device=src.device)
    else:
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=src.device)
    st = _lib.load().moe_mxfp8_quantize(rows, cols, int(tile_rows), _dtype_code(src, "src"),
                                        _ptr(src), _ptr(codes), _ptr(scales), _stream())
    check("moe_mxfp8_quantize", st)
    return codes, scales


def moe_mxfp8_quantize_weight(w: torch.Tensor):
    """A [E, n, k] weight in the layout the MXFP8 GEMMs read: (codes [E, n, k],
    scales k-tiled [E, k/128, n, 4])."""
    E, n, k = w.shape
    codes, scales = moe_mxfp8_quantize(w.reshape(E * n, k), tile_rows=n)
    return codes.reshape(E, n, k), scales


def moe_grouped_fc1_swiglu_mxfp8(x_codes, x_scales, sorted_token, tokens_per_expert, wg, wu,
                                 max_rows: int, act=None, queue: Optional[torch.Tensor] = None):
    """MXFP8 FC1 + SwiGLU: wg/wu from moe_mxfp8_quantize_weight; returns
    (act_codes [max_rows,f], act_scales k-tiled [f/128, max_rows, 4])."""
    T, h = x_codes.shape
    E, f, _ = wg[0].shape
    _need(x_codes, "x_codes", torch.uint8)
    _need(x_scales, "x_scales", torch.uint8, (T, h // 32))
    _need(tokens_per_expert, "tokens_per_expert", torch.int32, (E,))
    for name, (c, sc) in (("wg", wg), ("wu", wu)):
        _need(c, name, torch.uint8, (E, f, h))
        _need(sc, name + " scales", torch.uint8, (E, h // 128, f, 4))
    if sorted_token is not None:
        _need(sorted_token, "sorted_token", torch.int32)
        if sorted_token.numel() < max_rows:
            raise ValueError("sorted_token needs max_rows entries")
    elif T < max_rows:
        raise ValueError("without sorted_token, x holds the GEMM rows: it needs max_rows rows")
    if act is None:
        act = (torch.empty((max_rows, f), dtype=torch.uint8, device=x_codes.device),
               torch.empty((f // 128, max_rows, 4), dtype=torch.uint8, device=x_codes.device))
    else:
        _need(act[0], "act codes", torch.uint8, (max_rows, f))
        _need(act[1], "act scales", torch.uint8, (f // 128, max_rows, 4))
    st = _lib.load().moe_grouped_fc1_swiglu_mxfp8(
        E, h, f, max_rows, T, _ptr(x_codes), _ptr(x_scales), _ptr(sorted_token),
        _ptr(tokens_per_expert), _ptr(wg[0]), _ptr(wg[1]), _ptr(wu[0]), _ptr(wu[1]), _ptr(act[0]),
        _ptr(act[1]), _ptr(queue), _stream())
    check("moe_grouped_fc1_swiglu_mxfp8", st)
    return act


def moe_grouped_fc1_swiglu_mxfp8_shared(x_codes, x_scales, sorted_token, tokens_per_expert, wg,
                                        wu, max_rows: int, sg, su, act=None, shared_act=None,
                                        queue: Optional[torch.Tensor] = None):
    """The gathering MXFP8 FC1 of the routed experts and the shared expert's
    MXFP8 FC1 over all tokens in one launch; sg/su from
    moe_mxfp8_quantize_weight (E = 1); returns (act, shared_act), each
    (codes, k-tiled scales)."""
    T, h = x_codes.shape
    E, f, _ = wg[0].shape
    fs = sg[0].shape[1]
    _need(x_codes, "x_codes", torch.uint8)
    _need(x_scales, "x_scales", torch.uint8, (T, h // 32))
    _need(tokens_per_expert, "tokens_per_expert", torch.int32, (E,))
    _need(sorted_token, "sorted_token", torch.int32)
    if sorted_token.numel() < max_rows:
        raise ValueError("sorted_token needs max_rows entries")
    for name, (c, sc), rows, fdim in (("wg", wg, E, f), ("wu", wu, E, f), ("sg", sg, 1, fs),
                                      ("su", su, 1, fs)):
        _need(c, name, torch.uint8, (rows, fdim, h))
        _need(sc, name + " scales", torch.uint8, (rows, h // 128, fdim, 4))
    dev = x_codes.device
    if act is None:
        act = (torch.empty((max_rows, f), dtype=torch.uint8, device=dev),
               torch.empty((f // 128, max_rows, 4), dtype=torch.uint8, device=dev))
    if shared_act is None:
        shared_act = (torch.empty((T, fs), dtype=torch.uint8, device=dev),
                      torch.empty((fs // 128, T, 4), dtype=torch.uint8, device=dev))
    _need(act[0], "act codes", torch.uint8, (max_rows, f))
    _need(act[1], "act scales", torch.uint8, (f // 128, max_rows, 4))
    _need(shared_act[0], "shared act codes", torch.uint8, (T, fs))
    _need(shared_act[1], "shared act scales", torch.uint8, (fs // 128, T, 4))
    st = _lib.load().moe_grouped_fc1_swiglu_mxfp8_shared(
        E, h, f, max_rows, T, _ptr(x_codes), _ptr(x_scales), _ptr(sorted_token),
        _ptr(tokens_per_expert), _ptr(wg[0]), _ptr(wg[1]), _ptr(wu[0]), _ptr(wu[1]), _ptr(act[0]),
        _ptr(act[1]), fs, _ptr(sg[0]), _ptr(sg[1]), _ptr(su[0]), _ptr(su[1]), _ptr(shared_act[0]),
        _ptr(shared_act[1]), _ptr(queue), _stream())
    check("moe_grouped_fc1_swiglu_mxfp8_shared", st)
    return act, shared_act


def moe_grouped_fc2_mxfp8(act_codes, act_scales, tokens_per_expert, wd, expert_out=None,
                          queue: Optional[torch.Tensor] = None):
    """MXFP8 FC2 on FC1's act: wd from moe_mxfp8_quantize_weight; returns bf16 [max_rows,h]."""
    rows, f = act_codes.shape
    E, h, _ = wd[0].shape
    _need(act_codes, "act_codes", torch.uint8)
    _need(act_scales, "act_scales", torch.uint8, (f // 128, rows, 4))
    _need(wd[0], "wd", torch.uint8, (E, h, f))
    _need(wd[1], "wd scales", torch.uint8, (E, f // 128, h, 4))
    if expert_out is None:
        expert_out = torch.empty((rows, h), dtype=torch.bfloat16, device=act_codes.device)
    st = _lib.load().moe_grouped_fc2_mxfp8(E, h, f, rows, _ptr(act_codes), _ptr(act_scales),
                                           _ptr(tokens_per_expert), _ptr(wd[0]), _ptr(wd[1]),
                                           _ptr(expert_out), _ptr(queue), _stream())
    check("moe_grouped_fc2_mxfp8", st)
    return expert_out


def moe_grouped_fc2_mxfp8_shared(act_codes, act_scales, tokens_per_expert, wd, shared_act, sd,
                                 expert_out=None, shared_out=None,
                                 queue: Optional[torch.Tensor] = None):
    """The MXFP8 FC2 of the routed experts and the shared expert's MXFP8 FC2
    in one launch; shared_act as moe_grouped_fc1_swiglu_mxfp8_shared returns
    it, sd from moe_mxfp8_quantize_weight (E = 1); returns (expert_out,
    shared_out), bf16."""
    rows, f = act_codes.shape
    E, h, _ = wd[0].shape
    T, fs = shared_act[0].shape
    _need(act_codes, "act_codes", torch.uint8)
    _need(act_scales, "act_scales", torch.uint8, (f // 128, rows, 4))
    _need(tokens_per_expert, "tokens_per_expert", torch.int32, (E,))
    _need(wd[0], "wd", torch.uint8, (E, h, f))
    _need(wd[1], "wd scales", torch.uint8, (E, f // 128, h, 4))
    _need(shared_act[0], "shared act codes", torch.uint8, (T, fs))
    _need(shared_act[1], "shared act scales", torch.uint8, (fs // 128, T, 4))
    _need(sd[0], "sd", torch.uint8, (1, h, fs))
    _need(sd[1], "sd scales", torch.uint8, (1, fs // 128, h, 4))
    dev = act_codes.device
    if expert_out is None:
        expert_out = torch.empty((rows, h), dtype=torch.bfloat16, device=dev)
    if shared_out is None:
        shared_out = torch.empty((T, h), dtype=torch.bfloat16, device=dev)
    _need(expert_out, "expert_out", torch.bfloat16, (rows, h))
    _need(shared_out, "shared_out", torch.bfloat16, (T, h))
    st = _lib.load().moe_grouped_fc2_mxfp8_shared(
        E, h, f, rows, _ptr(act_codes), _ptr(act_scales), _ptr(tokens_per_expert), _ptr(wd[0]),
        _ptr(wd[1]), _ptr(expert_out), T, fs, _ptr(shared_act[0]), _ptr(shared_act[1]),
        _ptr(sd[0]), _ptr(sd[1]), _ptr(shared_out), _ptr(queue), _stream())
    check("moe_grouped_fc2_mxfp8_shared", st)
    return expert_out, shared_out


def moe_grouped_fc2_combine_mxfp8(act_codes, act_scales, tokens_per_expert, wd, permuted_probs,
                                  sorted_token, row_id_map, out=None):
    """Top-1 combine fused into the MXFP8 FC2: out[t] = p * y[row of t] (bf16
    [T,h]), zero for dropped tokens; bitwise moe_grouped_fc2_mxfp8 then
    moe_combine (K=1)."""
    rows, f = act_codes.shape
    E, h, _ = wd[0].shape
    _need(act_codes, "act_codes", torch.uint8)
    _need(act_scales, "act_scales", torch.uint8, (f // 128, rows, 4))
    _need(wd[0], "wd", torch.uint8, (E, h, f))
    _need(wd[1], "wd scales", torch.uint8, (E, f // 128, h, 4))
    _need(tokens_per_expert, "tokens_per_expert", torch.int32, (E,))
    T = row_id_map.shape[0]
    if row_id_map.dim() == 2 and row_id_map.shape[1] != 1:
        raise ValueError("moe_grouped_fc2_combine_mxfp8 is for top-1 routing (row_id_map [T, 1])")
    _need(row_id_map, "row_id_map", torch.int32)
    _need(permuted_probs, "permuted_probs", torch.float32, (rows,))
    _need(sorted_token, "sorted_token", torch.int32, (rows,))
    if out is None:
        out = torch.empty((T, h), dtype=torch.bfloat16, device=act_codes.device)
    _need(out, "out", torch.bfloat16, (T, h))
    st = _lib.load().moe_grouped_fc2_combine_mxfp8(
        E, h, f, rows, T, _ptr(act_codes), _ptr(act_scales), _ptr(tokens_per_expert), _ptr(wd[0]),
        _ptr(wd[1]), _ptr(permuted_probs), _ptr(sorted_token), _ptr(row_id_map), _ptr(out),
        _stream())
    check("moe_grouped_fc2_combine_mxfp8", st)
    return out


def moe_combine(expert_out: torch.Tensor, permuted_probs: torch.Tensor, row_id_map: torch.Tensor,
                shared_out: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = sum_k p * expert_out[row_id_map[t,k]] (+ shared_out[t])."""
    _need(expert_out, "expert_out")
    rows, h = expert_out.shape
    _need(permuted_probs, "permuted_probs", torch.float32, (rows,))
    _need(row_id_map, "row_id_map", torch.int32)
    T, K = row_id_map.shape
    if shared_out is not None:
        _need(shared_out, "shared_out", expert_out.dtype, (T, h))
    if out is None:
        out = torch.empty((T, h), dtype=expert_out.dtype, device=expert_out.device)
    _need(out, "out", expert_out.dtype, (T, h))
    st = _lib.load().moe_combine(T, h, K, _dtype_code(expert_out, "expert_out"), _ptr(expert_out),
                                 _ptr(permuted_probs), _ptr(row_id_map), rows, _ptr(shared_out),
                                 _ptr(out), _stream())
    check("moe_combine", st)
    return out


def moe_forward(inp: Dict[str, torch.Tensor], *, K: int, score: str = "softmax",
                pre_softmax: bool = True, capacity_factor: float = 0.0, min_capacity: int = 0,
                drop_policy: str = "position", pad_to_capacity: bool = False,
                gather: bool = False, want_logits: bool = False) -> Dict[str, torch.Tensor]:
    """route -> permute -> grouped SwiGLU experts -> combine (+ shared expert).
    With gather=True the permute writes no row copies and FC1 reads the
    token rows through sorted_token.

    `inp` holds the tensors datagen.make_inputs returns (x, w_router,
    optional b_router / expert_bias, w_gate, w_up, w_down, optional
    shared_gate / shared_up / shared_down).
    """
    x = inp["x"]
    r = moe_route(x, inp["w_router"], K=K, b_router=inp.get("b_router"),
                  expert_bias=inp.get("expert_bias"), score=score, pre_softmax=pre_softmax,
                  capacity_factor=capacity_factor, min_capacity=min_capacity,
                  drop_policy=drop_policy, pad_to_capacity=pad_to_capacity,
                  want_logits=want_logits)
    pm = moe_permute(x, r["routing_map"], r["probs"], K, r["max_rows"], copy_rows=not gather)
    if gather:
        act = moe_grouped_fc1_swiglu_gather(x, pm["sorted_token"], r["tokens_per_expert"],
                                            inp["w_gate"], inp["w_up"])
    else:
        act = moe_grouped_fc1_swiglu(pm["permuted_x"], r["tokens_per_expert"], inp["w_gate"],
                                     inp["w_up"])
    y = moe_grouped_fc2(act, r["tokens_per_expert"], inp["w_down"])
    shared_out = None
    if "shared_gate" in inp:
        T = x.shape[0]
        ones = torch.full((1,), T, dtype=torch.int32, device=x.device)
        s_act = moe_grouped_fc1_swiglu(x, ones, inp["shared_gate"][None], inp["shared_up"][None])
        shared_out = moe_grouped_fc2(s_act, ones, inp["shared_down"][None])
    out = moe_combine(y, pm["permuted_probs"], pm["row_id_map"], shared_out)
    res = dict(r)
    res.update(pm)
    res.update({"act": act, "expert_out": y, "shared_out": shared_out, "out": out})
    return res
