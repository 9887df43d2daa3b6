"""Loads libmoe.so (built in-tree) and declares its C signatures."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

c_i64, c_i32, c_sz, c_vp, c_f32 = (ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                                   ctypes.c_void_p, ctypes.c_float)

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SQRTSOFTPLUS = 0, 1, 2
MOE_DROP_POSITION, MOE_DROP_PROBS = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/moe.h
MOE_GEMM_QUEUE_BYTES = 2048  # include/moe.h
ABI_VERSION = 8  # moe_abi_version() of the library these signatures describe


class RouteDesc(ctypes.Structure):
    """Mirror of moe_route_desc."""

    _fields_ = [
        ("T", c_i64), ("h", c_i64), ("E", c_i64), ("K", c_i64),
        ("x_dtype", c_i32), ("score", c_i32), ("pre_softmax", c_i32),
        ("capacity_factor", c_f32), ("min_capacity", c_i64),
        ("drop_policy", c_i32), ("pad_to_capacity", c_i32),
    ]


# name -> (restype, argtypes); every function the header declares
SIGNATURES = {
    "moe_abi_version": (c_i32, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_clock_probe": (c_i32, [c_vp, c_i64, c_vp]),
    "moe_route_workspace_size": (c_sz, [ctypes.POINTER(RouteDesc)]),
    "moe_route_capacity": (c_i64, [ctypes.POINTER(RouteDesc)]),
    "moe_max_rows": (c_i64, [ctypes.POINTER(RouteDesc)]),
    "moe_route": (c_i32, [ctypes.POINTER(RouteDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                          c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_aux_loss_workspace_size": (c_sz, [c_i64, c_i64]),
    "moe_router_aux_loss": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz,
                                    c_vp]),
    "moe_accumulate_tokens_per_expert": (c_i32, [c_i64, c_vp, c_vp, c_vp]),
    "moe_update_expert_bias": (c_i32, [c_i64, c_vp, c_vp, c_f32, c_i32, c_vp]),
    "moe_permute_workspace_size": (c_sz, [c_i64, c_i64]),
    "moe_route_permute_workspace_size": (c_sz, [ctypes.POINTER(RouteDesc)]),
    "moe_route_permute": (c_i32, [ctypes.POINTER(RouteDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_vp, c_sz, c_vp]),
    "moe_route_permute_noalloc": (c_i32, [ctypes.POINTER(RouteDesc), c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_vp]),
    "moe_permute": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp,
                            c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_grouped_mlp": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc1_swiglu": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp,
                                       c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc1_swiglu_gather": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_i64, c_vp,
                                              c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc1_swiglu_gather_shared": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_i64,
                                                     c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                                     c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc2_shared": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp,
                                       c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_mxfp8_quantize": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc1_swiglu_mxfp8": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp,
                                             c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc1_swiglu_mxfp8_shared": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp,
                                                    c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                    c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                    c_vp]),
    "moe_grouped_fc2_mxfp8": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, c_vp, c_vp]),
    "moe_grouped_fc2_mxfp8_shared": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                             c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_vp, c_vp]),
    "moe_grouped_fc2_combine_mxfp8": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp,
                                              c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc2": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_grouped_fc2_combine": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_i32, c_i64, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_combine": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp,
                            c_vp]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.moe_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{path} has interface version {lib.moe_abi_version()}, these "
                               f"bindings expect {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        msg = load().moe_last_error()
        raise MoEError(fn, status, msg.decode() if msg else "")
