"""Host-only checks of the C interface: the library loads, exports every
symbol include/moe.h declares, and rejects bad arguments before touching
the GPU.  No call here reaches a HIP API."""
import ctypes
import os
import re

import pytest
import torch

import combine_router_gating_amd as moe
from combine_router_gating_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = moe.load()
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.SIGNATURES) == names
    assert lib.moe_abi_version() == 8 == _lib.ABI_VERSION


def test_route_desc_layout_matches_c():
    # int64 x4, int32 x3, float, int64, int32 x2: 64 bytes with natural alignment
    assert ctypes.sizeof(_lib.RouteDesc) == 64
    assert _lib.RouteDesc.min_capacity.offset == 48
    assert _lib.RouteDesc.drop_policy.offset == 56
    assert _lib.RouteDesc.pad_to_capacity.offset == 60


def _desc(**kw):
    base = dict(T=8192, h=2048, E=64, K=1, x_dtype=torch.bfloat16, capacity_factor=1.25)
    base.update(kw)
    return moe.route_desc(**base)


def test_capacity_and_max_rows():
    lib = moe.load()
    assert moe.moe_route_capacity(_desc()) == 160
    assert moe.moe_max_rows(_desc()) == 8192                        # min(T*K, E*cap)
    assert moe.moe_max_rows(_desc(capacity_factor=0.5)) == 64 * 64  # cap 64
    assert moe.moe_route_capacity(_desc(capacity_factor=0.0)) == -1
    assert moe.moe_max_rows(_desc(K=8, E=256, capacity_factor=0.0)) == 8192 * 8
    # capacity reaching T means nothing can drop
    assert moe.moe_route_capacity(_desc(capacity_factor=100.0)) == -1
    assert moe.moe_route_capacity(_desc(capacity_factor=0.5, min_capacity=100)) == 100
    d = _desc()
    assert lib.moe_route_workspace_size(ctypes.byref(d)) > 0


def _status(fn, *args):
    st = getattr(moe.load(), fn)(*args)
    msg = moe.load().moe_last_error().decode()
    return st, msg


@pytest.mark.parametrize("kw,code", [
    (dict(K=65, E=128), _lib.MOE_ERR_ARG),
    (dict(K=3, E=2), _lib.MOE_ERR_ARG),
    (dict(E=0), _lib.MOE_ERR_ARG),
    (dict(E=2000), _lib.MOE_ERR_ARG),
    (dict(h=12), _lib.MOE_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.MOE_ERR_ARG),
])
def test_route_rejects_bad_desc(kw, code):
    d = _desc(**kw)
    st, msg = _status("moe_route", ctypes.byref(d), *([None] * 10), None, 0, None)
    assert st == code and msg.startswith("moe_route")


def test_route_requires_outputs_and_workspace():
    d = _desc()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    st, msg = _status("moe_route", ctypes.byref(d), p, p, None, None, None, None, None,
                      None, None, None, None, 0, None)
    assert st == _lib.MOE_ERR_ARG and "required" in msg
    st, msg = _status("moe_route", ctypes.byref(d), p, p, None, None, None, None, None,
                      None, None, p, p, 1 << 30, None)
    assert st == _lib.MOE_ERR_ARG and "required" in msg
    st, msg = _status("moe_route", ctypes.byref(d), p, p, None, None, None, None, None,
                      p, p, p, None, 0, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    st, msg = _status("moe_route", ctypes.byref(d), p, p, None, p, None, None, None,
                      p, p, p, p, 1 << 30, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "sigmoid" in msg  # expert_bias with softmax


def test_permute_combine_mlp_reject_bad_sizes():
    p = ctypes.c_void_p(16)
    st, _ = _status("moe_permute", 10, 12, 4, 2, _lib.MOE_BF16, p, p, p, 20, p, p, p, p, p, p,
                    1 << 20, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED  # h % 8
    st, _ = _status("moe_permute", 10, 16, 4, 5, _lib.MOE_BF16, p, p, p, 20, p, p, p, p, p, p,
                    1 << 20, None)
    assert st == _lib.MOE_ERR_ARG  # K > E
    st, _ = _status("moe_permute", 10, 16, 4, 2, _lib.MOE_BF16, p, p, p, 20, p, p, p, p, p, p,
                    0, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    st, _ = _status("moe_combine", 10, 12, 2, _lib.MOE_BF16, p, p, p, 20, None, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED
    st, _ = _status("moe_combine", 10, 16, 0, _lib.MOE_BF16, p, p, p, 20, None, p, None)
    assert st == _lib.MOE_ERR_ARG
    st, msg = _status("moe_grouped_mlp", 8, 100, 256, 64, _lib.MOE_BF16, p, p, p, p, p, p, p, None,
                      None)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "multiples of 64" in msg
    st, _ = _status("moe_grouped_fc2", 0, 128, 256, 64, _lib.MOE_BF16, p, p, p, p, None, None)
    assert st == _lib.MOE_ERR_ARG
    st, _ = _status("moe_grouped_fc1_swiglu", 4, 64, 64, 8, 7, p, p, p, p, p, None, None)
    assert st == _lib.MOE_ERR_ARG  # dtype
    st, _ = _status("moe_grouped_fc1_swiglu", 4, 64, 64, 8, _lib.MOE_BF16, p, None, p, p, p, None,
                    None)
    assert st == _lib.MOE_ERR_ARG  # NULL counts


def test_mxfp8_entry_points_reject_bad_sizes():
    p = ctypes.c_void_p(16)
    st, _ = _status("moe_mxfp8_quantize", 4, 48, 0, _lib.MOE_BF16, p, p, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED  # cols % 32
    st, _ = _status("moe_mxfp8_quantize", 4, 96, 2, _lib.MOE_BF16, p, p, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED  # k-tiled: cols % 128
    st, _ = _status("moe_mxfp8_quantize", 6, 128, 4, _lib.MOE_BF16, p, p, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED  # k-tiled: rows % tile_rows
    st, _ = _status("moe_mxfp8_quantize", 4, 128, -1, _lib.MOE_BF16, p, p, p, None)
    assert st == _lib.MOE_ERR_ARG
    st, _ = _status("moe_mxfp8_quantize", 4, 128, 0, 7, p, p, p, None)
    assert st == _lib.MOE_ERR_ARG  # dtype
    st, _ = _status("moe_mxfp8_quantize", 4, 128, 0, _lib.MOE_BF16, None, p, p, None)
    assert st == _lib.MOE_ERR_ARG  # NULL source
    st, msg = _status("moe_grouped_fc1_swiglu_mxfp8", 4, 192, 256, 8, 8, p, p, None, p, p, p, p, p,
                      p, p, None, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "multiples of 128" in msg
    st, _ = _status("moe_grouped_fc1_swiglu_mxfp8", 0, 128, 128, 8, 8, p, p, None, p, p, p, p, p,
                    p, p, None, None)
    assert st == _lib.MOE_ERR_ARG  # E
    st, _ = _status("moe_grouped_fc1_swiglu_mxfp8", 4, 128, 128, 8, 8, p, p, None, None, p, p, p, p,
                    p, p, None, None)
    assert st == _lib.MOE_ERR_ARG  # NULL counts
    st, _ = _status("moe_grouped_fc2_mxfp8", 4, 128, 320, 8, p, p, p, p, p, p, None, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED  # f % 128
    st, _ = _status("moe_grouped_fc2_mxfp8", 4, 128, 128, 8, p, p, p, p, p, None, None, None)
    assert st == _lib.MOE_ERR_ARG  # NULL output


def test_mxfp8_shared_entry_points_validate_before_launching():
    p = ctypes.c_void_p(16)
    # fc1: E, h, f, max_rows, T, x codes/scales, sorted_token, counts, wg, wu (codes, scales),
    # act (codes, scales), fs, sg, su (codes, scales), shared act (codes, scales), queue, stream
    def fc1(fs=128, sorted_token=p, shared_act=p, T=8):
        return _status("moe_grouped_fc1_swiglu_mxfp8_shared", 4, 128, 128, 8, T, p, p, sorted_token,
                       p, p, p, p, p, p, p, fs, p, p, p, p, shared_act, p, None, None)
    st, msg = fc1(fs=192)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "multiples of 128" in msg  # the shared ffn
    st, msg = fc1(sorted_token=None)
    assert st == _lib.MOE_ERR_ARG and "sorted_token" in msg
    st, _ = fc1(shared_act=None)
    assert st == _lib.MOE_ERR_ARG
    st, _ = fc1(T=-1)
    assert st == _lib.MOE_ERR_ARG
    assert fc1(T=0)[0] == 0  # no tokens: a no-op

    # fc2: E, h, f, max_rows, act (codes, scales), counts, wd (codes, scales), expert_out, T, fs,
    # shared act (codes, scales), sd (codes, scales), shared_out, queue, stream
    def fc2(fs=128, shared_out=p, T=8):
        return _status("moe_grouped_fc2_mxfp8_shared", 4, 128, 128, 8, p, p, p, p, p, p, T, fs, p,
                       p, p, p, shared_out, None, None)
    st, msg = fc2(fs=64)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "multiples of 128" in msg
    st, _ = fc2(shared_out=None)
    assert st == _lib.MOE_ERR_ARG
    assert fc2(T=0)[0] == 0


def test_wrapper_rejects_cpu_tensors():
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        moe.moe_route(x, torch.zeros(2, 8), K=1)


def test_product_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "combine_router_gating_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f


def test_max_rows_with_padding_to_capacity():
    d = _desc(capacity_factor=0.5, pad_to_capacity=True)          # cap 64 < T
    assert moe.moe_max_rows(d) == 64 * 64
    d = _desc(capacity_factor=100.0, pad_to_capacity=True)        # cap >= T: every pair
    assert moe.moe_max_rows(d) == 8192 * 64
    d = _desc(capacity_factor=0.0, pad_to_capacity=True)          # dropless: no padding
    assert moe.moe_max_rows(d) == 8192


def test_route_rejects_bad_policy_and_score():
    d = _desc()
    d.drop_policy = 5
    st, msg = _status("moe_route", ctypes.byref(d), *([None] * 10), None, 0, None)
    assert st == _lib.MOE_ERR_ARG and "drop_policy" in msg
    d = _desc()
    d.score = 3
    st, msg = _status("moe_route", ctypes.byref(d), *([None] * 10), None, 0, None)
    assert st == _lib.MOE_ERR_ARG and "score" in msg
    with pytest.raises(ValueError):
        moe.route_desc(8, 8, 4, 1, torch.float32, score="tanh")
    with pytest.raises(ValueError):
        moe.route_desc(8, 8, 4, 1, torch.float32, drop_policy="random")


def test_side_output_entry_points_reject_bad_arguments():
    p = ctypes.c_void_p(16)
    st, _ = _status("moe_router_aux_loss", 10, 0, 1, 0, p, p, p, p, 1 << 20, None)
    assert st == _lib.MOE_ERR_ARG                                   # E = 0
    st, _ = _status("moe_router_aux_loss", 10, 4, 5, 0, p, p, p, p, 1 << 20, None)
    assert st == _lib.MOE_ERR_ARG                                   # K > E
    st, _ = _status("moe_router_aux_loss", 10, 4, 2, 9, p, p, p, p, 1 << 20, None)
    assert st == _lib.MOE_ERR_ARG                                   # score
    st, _ = _status("moe_router_aux_loss", 10, 4, 2, 0, p, p, None, p, 1 << 20, None)
    assert st == _lib.MOE_ERR_ARG                                   # no output
    st, _ = _status("moe_router_aux_loss", 100, 4, 2, 0, p, p, p, p, 4, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    assert moe.load().moe_aux_loss_workspace_size(100, 4) >= 2 * 4 * 4
    st, _ = _status("moe_accumulate_tokens_per_expert", 0, p, p, None)
    assert st == _lib.MOE_ERR_ARG
    st, _ = _status("moe_accumulate_tokens_per_expert", 4, None, p, None)
    assert st == _lib.MOE_ERR_ARG
    st, _ = _status("moe_update_expert_bias", 2000, p, p, ctypes.c_float(0.1), 1, None)
    assert st == _lib.MOE_ERR_ARG
    st, _ = _status("moe_update_expert_bias", 4, p, None, ctypes.c_float(0.1), 1, None)
    assert st == _lib.MOE_ERR_ARG


def test_fused_entry_points_reject_bad_arguments_before_launching():
    p = ctypes.c_void_p(16)
    big = 1 << 40
    d = _desc(K=65, E=128)
    st, _ = _status("moe_route_permute", ctypes.byref(d), *([None] * 10), 0, *([None] * 5), None,
                    0, None)
    assert st == _lib.MOE_ERR_ARG  # bad descriptor
    d = _desc()
    # route arguments complete, permute outputs missing: refused before any launch
    st, msg = _status("moe_route_permute", ctypes.byref(d), p, p, None, None, None, None, None,
                      p, p, p, 100, None, p, p, p, None, p, big, None)
    assert st == _lib.MOE_ERR_ARG and "expert_offsets" in msg
    st, msg = _status("moe_route_permute", ctypes.byref(d), p, p, None, None, None, None, None,
                      p, p, p, 100, p, p, p, p, p, p, 16, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    st, _ = _status("moe_grouped_fc2_combine", 8, 128, 256, 64, _lib.MOE_F32, 10, p, p, p, p, p, p,
                    p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED  # bf16 only
    st, _ = _status("moe_grouped_fc2_combine", 8, 128, 256, 64, _lib.MOE_BF16, -1, p, p, p, p, p,
                    p, p, None)
    assert st == _lib.MOE_ERR_ARG  # T
    st, _ = _status("moe_grouped_fc2_combine", 8, 128, 256, 64, _lib.MOE_BF16, 10, p, p, p, p, p,
                    None, p, None)
    assert st == _lib.MOE_ERR_ARG  # NULL row_id_map
    st, msg = _status("moe_grouped_fc2_combine", 8, 100, 256, 64, _lib.MOE_BF16, 10, p, p, p, p, p,
                      p, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "multiples of 64" in msg

    st, _ = _status("moe_grouped_fc2_combine_mxfp8", 8, 128, 256, 64, -1, p, p, p, p, p, p, p, p,
                    p, None)
    assert st == _lib.MOE_ERR_ARG  # T
    st, _ = _status("moe_grouped_fc2_combine_mxfp8", 8, 128, 256, 64, 10, p, p, p, p, p, p, p,
                    None, p, None)
    assert st == _lib.MOE_ERR_ARG  # NULL row_id_map
    st, _ = _status("moe_grouped_fc2_combine_mxfp8", 8, 128, 256, 64, 10, p, p, p, p, p, None, p,
                    p, p, None)
    assert st == _lib.MOE_ERR_ARG  # NULL probs with rows to combine
    st, msg = _status("moe_grouped_fc2_combine_mxfp8", 8, 192, 256, 64, 10, p, p, p, p, p, p, p,
                      p, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED and "multiples of 128" in msg


def test_noalloc_rejects_layers_beyond_the_static_scratch():
    """moe_route_permute_noalloc refuses, before any HIP call, a layer whose
    workspace exceeds the static scratch (T=65536, E=256 needs ~80 MiB)."""
    lib = moe.load()
    d = moe.route_desc(65536, 4096, 256, 8, torch.bfloat16, "sigmoid", True, 0.0, 0, "position",
                       False)
    need = int(lib.moe_route_permute_workspace_size(ctypes.byref(d)))
    assert need > _lib.MOE_NOALLOC_SCRATCH_BYTES
    st = lib.moe_route_permute_noalloc(ctypes.byref(d), *([None] * 10), 65536 * 8,
                                       *([None] * 5), None)
    assert st == _lib.MOE_ERR_UNSUPPORTED
    assert b"static scratch" in lib.moe_last_error()
    # the limit the header states is the one the library applies
    text = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in text
    assert _lib.MOE_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_clock_probe_rejects_bad_arguments_before_launching():
    """moe_clock_probe validates on the host: no launch for a null output or
    a spin outside (0, 1 s]."""
    lib = moe.load()
    out = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert lib.moe_clock_probe(None, 100, None) == 1
    assert lib.moe_clock_probe(out, 0, None) == 1
    assert lib.moe_clock_probe(out, 1000001, None) == 1
    assert b"spin_us" in lib.moe_last_error()
