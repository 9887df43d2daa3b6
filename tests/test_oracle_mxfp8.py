"""Pins of the oracle's MXFP8 quantisation and FP8 expert MLP against a
library routine (torch's float8_e4m3fn conversion), a hand-derived block
(tests/golden/mxfp8_worked.json), closed forms and error bounds."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mx, swiglu_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_rounding_matches_torch_float8():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * 60, rng.standard_normal(20000) * 1e-2,
                        np.linspace(-448, 448, 20001), [0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11,
                                                        2.0 ** -7 * 1.0625, 240.0 + 8.0]])
    v = v[np.abs(v) <= 448].astype(np.float32).astype(np.float64)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(mx.e4m3_round(v), t.to(torch.float64).numpy())
    np.testing.assert_array_equal(mx.e4m3_bits(mx.e4m3_round(v)), t.view(torch.uint8).numpy())


def test_e4m3_saturates_and_codes_roundtrip():
    assert mx.e4m3_round(np.array([460.0, 470.0, 1e6, -1e6])).tolist() == [448.0, 448.0, 448.0, -448.0]
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7f) != 0x7f]                       # drop the NaN codes
    vals = mx.e4m3_value(codes)
    np.testing.assert_array_equal(mx.e4m3_bits(vals)[vals != 0], codes[vals != 0])
    assert np.unique(np.abs(vals)).size == 127                   # 0 and 126 magnitudes


def test_mx_block_worked():
    g = json.load(open(os.path.join(GOLDEN, "mxfp8_worked.json")))
    v = np.zeros(32)
    v[:4] = g["values"]
    codes, scales = mx.mx_quantize(v)
    assert scales.tolist() == [g["scale_code"]]
    assert codes[:4].tolist() == g["codes"] and not codes[4:].any()
    np.testing.assert_array_equal(mx.mx_dequantize(codes, scales)[:4], g["dequantised"])


def test_mx_closed_forms():
    # all-zero block: smallest scale, zero codes
    c, s = mx.mx_quantize(np.zeros((3, 64)))
    assert not c.any() and (s == 0).all()
    # powers of two and small integers within 3 mantissa bits are exact
    rng = np.random.default_rng(1)
    p2 = np.ldexp(1.0, rng.integers(-20, 20, size=(5, 1)))
    v = rng.integers(-15, 16, size=(5, 96)).astype(np.float64) * p2
    v[:, ::32] = (16 * p2)[:, :1]   # block amax 16*2^s: X = 2^(s-4), every value a 4-bit integer * 16
    np.testing.assert_array_equal(mx.mx_roundtrip(v), v)
    # scale = 2^(floor(log2 amax) - 8): amax in [2^k, 2^(k+1))
    for k in (-30, -3, 0, 7, 40):
        b = np.full(32, 2.0 ** k * 1.3)
        _, s = mx.mx_quantize(b)
        assert int(s[0]) == k - 8 + 127


def test_mx_error_bound():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 3)
    r = mx.mx_roundtrip(v)
    b = v.reshape(64, 8, 32)
    amax = np.abs(b).max(-1, keepdims=True)
    X = np.ldexp(1.0, np.floor(np.log2(amax)).astype(int) - 8)
    scaled = np.abs(b) / X
    err = np.abs(r.reshape(64, 8, 32) - b) / X
    # not saturated: at most half an E4M3 step (step = 2^(e-3), or 2^-9 for subnormals)
    e = np.floor(np.log2(np.maximum(scaled, 2.0 ** -6)))
    half_step = np.ldexp(0.5, (e - 3).astype(int))
    ok = scaled <= 448
    assert (err[ok] <= half_step[ok] * (1 + 1e-12)).all()
    # saturated elements (scaled in (448, 512)) land on 448
    sat = ~ok
    assert sat.any()
    rs = np.abs(r.reshape(64, 8, 32)) / X
    assert (rs[sat] == 448.0).all()


def test_fp8_mlp_equals_exact_mlp_when_operands_are_representable():
    """Operands already MXFP8 values: the FP8 MLP's products are the exact
    products, so its y differs from the bf16-stored MLP only through the
    act quantisation, which is an MXFP8 roundtrip of the same act."""
    rng = np.random.default_rng(3)
    h, f = 64, 96
    x = mx.mx_roundtrip(rng.standard_normal((5, h)))
    wg = mx.mx_roundtrip(rng.standard_normal((f, h)) * 0.05)
    wu = mx.mx_roundtrip(rng.standard_normal((f, h)) * 0.05)
    wd = mx.mx_roundtrip(rng.standard_normal((h, f)) * 0.05)
    act_q, y = mx.swiglu_rows_mxfp8(x, wg, wu, wd)
    g, u = x @ wg.T, x @ wu.T
    act = g / (1 + np.exp(-g)) * u
    np.testing.assert_array_equal(act_q, mx.mx_roundtrip(act))
    from oracle import round_bf16
    np.testing.assert_array_equal(y, round_bf16(act_q @ wd.T))
    # and it stays close to the unquantised bf16 MLP (quantisation error only)
    _, y16 = swiglu_rows(x, wg, wu, wd, "f32")
    assert np.abs(y - y16).max() <= 0.1 * np.abs(y16).max()
