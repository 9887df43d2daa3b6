"""MXFP8 (OCP Microscaling) quantisation and the FP8 expert MLP.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name FP8 among the techniques of Megatron Core MoE training
("Scalable Training of Mixture-of-Experts Models with Megatron Core",
FP8/FP4 低精度训练: FP8 halves communication and activation storage and speeds
up the GEMMs; precision-critical paths stay in higher precision) but give
no scaling recipe.  Reading taken here: the OCP Microscaling (MX) v1.0
MXFP8-E4M3 format, which gfx950's scaled MFMA executes natively:

  * a block is 32 consecutive values along the reduction dimension;
  * the block's shared scale is a power of two X = 2^(floor(log2(amax)) - 8)
    stored as an E8M0 byte (exponent + 127; 8 is the exponent of E4M3's
    largest normal, 448 = 1.75 * 2^8), clamped to the E8M0 range; an
    all-zero block gets the smallest scale, 2^-127;
  * each element is V / X rounded to the nearest E4M3 value (ties to even),
    saturated to +-448.  E4M3 (OCP "E4M3FN"): sign, 4 exponent bits (bias
    7), 3 mantissa bits, subnormals 2^-6 * m/8, no infinities.

The FP8 expert MLP: x and the three weight matrices are MXFP8 with blocks
along h (W_gate, W_up, x) or f (W_down, act); g = dq(x) . dq(W_gate),
u = dq(x) . dq(W_up) exactly (float64 here), act = silu(g) * u, then act is
quantised to MXFP8 along f and y = dq(act) . dq(W_down), rounded once to
bf16.  The routing, permute and combine are the layer's usual ones.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal
E4M3_MIN_EXP = -6      # exponent of the smallest normal; subnormal step 2^-9
E8M0_BIAS = 127


def e4m3_round(v) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value, ties to even,
    saturating to +-448.  Returns float64 values (exactly representable)."""
    v = np.asarray(v, F64)
    a = np.abs(v)
    out = np.zeros_like(a)
    nz = a > 0
    _, ex = np.frexp(a[nz])                 # a = m * 2^ex, 0.5 <= m < 1
    e = np.maximum(ex - 1, E4M3_MIN_EXP)    # unbiased exponent (normals), subnormal floor
    q = np.ldexp(1.0, e - 3)                # quantum: 3 mantissa bits
    out[nz] = np.rint(a[nz] / q) * q        # np.rint: ties to even
    out = np.minimum(out, E4M3_MAX)
    return np.copysign(out, v)


def e4m3_bits(v) -> np.ndarray:
    """E4M3 code bytes of values that are already E4M3 (as e4m3_round returns)."""
    v = np.asarray(v, F64)
    a = np.abs(v)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    code = np.zeros(a.shape, np.uint8)
    nz = a > 0
    _, ex = np.frexp(a[nz])
    e = ex - 1
    sub = e < E4M3_MIN_EXP
    mant_norm = np.rint((a[nz] / np.ldexp(1.0, e) - 1.0) * 8).astype(np.int64)
    mant_sub = np.rint(a[nz] / np.ldexp(1.0, E4M3_MIN_EXP - 3)).astype(np.int64)
    c = np.where(sub, mant_sub, ((e + 7) << 3) | mant_norm)
    code[nz] = c.astype(np.uint8)
    return code | sign


def e4m3_value(code) -> np.ndarray:
    """float64 value of E4M3 code bytes (0x7f / 0xff, the NaN codes, are not produced)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, np.ldexp(m.astype(F64), E4M3_MIN_EXP - 3),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    return s * val


def mx_quantize(v, axis: int = -1):
    """MXFP8 of float64 values along `axis` (length a multiple of 32).

    Returns (codes uint8, same shape; scales uint8 E8M0, that axis / 32)."""
    v = np.moveaxis(np.asarray(v, F64), axis, -1)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("length along the blocked axis must be a multiple of 32")
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.abs(b).max(axis=-1)
    e = np.full(amax.shape, -E8M0_BIAS, np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])
    e[nz] = (ex - 1) - E4M3_EMAX            # floor(log2 amax) - 8
    e = np.clip(e, -E8M0_BIAS, E8M0_BIAS)
    X = np.ldexp(1.0, e)
    q = e4m3_round(b / X[..., None])
    codes = e4m3_bits(q).reshape(v.shape)
    scales = (e + E8M0_BIAS).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def mx_dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    c = np.moveaxis(np.asarray(codes, np.uint8), axis, -1)
    s = np.moveaxis(np.asarray(scales, np.uint8), axis, -1)
    vals = e4m3_value(c)
    X = np.ldexp(1.0, s.astype(np.int64) - E8M0_BIAS)
    out = vals.reshape(vals.shape[:-1] + (s.shape[-1], BLOCK)) * X[..., None]
    return np.moveaxis(out.reshape(vals.shape), -1, axis)


def mx_roundtrip(v, axis: int = -1) -> np.ndarray:
    """dq(q(v)): the values an MXFP8 operand holds."""
    return mx_dequantize(*mx_quantize(v, axis), axis)


def swiglu_rows_mxfp8(x_dq, wg_dq, wu_dq, wd_dq):
    """FP8 expert MLP on rows whose operands are already MXFP8 values
    (dequantised): returns (act as MXFP8 values, y rounded to bf16)."""
    from .moe import round_bf16
    g = np.asarray(x_dq, F64) @ np.asarray(wg_dq, F64).T
    u = np.asarray(x_dq, F64) @ np.asarray(wu_dq, F64).T
    with np.errstate(over="ignore"):
        act = g / (1.0 + np.exp(-g)) * u
    act_q = mx_roundtrip(act, axis=-1)
    y = round_bf16(act_q @ np.asarray(wd_dq, F64).T)
    return act_q, y
