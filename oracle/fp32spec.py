"""A fixed fp32 evaluation of exp and of the logistic sigmoid.

Test infrastructure only (the oracle).  Product code never imports this.

Sigmoid scoring selects experts from fp32 scores plus an fp32 expert bias
(Megatron Core MoE 源码路径解析, §5 "Score function": the scores are the
sigmoid of the fp32 logits, the bias is added for the top-k choice only).
The page does not say how the fp32 sigmoid is evaluated, and two correct
implementations may differ in the last bit, which can flip a top-k choice.
So the oracle and the GPU each evaluate the same written-down sequence of
IEEE fp32 operations (every multiply, add and divide rounded to nearest
even, no fused multiply-add), and the selection is then bit-identical.

exp_spec(y), y <= 0:
  * y < -86: result 0 (keeps every nonzero result in the fp32 normal range);
  * n = rint(y * log2(e)), halves to even, log2(e) rounded to fp32;
  * Cody-Waite reduction r = (y - n*C1) - n*C2, where C1 is ln 2 cut to
    12 significant bits (so n*C1 is exact for |n| < 2^12) and C2 is the fp32
    value nearest to ln 2 - C1;
  * p = Horner evaluation of sum_{k=0..7} r^k / k!, each coefficient the
    fp32 value nearest to 1/k!;
  * result ldexp(p, n).
sigmoid_spec(x): a = |x|, e = exp_spec(-a); 1/(1+e) for x >= 0, else
e/(1+e).

The same page names a third score function, the square root of softplus,
which is used like the sigmoid (a bias may shift the choice; the probs are
the chosen scores normalised to sum 1).  It gets the same treatment:
log1p_spec(u), 0 <= u <= 1:
  * s = u / (2 + u)  (so 1 + u = (1 + s) / (1 - s) and log1p(u) = 2 atanh(s),
    with 0 <= s <= 1/3);
  * q = Horner evaluation of sum_{j=0..7} s2^j / (2j + 1), s2 = s*s, each
    coefficient the fp32 value nearest to 1/(2j+1);
  * result (2*s) * q.
softplus_spec(x): x itself when x > 20 (the usual threshold above which
softplus(x) and x agree in fp32); otherwise max(x, 0) + log1p_spec(e) with
e = exp_spec(-|x|).
sqrtsoftplus_spec(x): the correctly rounded fp32 square root of
softplus_spec(x).

The constants are derived here from the mathematics (math.log, factorials).
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
_LOG2E = F32(1.0 / math.log(2.0))
_C1 = F32(math.floor(math.log(2.0) * 4096.0) / 4096.0)
_C2 = F32(math.log(2.0) - float(_C1))
_TAYLOR = [F32(1.0 / math.factorial(k)) for k in range(8)]
_EXP_FLOOR = F32(-86.0)
_ATANH = [F32(1.0 / (2 * j + 1)) for j in range(8)]
_SOFTPLUS_LINEAR = F32(20.0)


def exp_spec(y: np.ndarray) -> np.ndarray:
    """exp(y) for fp32 y <= 0, by the fixed operation sequence above."""
    y = np.asarray(y, dtype=F32)
    n = np.rint(y * _LOG2E)                       # fp32 multiply, round half even
    r = (y - n * _C1) - n * _C2                   # each op rounded separately
    p = np.full_like(r, _TAYLOR[7])
    for k in range(6, -1, -1):
        p = p * r + _TAYLOR[k]                    # multiply, then add: no fma
    out = np.ldexp(p, n.astype(np.int32)).astype(F32)
    return np.where(y < _EXP_FLOOR, F32(0.0), out).astype(F32)


def sigmoid_spec(x: np.ndarray) -> np.ndarray:
    """Logistic sigmoid of fp32 x by the fixed operation sequence above."""
    x = np.asarray(x, dtype=F32)
    e = exp_spec(-np.abs(x))
    one = F32(1.0)
    den = one + e
    pos = one / den
    neg = e / den
    return np.where(x >= F32(0.0), pos, neg).astype(F32)


def log1p_spec(u: np.ndarray) -> np.ndarray:
    """log(1 + u) for fp32 u in [0, 1], by the fixed operation sequence above."""
    u = np.asarray(u, dtype=F32)
    s = u / (F32(2.0) + u)
    s2 = s * s
    q = np.full_like(s, _ATANH[7])
    for j in range(6, -1, -1):
        q = q * s2 + _ATANH[j]                    # multiply, then add: no fma
    return ((F32(2.0) * s) * q).astype(F32)


def softplus_spec(x: np.ndarray) -> np.ndarray:
    """softplus(x) = log(1 + e^x) of fp32 x by the fixed sequence above."""
    x = np.asarray(x, dtype=F32)
    e = exp_spec(-np.abs(x))
    body = np.maximum(x, F32(0.0)) + log1p_spec(e)
    return np.where(x > _SOFTPLUS_LINEAR, x, body).astype(F32)


def sqrtsoftplus_spec(x: np.ndarray) -> np.ndarray:
    """sqrt(softplus(x)) of fp32 x: softplus_spec, then an IEEE square root."""
    return np.sqrt(softplus_spec(x)).astype(F32)
