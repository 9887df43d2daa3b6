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
