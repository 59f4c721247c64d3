"""Per-block statistics the scheduler consumes.

Test infrastructure only (see oracle/__init__.py).

[gist] §2.A: Gamma_{t-1}, the relative input-output difference of a
transformer block at the previous step, predicts the quantization
sensitivity of its linears ([yly] §一 says the same).  [gist] §2.B: the
similarity of Delta_{t-1} and Delta_{t-2} (the residual deltas of the last
two computed steps) predicts whether the block can be skipped.  [yly] §三:
the outlier ratio, maximum over mean of the input, flags a step whose input
is hard to quantize.

Readings:
* Delta = out - in, computed in fp32 from the bf16 tensors and cached as
  bf16 (round to nearest even).
* Gamma = ||out - in||_F / ||in||_F over the block's whole [tokens, hidden]
  tensor; r = ||Delta_new - Delta_prev||_F / ||Delta_prev||_F over the stored
  bf16 deltas.  Edge cases: ||in|| = 0 gives Gamma = 0 when out == in and
  +inf otherwise; ||Delta_prev|| = 0 (or no previous delta) gives r = +inf.
* outlier ratio = max|x| / (sum|x| / n); an all-zero tensor has ratio 1.

block_stats returns eight float64 sums / maxima, in this order:
  [sum d^2, sum in^2, sum (Dnew - Dprev)^2, sum Dprev^2,
   max|in|, sum|in|, max|out|, sum|out|]

Low-precision delta cache ([yly] §七: the cache's extra memory can be
reduced by storing it in low precision).  block_stats_mx8 caches Delta in
MXFP8 (E4M3 elements, one E8M0 scale per 32 consecutive elements, the MX
conversion of oracle/quant.py) instead of bf16: Delta_new = MXFP8(d) with d
as above, and entries 2 and 3 use the dequantized stored deltas (what a
later step reads back).  The other six entries are unchanged.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16


def block_stats(in_bits, out_bits, dprev_bits=None):
    """Returns (Delta_new bf16 bits, stats float64[8])."""
    xi = bf16_to_f32(in_bits)
    xo = bf16_to_f32(out_bits)
    d = (xo - xi).astype(np.float32)                 # fp32 RN
    dnew = f32_to_bf16(d)
    d64 = d.astype(np.float64)
    i64 = xi.astype(np.float64)
    o64 = xo.astype(np.float64)
    st = np.zeros(8)
    if xi.size == 0:
        return dnew, st
    st[0] = np.sum(d64 * d64)
    st[1] = np.sum(i64 * i64)
    if dprev_bits is not None:
        dn = bf16_to_f32(dnew).astype(np.float64)
        dp = bf16_to_f32(dprev_bits).astype(np.float64)
        st[2] = np.sum((dn - dp) ** 2)
        st[3] = np.sum(dp * dp)
    st[4] = np.max(np.abs(i64))
    st[5] = np.sum(np.abs(i64))
    st[6] = np.max(np.abs(o64))
    st[7] = np.sum(np.abs(o64))
    return dnew, st


def block_stats_mx8(in_bits, out_bits, dprev=None):
    """dprev: None or (codes u8 [n], E8M0 scales u8 [n/32]) of the cached
    delta, n % 32 == 0.  Returns ((codes, scales) of Delta_new, stats
    float64[8])."""
    from .quant import mx_quantize, mx_dequantize
    xi = bf16_to_f32(in_bits).reshape(1, -1)
    xo = bf16_to_f32(out_bits).reshape(1, -1)
    n = xi.size
    assert n % 32 == 0
    d = (xo - xi).astype(np.float32)                 # fp32 RN
    q, sc = mx_quantize(d, "e4m3")
    st = np.zeros(8)
    if n == 0:
        return (q.reshape(-1), sc.reshape(-1)), st
    d64 = d.astype(np.float64)
    i64 = xi.astype(np.float64)
    o64 = xo.astype(np.float64)
    st[0] = np.sum(d64 * d64)
    st[1] = np.sum(i64 * i64)
    if dprev is not None:
        dn = mx_dequantize(q, sc, "e4m3")
        dp = mx_dequantize(np.asarray(dprev[0]).reshape(1, -1), np.asarray(dprev[1]).reshape(1, -1), "e4m3")
        st[2] = np.sum((dn - dp) ** 2)
        st[3] = np.sum(dp * dp)
    st[4] = np.max(np.abs(i64))
    st[5] = np.sum(np.abs(i64))
    st[6] = np.max(np.abs(o64))
    st[7] = np.sum(np.abs(o64))
    return (q.reshape(-1), sc.reshape(-1)), st


def gamma(st) -> float:
    num, den = float(st[0]), float(st[1])
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return math.sqrt(num / den)


def delta_change(st) -> float:
    num, den = float(st[2]), float(st[3])
    if den == 0.0:
        return math.inf
    return math.sqrt(num / den)


def outlier_ratio(max_abs: float, sum_abs: float, n: int) -> float:
    if sum_abs == 0.0 or n == 0:
        return 1.0
    return float(max_abs) / (float(sum_abs) / n)
