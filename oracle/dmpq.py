"""Per-block scheduler: dynamic precision (DMPQ), temporal delta cache (TDC),
purified delta refresh (PDR) and the restart rule.

Test infrastructure only (see oracle/__init__.py).

What the pages fix:
* [gist] §2.A / [yly] §一: low Gamma_{t-1} -> NVFP4, high -> INT8.
* [gist] §2.B / [yly] §二: skip the block and reuse the cached delta when
  Delta_{t-1} and Delta_{t-2} are similar; an error accumulator forces a full
  compute (cache refresh) once the accumulated drift passes a threshold.
* [gist] §2.C / [yly] §三: before a delta is written to the cache, outliers
  (max/mean of the input) or temporal uncertainty force full precision
  (FP16/BF16) for that step.
* [yly] §三: the first recompute after a skip has no previous difference to
  go on, so the whole block runs INT8.

Readings: one accumulator per block with its own
threshold tau_acc, reset on every compute; only computed deltas enter the
history; temporal uncertainty is read as r_last > tau_u (off by default);
ties: Gamma == gamma -> INT8, r == tau -> compute, ratio == rho -> quantized.

One call per block per denoising step:
  1. fold in the stats of the last step if it was computed;
  2. skip test;
  3. otherwise pick BF16 / INT8 / NVFP4.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

from .stats import gamma as _gamma, delta_change as _delta_change

SKIP, NVFP4, INT8, BF16 = 0, 1, 2, 3
ACTION_NAMES = {SKIP: "skip", NVFP4: "nvfp4", INT8: "int8", BF16: "bf16"}


@dataclass
class Params:
    gamma: float = 0.1       # Gamma threshold, NVFP4 below, INT8 at/above
    tau: float = 0.05        # skip when r < tau ...
    tau_acc: float = 0.15    # ... and the accumulated r stays below tau_acc
    rho: float = 50.0        # BF16 when the input outlier ratio exceeds rho
    tau_u: float = math.inf  # BF16 when r exceeds tau_u (temporal uncertainty)
    warmup: int = 2          # no skip before this step index


@dataclass
class State:
    step: int = 0
    has_d1: bool = False
    has_d2: bool = False
    skipped_last: bool = False
    has_gamma: bool = False
    gamma_prev: float = 0.0
    r_last: float = math.inf
    acc: float = 0.0


def dmpq_step(p: Params, s: State, last_stats, in_ratio: float) -> int:
    """last_stats: the 8 block statistics of the previous step if that step
    was computed, else None.  Mutates s and returns the action."""
    if last_stats is not None:
        s.gamma_prev = _gamma(last_stats)
        s.has_gamma = True
        if s.has_d1:
            s.r_last = _delta_change(last_stats)
        s.has_d2 = s.has_d1
        s.has_d1 = True
        s.skipped_last = False
        s.acc = 0.0
    t = s.step
    s.step += 1
    if (t >= p.warmup and s.has_d2 and s.r_last < p.tau
            and s.acc + s.r_last < p.tau_acc):
        s.acc += s.r_last
        s.skipped_last = True
        return SKIP
    if in_ratio > p.rho or (s.has_d2 and s.r_last > p.tau_u):
        return BF16
    if s.skipped_last or not s.has_gamma:
        return INT8
    if s.gamma_prev >= p.gamma:
        return INT8
    return NVFP4


def budget_gamma(gammas, avg_bits: float) -> float:
    """Bit-budget mode ([gist] §2.A / [yly] §一: Gamma_{t-1} ranks the blocks'
    sensitivity; [yly] §四: the W4A6 operating point averages 6 activation
    bits).  At the start of a step, rank the blocks by Gamma_{t-1} and give
    INT8 (8 bits) to the k most sensitive, NVFP4 (4 bits) to the rest, with
    k = floor(n * (avg_bits - 4) / 4) clamped to [0, n]: the threshold passed
    to dmpq_step as gamma is the k-th largest Gamma (+inf when k = 0).
    Ties at the boundary all take INT8 (Gamma == gamma -> INT8), so the INT8
    count can exceed k only by such ties.  Forced decisions (the restart
    INT8, BF16, skips) stay outside the budget."""
    g = sorted((float(x) for x in gammas), reverse=True)
    n = len(g)
    if n == 0 or not math.isfinite(avg_bits):
        return math.inf
    k = int(math.floor(n * (avg_bits - 4.0) / 4.0))
    k = max(0, min(n, k))
    return math.inf if k == 0 else g[k - 1]


def depth_params(p: Params, depth: int, n_blocks: int, s_shallow: float, s_deep: float) -> Params:
    """Depth-aware caching thresholds.  [yly] §五: blocks at different depths
    of the transformer show different temporal stability, which the page
    offers as the basis of a layered caching policy; it gives no formula.

    Reading: a block's two skip thresholds (tau and tau_acc) are the common
    ones scaled by a factor that moves linearly with the block's relative
    depth d = depth / (n_blocks - 1) (d = 0 for a single block), from
    s_shallow at the first block to s_deep at the last:
        s = s_shallow + (s_deep - s_shallow) * d
        tau_b = tau * s,  tau_acc_b = tau_acc * s
    in float64, in that order.  A factor above 1 lets a block skip more
    (and drift further before a refresh), below 1 less, 0 never.  The
    precision thresholds (gamma, rho, tau_u) and warmup are unchanged: the
    page ties depth to temporal redundancy only.  s_shallow = s_deep = 1 is
    the uniform scheduler."""
    if n_blocks <= 0 or not 0 <= depth < n_blocks:
        raise ValueError("depth outside [0, n_blocks)")
    for v in (s_shallow, s_deep):
        if not (math.isfinite(v) and v >= 0.0):
            raise ValueError("depth factors must be finite and >= 0")
    d = 0.0 if n_blocks == 1 else float(depth) / float(n_blocks - 1)
    s = s_shallow + (s_deep - s_shallow) * d
    return replace(p, tau=p.tau * s, tau_acc=p.tau_acc * s)
