"""Pins for oracle/dmpq.py: hand-derived decision sequences."""
import json
import math
import os

import numpy as np

from oracle import dmpq as D

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load_sequence():
    with open(os.path.join(GOLD, "dmpq_sequence.json")) as f:
        return json.load(f)


def test_hand_sequence():
    g = load_sequence()
    p = D.Params(**g["params"])
    s = D.State()
    got = []
    for name, ratio, _ in g["calls"]:
        st = None if name is None else np.array(g["stats"][name])
        got.append(D.ACTION_NAMES[D.dmpq_step(p, s, st, ratio)])
    assert got == [c[2] for c in g["calls"]]


def test_constant_r_skip_run_length():
    # constant r < tau gives runs of exactly ceil(tau_acc / r) - 1 skips
    for r, tau_acc in ((0.01, 0.035), (0.02, 0.1), (0.03, 0.2)):
        p = D.Params(gamma=1.0, tau=0.05, tau_acc=tau_acc, rho=1e9, warmup=2)
        s = D.State()
        st = np.array([0.0, 1.0, r * r, 1.0, 1, 1, 1, 1])
        acts, last = [], None
        for t in range(60):
            a = D.dmpq_step(p, s, last, 1.0)
            acts.append(a)
            last = None if a == D.SKIP else st
        runs, cur = [], 0
        for a in acts[2:]:
            if a == D.SKIP:
                cur += 1
            elif cur:
                runs.append(cur)
                cur = 0
        want = math.ceil(tau_acc / r) - 1
        assert runs and all(x == want for x in runs), (r, tau_acc, runs, want)


def test_warmup_blocks_skips_and_ties():
    # binary-exact values so the ties are exact: Gamma = 0.125, r = 0.25
    p = D.Params(gamma=0.125, tau=0.25, tau_acc=4.0, rho=3.0, warmup=5)
    s = D.State()
    st = np.array([2.0 ** -6, 1.0, 2.0 ** -4, 1.0, 1, 1, 1, 1])
    acts = [D.dmpq_step(p, s, None if t == 0 else st, 3.0) for t in range(8)]
    # Gamma == gamma -> INT8 (tie), r == tau -> compute (tie), ratio == rho -> quantized
    assert acts[0] == D.INT8
    assert all(a == D.INT8 for a in acts[1:])
    acts = [D.dmpq_step(p, s, st, 3.0000001) for _ in range(2)]
    assert acts == [D.BF16, D.BF16]


# ---- bit-budget mode

def test_budget_gamma_closed_forms():
    g = [0.3, 0.05, 0.2, 0.01, 0.12, 0.07]          # sorted: .3 .2 .12 .07 .05 .01
    assert D.budget_gamma(g, 6.0) == 0.12            # k = 3: the three largest go INT8
    assert D.budget_gamma(g, 4.0) == math.inf        # k = 0: all NVFP4
    assert D.budget_gamma(g, 8.0) == 0.01            # k = 6: all INT8
    assert D.budget_gamma(g, 5.0) == 0.3             # k = floor(6 * 1 / 4) = 1: the largest
    assert D.budget_gamma(g, 3.0) == math.inf and D.budget_gamma(g, 9.0) == 0.01
    assert D.budget_gamma([], 6.0) == math.inf


def test_budget_gamma_meets_the_average():
    rng = np.random.Generator(np.random.PCG64(77))
    for trial in range(200):
        n = int(rng.integers(1, 60))
        g = rng.uniform(0, 0.3, n)
        bits = float(rng.uniform(4, 8))
        thr = D.budget_gamma(g, bits)
        int8 = int(np.sum(g >= thr))
        # distinct Gammas: exactly k INT8 blocks, and the average fits the budget
        assert int8 == max(0, min(n, int(np.floor(n * (bits - 4) / 4))))
        assert (8 * int8 + 4 * (n - int8)) / n <= bits + 1e-12


def test_budget_gamma_ties_take_int8():
    assert D.budget_gamma([0.1, 0.1, 0.1, 0.1], 6.0) == 0.1   # k = 2, all four tie -> all INT8


# ---- depth-aware caching thresholds

def _skip_runs(p, r, steps=80):
    """Skip run lengths of one block fed a constant delta change r."""
    s = D.State()
    st = np.array([0.0, 1.0, r * r, 1.0, 1, 1, 1, 1])
    acts, last = [], None
    for _ in range(steps):
        a = D.dmpq_step(p, s, last, 1.0)
        acts.append(a)
        last = None if a == D.SKIP else st
    runs, cur = [], 0
    for a in acts[2:]:
        if a == D.SKIP:
            cur += 1
        elif cur:
            runs.append(cur)
            cur = 0
    return runs


def test_depth_params_endpoints_and_midpoint_exact():
    base = D.Params(gamma=0.1, tau=0.05, tau_acc=0.15, rho=50.0, warmup=2)
    first = D.depth_params(base, 0, 30, 0.5, 1.5)
    last = D.depth_params(base, 29, 30, 0.5, 1.5)
    mid = D.depth_params(base, 2, 5, 0.5, 1.5)              # d = 1/2 exactly
    # halving and the 3/2 factor of dyadic steps: every value below is exact
    assert first.tau == 0.05 * 0.5 and first.tau_acc == 0.15 * 0.5
    assert last.tau == 0.05 * 1.5 and last.tau_acc == 0.15 * 1.5
    assert mid.tau == 0.05 and mid.tau_acc == 0.15
    for q in (first, last, mid):
        assert (q.gamma, q.rho, q.tau_u, q.warmup) == (base.gamma, base.rho, base.tau_u, base.warmup)
    # a single block sits at depth 0
    assert D.depth_params(base, 0, 1, 0.25, 4.0).tau == 0.05 * 0.25


def test_depth_params_unit_profile_is_the_uniform_scheduler():
    base = D.Params(gamma=0.07, tau=0.043, tau_acc=0.131, rho=12.5, tau_u=0.9, warmup=3)
    for depth in range(17):
        assert D.depth_params(base, depth, 17, 1.0, 1.0) == base


def test_depth_params_linear_and_monotone():
    base = D.Params(tau=2.0 ** -4, tau_acc=2.0 ** -3)
    n = 9                                                    # d = depth / 8, dyadic
    taus = [D.depth_params(base, k, n, 0.5, 2.5).tau for k in range(n)]
    assert taus == [2.0 ** -4 * (0.5 + 2.0 * k / 8) for k in range(n)]
    assert all(a < b for a, b in zip(taus, taus[1:]))
    down = [D.depth_params(base, k, n, 2.5, 0.5).tau for k in range(n)]
    assert down == taus[::-1]


def test_depth_profile_skip_runs_closed_form():
    """Constant r = 2^-7 under tau = 2^-4, tau_acc = 2^-3 (every sum exact):
    a block skips while (k + 1) r < tau_acc_b, i.e. runs of
    tau_acc_b / r - 1 skips: 7 at factor 1/2 (shallow end), 19 at 5/4 (the
    middle of nine blocks), 31 at 2 (deep end); factor 0 never skips."""
    base = D.Params(gamma=1.0, tau=2.0 ** -4, tau_acc=2.0 ** -3, rho=1e9, warmup=2)
    r = 2.0 ** -7
    want = {0: 7, 4: 19, 8: 31}                              # depths of n = 9: factors 1/2, 5/4, 2
    for depth, run in want.items():
        p = D.depth_params(base, depth, 9, 0.5, 2.0)
        s = 0.5 + 1.5 * depth / 8
        assert p.tau_acc == 2.0 ** -3 * s
        runs = _skip_runs(p, r)
        assert runs and all(x == run for x in runs), (depth, runs)
    assert _skip_runs(D.depth_params(base, 3, 9, 0.0, 0.0), r) == []


def test_depth_params_rejects():
    import pytest
    base = D.Params()
    for args in ((-1, 4, 1.0, 1.0), (4, 4, 1.0, 1.0), (0, 0, 1.0, 1.0), (0, 4, -0.5, 1.0),
                 (0, 4, 1.0, math.inf), (0, 4, math.nan, 1.0)):
        with pytest.raises(ValueError):
            D.depth_params(base, *args)
