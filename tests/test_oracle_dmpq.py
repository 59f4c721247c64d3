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
