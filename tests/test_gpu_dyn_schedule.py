"""Closed-loop schedule study (30 blocks x 50 steps) through the library:
block_stats on the GPU and dmpq_step in C, against the oracle's own loop.

Small tokens (M = 35, hidden 1920): the whole loop runs on both sides and
the 1500 actions must be identical, the statistics within 1e-5 relative
(maxima exact).  The oracle-side margins of every compared statistic to its
threshold are far above that tolerance for these seeds, so no decision can
flip on rounding.  Full size (M = 4446): the library's loop runs alone,
every action must occur, and the statistics and Delta_new of sampled
computed steps are checked against the oracle on the same operands."""
import numpy as np
import pytest

import synth
import video_diffusion_transformer_block_amd as V
from oracle import dmpq as OD, stats as OS
from helpers import host_bits, need_gpu, log
import dyn_loop

pytestmark = pytest.mark.gpu


def same_stats(got, want):
    got, want = np.asarray(got), np.asarray(want)
    assert got[4] == want[4] and got[6] == want[6], (got, want)
    assert np.allclose(got, want, rtol=1e-5, atol=0), (got, want)


def test_closed_loop_matches_oracle():
    need_gpu()
    w = synth.DynWorkload(M=35)
    p = dict(gamma=0.1, tau=0.05, tau_acc=0.15, rho=400.0)
    log("dyn loop M=35 oracle side")
    want_acts, want_stats = dyn_loop.oracle_loop(w, OD.Params(**p))
    assert set(np.unique(want_acts).tolist()) == {0, 1, 2, 3}
    log("dyn loop M=35 library side")
    got_acts, got_stats = dyn_loop.gpu_loop(w, V.dmpq_params(**p))
    bad = np.argwhere(got_acts != want_acts)
    assert len(bad) == 0, f"first differing (block, step): {bad[:5].tolist()}"
    assert set(got_stats) == set(want_stats)
    for k in want_stats:
        same_stats(got_stats[k], want_stats[k])


def test_closed_loop_budget_mode_matches_oracle():
    """Bit-budget mode (an average of 6 activation bits over the ranked
    blocks): each step's Gamma threshold is the k-th largest Gamma_{t-1},
    computed by the library in C and by the oracle; the 1500 actions match
    and NVFP4 and INT8 both occur."""
    need_gpu()
    w = synth.DynWorkload(M=35)
    p = dict(gamma=0.1, tau=0.05, tau_acc=0.15, rho=400.0)
    want_acts, _ = dyn_loop.oracle_loop(w, OD.Params(**p), budget=6.0)
    got_acts, _ = dyn_loop.gpu_loop(w, V.dmpq_params(**p), budget=6.0)
    bad = np.argwhere(got_acts != want_acts)
    assert len(bad) == 0, f"first differing (block, step): {bad[:5].tolist()}"
    counts = np.bincount(want_acts.ravel(), minlength=4)
    log(f"  budget mode actions skip/nvfp4/int8/bf16 = {counts.tolist()}")
    assert counts[1] > 0 and counts[2] > 0


def test_closed_loop_full_size_sampled():
    need_gpu()
    w = synth.DynWorkload()
    rng = np.random.Generator(np.random.PCG64(8000))
    sample = {(int(rng.integers(0, w.blocks)), int(rng.integers(0, w.steps))) for _ in range(24)}
    checked = []

    def on_sample(b, t, x, out, cache, dnew, s):
        dp = host_bits(cache) if cache is not None else None
        dn_o, s_o = OS.block_stats(host_bits(x), host_bits(out), dp)
        assert np.array_equal(host_bits(dnew), dn_o), (b, t)
        same_stats(s, s_o)
        checked.append((b, t))

    log(f"dyn loop M={w.M} library side, {len(sample)} sampled pairs")
    acts, stats = dyn_loop.gpu_loop(w, V.dmpq_params(gamma=0.1, tau=0.05, tau_acc=0.15, rho=1000.0),
                                    sample, on_sample)
    counts = np.bincount(acts.ravel(), minlength=4)
    log(f"  actions skip/nvfp4/int8/bf16 = {counts.tolist()}, checked {len(checked)}")
    assert (counts > 0).all()
    assert len(checked) >= 8


def _decision_margins(w, p, profile):
    """Oracle loop with every compared quantity's relative distance to its
    threshold: r_last vs tau_b (and acc + r vs tau_acc_b where r < tau_b),
    Gamma_{t-1} vs gamma, the outlier ratio vs rho."""
    import math
    mins = {"tau": math.inf, "tau_acc": math.inf, "gamma": math.inf, "rho": math.inf}

    def rec(b, t, a, ratio, pb, before, last):
        r, has_d2, acc, g, hg = before.r_last, before.has_d2, before.acc, before.gamma_prev, before.has_gamma
        if last is not None:
            g, hg = OS.gamma(last), True
            if before.has_d1:
                r = OS.delta_change(last)
            has_d2, acc = before.has_d1, 0.0
        if t >= pb.warmup and has_d2 and math.isfinite(r):
            mins["tau"] = min(mins["tau"], abs(r - pb.tau) / pb.tau)
            if r < pb.tau:
                mins["tau_acc"] = min(mins["tau_acc"], abs(acc + r - pb.tau_acc) / pb.tau_acc)
        if a != OD.SKIP:
            mins["rho"] = min(mins["rho"], abs(ratio - pb.rho) / pb.rho)
            if hg and math.isfinite(g):
                mins["gamma"] = min(mins["gamma"], abs(g - pb.gamma) / pb.gamma)

    acts, stats = dyn_loop.oracle_loop(w, p, record=rec, profile=profile)
    return acts, stats, mins


def test_closed_loop_depth_profile_matches_oracle():
    """Depth-aware caching thresholds: tau and tau_acc scaled from 1/2 at the
    first block to 3/2 at the last (dmpq_depth_params in C, depth_params in
    the oracle).  Every compared statistic stays at least 1e-4 (relative)
    from its block's threshold on the oracle side, ten times the statistics
    tolerance, so the 1500 actions must be identical; the profile moves
    skips from the shallow third of the blocks to the deep third."""
    need_gpu()
    w = synth.DynWorkload(M=35)
    p = dict(gamma=0.1, tau=0.05, tau_acc=0.15, rho=400.0)
    prof = (0.5, 1.5)
    want_acts, want_stats, mins = _decision_margins(w, OD.Params(**p), prof)
    log(f"  depth profile margins {mins}")
    assert min(mins.values()) >= 1e-4
    got_acts, got_stats = dyn_loop.gpu_loop(w, V.dmpq_params(**p), profile=prof)
    bad = np.argwhere(got_acts != want_acts)
    assert len(bad) == 0, f"first differing (block, step): {bad[:5].tolist()}"
    for k in want_stats:
        same_stats(got_stats[k], want_stats[k])
    counts = np.bincount(got_acts.ravel(), minlength=4)
    uni, _ = dyn_loop.oracle_loop(w, OD.Params(**p))
    third = w.blocks // 3
    sk = (got_acts == OD.SKIP).sum(1)
    sk_u = (uni == OD.SKIP).sum(1)
    log(f"  depth profile actions skip/nvfp4/int8/bf16 = {counts.tolist()}; skips by depth third "
        f"{[int(sk[:third].sum()), int(sk[third:2 * third].sum()), int(sk[2 * third:].sum())]} (uniform "
        f"{[int(sk_u[:third].sum()), int(sk_u[third:2 * third].sum()), int(sk_u[2 * third:].sum())]})")
    assert (counts > 0).all()
    assert sk[:third].sum() < sk_u[:third].sum() and sk[2 * third:].sum() > sk_u[2 * third:].sum()
