"""Pins for oracle/stats.py: closed forms on bf16-exact inputs."""
import math

import numpy as np

from oracle import formats as F, stats as S

RNG = np.random.Generator(np.random.PCG64(15))


def _bits(a):
    return F.f32_to_bf16(np.asarray(a, np.float32))


def test_gamma_closed_form():
    x = RNG.integers(-16, 17, size=(40, 96)).astype(np.float32) * 8
    out = x * np.float32(1.125)                  # out - in = in / 8 exactly
    dnew, st = S.block_stats(_bits(x), _bits(out))
    assert S.gamma(st) == 0.125
    assert np.array_equal(F.bf16_to_f32(dnew), x / 8)
    assert st[2] == 0 and st[3] == 0 and S.delta_change(st) == math.inf


def test_delta_change_closed_form():
    d = RNG.choice([-8.0, -4.0, 4.0, 8.0], size=(30, 64)).astype(np.float32)
    x = RNG.integers(-4, 5, size=(30, 64)).astype(np.float32) * 16
    dprev = d * np.float32(1.25)
    _, st = S.block_stats(_bits(x), _bits(x + d), _bits(dprev))
    assert abs(S.delta_change(st) - 0.2) < 1e-15


def test_outlier_ratio_closed_forms():
    n = 1000
    x = np.full(n, -3.0, np.float32)
    _, st = S.block_stats(_bits(x), _bits(x))
    assert S.outlier_ratio(st[4], st[5], n) == 1.0
    V = 512.0
    x = np.ones(n, np.float32)
    x[17] = V
    _, st = S.block_stats(_bits(x), _bits(x))
    assert abs(S.outlier_ratio(st[4], st[5], n) - V * n / (V + n - 1)) < 1e-12
    assert S.outlier_ratio(0.0, 0.0, n) == 1.0


def test_edge_cases():
    z = np.zeros(64, np.float32)
    _, st = S.block_stats(_bits(z), _bits(z), _bits(z))
    assert S.gamma(st) == 0.0 and S.delta_change(st) == math.inf
    _, st = S.block_stats(_bits(z), _bits(z + 1))
    assert S.gamma(st) == math.inf


def test_delta_rounding_and_sums():
    x = RNG.standard_normal(5000).astype(np.float32)
    o = RNG.standard_normal(5000).astype(np.float32)
    xb, ob = _bits(x), _bits(o)
    dnew, st = S.block_stats(xb, ob, None)
    xf, of = F.bf16_to_f32(xb), F.bf16_to_f32(ob)
    # fp32 subtraction of two bf16 values, then one RNE to bf16
    assert np.array_equal(dnew, F.f32_to_bf16(of - xf))
    assert math.isclose(st[0], float(np.sum((of - xf).astype(np.float64) ** 2)), rel_tol=1e-12)
    assert st[4] == np.abs(xf).max() and st[6] == np.abs(of).max()
    assert math.isclose(st[5], float(np.abs(xf.astype(np.float64)).sum()), rel_tol=1e-12)
