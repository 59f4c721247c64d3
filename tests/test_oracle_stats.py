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


# ---- the low-precision (MXFP8) delta cache

def _mx8_exact(vals, e=0):
    """MXFP8 encoding of values exactly representable as e4m3 * 2^e, built
    with torch's E4M3 cast (independent of the oracle's encoder)."""
    import torch
    v = np.asarray(vals, np.float64).reshape(-1) / 2.0 ** e
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy(), v)
    return codes, np.full(v.size // 32, 127 + e, np.uint8)


def _mx8_values(codes, scales):
    import torch
    v = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(np.exp2(np.asarray(scales, np.float64) - 127), 32)


def test_mx8_cache_exact_delta_and_gamma():
    x = RNG.integers(-16, 17, size=(40, 96)).astype(np.float32) * 8
    # every 32-element block holds a +-16 delta, so its exponent is 4 - 8 and
    # every integer delta in [-16, 16] is an exact E4M3 value times 2^-4 (a
    # block whose largest delta were 15 would clip it: 15 * 2^5 > 448)
    x.reshape(-1)[::32] = 128
    out = x * np.float32(1.125)                  # out - in = in / 8: integers in [-16, 16]
    (q, sc), st = S.block_stats_mx8(_bits(x), _bits(out))
    assert q.shape == (40 * 96,) and sc.shape == (40 * 96 // 32,)
    assert np.array_equal(_mx8_values(q, sc), (x / 8).reshape(-1))
    assert S.gamma(st) == 0.125 and st[2] == 0 and st[3] == 0
    _, st16 = S.block_stats(_bits(x), _bits(out))
    assert np.array_equal(st[[0, 1, 4, 5, 6, 7]], st16[[0, 1, 4, 5, 6, 7]])


def test_mx8_cache_delta_change_closed_form():
    d = RNG.choice([-8.0, -4.0, 4.0, 8.0], size=(30, 64)).astype(np.float32)
    x = RNG.integers(-4, 5, size=(30, 64)).astype(np.float32) * 16
    prev = _mx8_exact(d * 1.25)                  # +-5, +-10: exact in E4M3
    _, st = S.block_stats_mx8(_bits(x), _bits(x + d), prev)
    assert abs(S.delta_change(st) - 0.2) < 1e-15


def test_mx8_cache_uses_stored_deltas():
    """d = 1 + 2^-5 is not an E4M3 value (3 mantissa bits): the stored delta
    rounds to 1, and the similarity terms are taken on the stored values."""
    n = 64
    x = np.zeros(n, np.float32)
    out = np.full(n, 1 + 2.0 ** -5, np.float32)
    (q, sc), st = S.block_stats_mx8(_bits(x), _bits(out), _mx8_exact(np.ones(n)))
    assert np.array_equal(_mx8_values(q, sc), np.ones(n))
    assert st[2] == 0.0 and st[3] == n
    assert st[0] == n * (1 + 2.0 ** -5) ** 2


def test_mx8_cache_halves_the_bytes():
    n = 4096
    x = RNG.standard_normal(n).astype(np.float32)
    (q, sc), _ = S.block_stats_mx8(_bits(x), _bits(x * np.float32(1.5)))
    assert q.nbytes + sc.nbytes == n + n // 32          # against 2n for bf16
