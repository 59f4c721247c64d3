"""Pins for the fp32 GELU of the fused FFN path (oracle/quant.py exp32,
gelu32): float64 references of e^z and of y * sigmoid(2u) (the tanh-form
GELU), special values, and the bf16 activation it feeds."""
import math

import numpy as np

from oracle import formats as F, quant as Q

ULP = 2.0 ** -24


def test_exp32_within_two_ulps():
    z = np.concatenate([np.linspace(-80, 88, 400001), [0.0, -0.0, 1.0, -1.0, 88.0]]).astype(np.float32)
    e = Q.exp32(z).astype(np.float64)
    ref = np.exp(z.astype(np.float64))
    assert np.max(np.abs(e - ref) / ref) <= 2 * ULP
    assert Q.exp32(np.float32(0.0)) == 1.0
    assert np.isinf(Q.exp32(np.float32(90.0)))          # overflows through the two exact scalings
    assert 0 < Q.exp32(np.float32(-80.0)) < 2e-35


def _gelu64(y):
    y = np.asarray(y, np.float64)
    u = math.sqrt(2 / math.pi) * (y + 0.044715 * y ** 3)
    with np.errstate(over="ignore"):
        return y / (1 + np.exp(-2 * u))


def test_gelu32_against_float64():
    y = np.linspace(-12, 12, 600001).astype(np.float32)
    g = Q.gelu32(y).astype(np.float64)
    ref = _gelu64(y)
    big = np.abs(ref) > 1e-6
    assert np.max(np.abs(g - ref)[big] / np.abs(ref[big])) <= 64 * ULP
    mid = np.abs(ref) > 1e-30
    assert np.max(np.abs(g - ref)[mid] / np.abs(ref[mid])) <= 256 * ULP
    assert np.max(np.abs(g - ref)[~mid]) < 1e-34


def test_gelu32_special_values():
    y = np.array([0.0, -0.0, 5.0, 40.0, 1e30, 3e38, -20.0, -1e30, -3e38, 1e-30, -1e-30], np.float32)
    g = Q.gelu32(y)
    assert g[0] == 0 and not np.signbit(g[0]) and g[1] == 0 and np.signbit(g[1])
    assert np.array_equal(g[2:6], y[2:6])                 # sigmoid rounds to 1
    assert np.all(g[6:9] == 0) and np.all(np.signbit(g[6:9]))
    assert g[9] == np.float32(5e-31) and g[10] == np.float32(-5e-31)   # y / 2 near zero


def test_gelu_activation_feeds_the_quantizer():
    rng = np.random.Generator(np.random.PCG64(44))
    x = F.f32_to_bf16(rng.standard_normal((8, 128)).astype(np.float32) * 3)
    r = Q.hadamard_quantize(x, 64, "mxfp4", gelu=True)
    g = F.f32_to_bf16(Q.gelu32(F.bf16_to_f32(x)))
    assert np.array_equal(r["q"], Q.hadamard_quantize(g, 64, "mxfp4")["q"])
    assert np.all(F.bf16_to_f32(g) >= -0.17)              # GELU's minimum is about -0.17
