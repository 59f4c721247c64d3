"""Pins for oracle/hadamard.py: closed forms of the Sylvester matrix, exact
agreement with a dense integer product, the butterfly order, and the scale."""
import numpy as np
import pytest

from oracle import hadamard as H

RNG = np.random.Generator(np.random.PCG64(12))


@pytest.mark.parametrize("b", H.VALID_BLOCKS)
def test_sylvester_orthogonal_symmetric_recursive(b):
    h = H.sylvester(b)
    assert np.array_equal(h @ h.T, b * np.eye(b, dtype=np.int64))
    assert np.array_equal(h, h.T)
    half = H.sylvester(b // 2) if b > 16 else None
    if half is not None:
        assert np.array_equal(h, np.block([[half, half], [half, -half]]))


@pytest.mark.parametrize("b", H.VALID_BLOCKS)
def test_fwht_equals_dense_product_on_small_integers(b):
    # small integers keep every partial sum exact in fp32
    x = RNG.integers(-50, 51, size=(7, 4 * b)).astype(np.int64)
    got = H.fwht_unscaled(x.astype(np.float32), b).astype(np.int64)
    h = H.sylvester(b)
    want = (x.reshape(7, 4, b) @ h).reshape(7, 4 * b)
    assert np.array_equal(got, want)
    # applying it twice gives b * x
    twice = H.fwht_unscaled(got.astype(np.float32), b).astype(np.int64)
    assert np.array_equal(twice, b * x)


@pytest.mark.parametrize("b", H.VALID_BLOCKS)
def test_orthonormal_energy_and_round_trip(b):
    x = RNG.standard_normal((16, 2 * b)).astype(np.float32)
    y = H.block_hadamard_f32(x, b)
    nx = np.linalg.norm(x.astype(np.float64), axis=1)
    ny = np.linalg.norm(y.astype(np.float64), axis=1)
    assert np.allclose(nx, ny, rtol=1e-6)
    back = H.block_hadamard_f32(y, b)
    assert np.allclose(back, x, rtol=0, atol=1e-5 * np.abs(x).max())


def test_butterfly_order_hand_example():
    # b = 16, x0 = 1, x1 = 2^-24, x2 = -2^-24.  Stage h=1 first rounds
    # 1 + 2^-24 to 1 (tie to even) and keeps x2 + x3 = -2^-24, so
    # y0 = (1 - 2^-24) / 4.  The exact sum (or stage h=2 first) would give 1/4.
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 1.0, 2.0 ** -24, -(2.0 ** -24)
    y = H.block_hadamard_f32(x, 16)
    assert y[0, 0] == np.float32((1 - 2.0 ** -24) / 4)
    assert y[0, 0] != np.float32(0.25)


def test_scale_constants():
    for b, e in ((16, 2), (64, 3), (256, 4)):
        f, exact = H.scale_factor(b)
        assert exact and f == np.float32(2.0 ** -e)
    # RN_fp32(sqrt 2) = 0x3FB504F3 (1.41421353816986083984375)
    for b, k in ((32, 3), (128, 4)):
        f, exact = H.scale_factor(b)
        assert not exact
        assert f.view(np.uint32) == np.uint32(0x3FB504F3 - (k << 23))
        assert f == np.float32(1 / np.sqrt(b))
        # within half an ulp of the exact value
        assert abs(float(f) - 1 / np.sqrt(b)) <= float(np.spacing(f)) / 2


def test_bf16_input_path():
    x = RNG.standard_normal((3, 64)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)        # truncation is fine here
    xt = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(H.block_hadamard_bf16(bits, 64), H.block_hadamard_f32(xt, 64))
