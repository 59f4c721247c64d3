"""Pins for oracle/formats.py against the format definitions and library casts."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

RNG = np.random.Generator(np.random.PCG64(11))


def test_bf16_rne_matches_torch():
    x = np.concatenate([
        RNG.standard_normal(200000).astype(np.float32) * 10,
        RNG.standard_normal(1000).astype(np.float32) * 1e-38,
        # exact ties: low 16 bits == 0x8000 around even and odd kept mantissas
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        ((np.arange(1000, dtype=np.uint32) + 0x3F800000) & 0xFFFF0000 | 0x8000).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16(x), ref)
    back = F.bf16_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_e4m3_decode_all_bytes_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = F.e4m3_to_float(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert F.e4m3_to_float(np.array([0x7E]))[0] == 448.0
    assert F.e4m3_to_float(np.array([0x01]))[0] == 2.0 ** -9
    assert F.e4m3_to_float(np.array([0x08]))[0] == 2.0 ** -6


def _e4m3_grid_points():
    pos = F.e4m3_to_float(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2
    pts = np.concatenate([pos, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    return np.concatenate([pts, up, dn])


def test_e4m3_encode_matches_torch_in_range():
    # torch's cast is RNE but not saturating; compare where both agree in
    # definition (|v| < 464, the midpoint between 448 and the NaN code).
    x = np.concatenate([_e4m3_grid_points(),
                        np.abs(RNG.standard_normal(200000)).astype(np.float32) * 50,
                        np.abs(RNG.standard_normal(20000)).astype(np.float32) * 1e-3])
    x = x[(x < 464) & (x >= 0)]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.float_to_e4m3(x), ref)


def test_e4m3_encode_saturates():
    x = np.array([448, 449, 463.9, 464, 480, 1e4, 3e38], dtype=np.float32)
    assert np.all(F.float_to_e4m3(x) == 0x7E)
    assert np.all(F.float_to_e4m3(-x) == 0xFE)


def test_e4m3_encode_brute_force_exact():
    # exact rational nearest search with ties to the even code
    pos = [Fraction(float(v)) for v in F.e4m3_to_float(np.arange(0x7F))]
    x = np.concatenate([_e4m3_grid_points()[::7],
                        np.abs(RNG.standard_normal(300)).astype(np.float32)])
    for v in x:
        fv = min(Fraction(float(v)), Fraction(448))
        best = min(range(0x7F), key=lambda c: (abs(pos[c] - fv), c % 2))
        assert F.float_to_e4m3(np.array([v]))[0] == best, v


E2M1_DEF = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def test_e2m1_decode_table():
    for c in range(16):
        mag = E2M1_DEF[c & 7]
        v = F.e2m1_to_float(np.array([c]))[0]
        assert v == (-mag if c & 8 else mag)
        assert np.signbit(v) == bool(c & 8)


def _e2m1_by_interval(a):
    # the round-to-nearest-even decision table written as intervals
    if a <= 0.25: return 0
    if a < 0.75: return 1
    if a <= 1.25: return 2
    if a < 1.75: return 3
    if a <= 2.5: return 4
    if a < 3.5: return 5
    if a <= 5.0: return 6
    return 7


def test_e2m1_encode_interval_table():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0, .5, 1, 1.5, 2, 3, 4, 6, 7, 100, 1e30],
                    dtype=np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                          np.nextafter(mids, np.float32(0)),
                          np.abs(RNG.standard_normal(1000000)).astype(np.float32) * 3,
                          np.abs(RNG.standard_normal(10000)).astype(np.float32) * 1e-3])
    got = F.float_to_e2m1(pts)
    want = np.array([_e2m1_by_interval(float(a)) for a in pts], dtype=np.uint8)
    assert np.array_equal(got, want)
    neg = F.float_to_e2m1(-pts)
    assert np.array_equal(neg, want | 8)
    assert F.float_to_e2m1(np.array([-0.0], np.float32))[0] == 8
    assert F.float_to_e2m1(np.array([np.inf], np.float32))[0] == 7


def test_nibble_order():
    assert F.pack_nibbles(np.array([[1, 2, 0xF, 0]], np.uint8)).tolist() == [[0x21, 0x0F]]
    c = RNG.integers(0, 16, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)
