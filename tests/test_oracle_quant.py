"""Pins for oracle/quant.py: hand-derived fixtures and the invariants the
encodings must satisfy on any input."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import formats as F, quant as Q, hadamard as H

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.Generator(np.random.PCG64(13))


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_nvfp4_hand_fixture():
    g = _load("nvfp4_hand_K48.json")
    y = np.array([[float(v) for v in g["y"]]], dtype=np.float32)
    q, s, (amax, gs) = Q.nvfp4_quantize(y)
    assert amax == np.float32(g["amax"]) and gs == np.float32(g["gs"])
    assert s.tolist() == [g["scales"]]
    assert F.unpack_nibbles(q).tolist() == [g["codes"]]


def test_int8_hand_fixture():
    g = _load("int8_hand.json")
    y = np.array(g["y"], dtype=np.float32)
    q, s = Q.int8_quantize(y)
    assert q.tolist() == g["q"]
    assert s.tolist() == g["scales"]


def _groups_with_normal_scale(s8):
    e = (s8.astype(np.int64) >> 3) & 0xF
    return e > 0


def test_nvfp4_invariants_tiny_config():
    d = synth.tiny_layer()
    y = H.block_hadamard_bf16(d["x"], 64)
    q, s8, (amax, gs) = Q.nvfp4_quantize(y)
    codes = F.unpack_nibbles(q).reshape(256, 16, 16)
    yg = y.reshape(256, 16, 16)
    assert amax == np.abs(y).max()
    # absmax element of every normal-scale group saturates the grid (code 7)
    arg = np.argmax(np.abs(yg), axis=-1)
    top = np.take_along_axis(codes, arg[..., None], -1)[..., 0]
    normal = _groups_with_normal_scale(s8)
    assert normal.any()
    assert np.all((top[normal] & 7) == 7)
    # dequantization error: within half a grid step at |v|, times the scale
    deq = Q.nvfp4_dequantize(q, s8, gs).reshape(256, 16, 16)
    sdec = (F.e4m3_to_float(s8) * float(gs))[..., None]
    v = np.abs(yg) / np.where(sdec == 0, 1, sdec)
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    err = np.abs(deq - yg)
    bound = half_step * sdec * (1 + 1e-6) + np.where(v > 6, (v - 6) * sdec, 0)
    assert np.all(err <= bound + 1e-30)
    # sign bits follow the input
    assert np.all(((codes & 8) > 0) == np.signbit(yg))


def test_nvfp4_zero_tensor_and_zero_groups():
    y = np.zeros((3, 32), np.float32)
    q, s, (amax, gs) = Q.nvfp4_quantize(y)
    assert amax == 0 and gs == 1 and not q.any() and not s.any()
    y[1, 16:] = RNG.standard_normal(16).astype(np.float32)
    q, s, _ = Q.nvfp4_quantize(y)
    assert s[0].tolist() == [0, 0] and s[1, 0] == 0 and s[1, 1] != 0
    assert not F.unpack_nibbles(q)[1, :16].any()


def test_nvfp4_given_amax_saturates():
    y = RNG.standard_normal((4, 64)).astype(np.float32)
    true = np.abs(y).max()
    q, s, (amax, gs) = Q.nvfp4_quantize(y, amax=true / 4)
    assert amax == np.float32(true / 4)
    # the group holding the true max needs a scale above 448: saturated
    r, c = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert s[r, c // 16] == 0x7E
    assert (F.unpack_nibbles(q)[r, c] & 7) == 7
    # non-finite or tiny given amax -> all zero
    for bad in (np.inf, np.nan, 0.0, -1.0, 2.0 ** -101):
        q, s, (_, gs) = Q.nvfp4_quantize(y, amax=bad)
        assert not q.any() and not s.any() and gs == 1


def test_nvfp4_subnormal_scales_and_underflow():
    # a tensor with one large group and one group 2^-16 smaller: the small
    # group's scale is subnormal in E4M3; a group 2^-20 smaller rounds to 0.
    y = np.zeros((1, 48), np.float32)
    y[0, 0] = 2688.0
    y[0, 16:32] = RNG.uniform(-1, 1, 16).astype(np.float32) * 2688 * 2.0 ** -16
    y[0, 32:48] = RNG.uniform(-1, 1, 16).astype(np.float32) * 2688 * 2.0 ** -20
    q, s, _ = Q.nvfp4_quantize(y)
    assert s[0, 0] == 0x7E
    assert 0 < s[0, 1] < 0x08            # subnormal E4M3
    assert s[0, 2] == 0 and not F.unpack_nibbles(q)[0, 32:].any()


def test_int8_invariants():
    y = (RNG.laplace(size=(50, 192)) * 3).astype(np.float32)
    y[7] = 0
    q, s = Q.int8_quantize(y)
    assert s[7] == 0 and not q[7].any()
    rows = np.arange(50) != 7
    a = np.abs(y).max(axis=1)
    assert np.all(s[rows] == (a[rows] / np.float32(127)).astype(np.float32))
    arg = np.argmax(np.abs(y), axis=1)
    assert np.all(np.abs(q[rows, arg[rows]]) == 127)
    err = np.abs(Q.int8_dequantize(q, s) - y)
    assert np.all(err[rows] <= (s[rows, None].astype(np.float64) * (0.5 + 1e-5)))
    assert q.min() >= -127


def test_activation_stats_closed_form():
    # constant-magnitude input: max|x| = mean|x|; b = 16 Hadamard of a
    # constant block is sqrt(16) * e_0, so max|y| = 4 and sum|y| = 4 per block
    x = np.full((2, 32), 1.0, np.float32)
    x[1] *= -1
    bits = F.f32_to_bf16(x)
    r = Q.hadamard_quantize(bits, 16, "int8")
    st = r["stats"]
    assert st[0] == 1.0 and st[1] == 64.0
    assert st[2] == 4.0 and st[3] == 4.0 * 4


def test_weight_prep_rotation_cancels():
    # X W^T equals (X H)(W H)^T: quantized W4A8 product stays close to the
    # bf16 product, which fails for a missing rotation on either side.
    from oracle import gemm as G
    d = synth.tiny_layer()
    x = F.bf16_to_f32(d["x"]).astype(np.float64)
    w = F.bf16_to_f32(d["w"]).astype(np.float64)
    ref = x @ w.T
    wq, ws, wgs = Q.prepare_weight(d["w"], 64)
    a = Q.hadamard_quantize(d["x"], 64, "int8")
    y64, _ = G.qgemm_w4a8(a["q"], a["scales"], wq, ws, wgs, out_dtype="f32")
    rel = np.linalg.norm(y64 - ref) / np.linalg.norm(ref)
    assert rel < 0.15, rel
    a4 = Q.hadamard_quantize(d["x"], 64, "nvfp4")
    y4, _ = G.qgemm_w4a4(a4["q"], a4["scales"], a4["gs"], wq, ws, wgs, out_dtype="f32")
    rel4 = np.linalg.norm(y4 - ref) / np.linalg.norm(ref)
    assert rel < rel4 < 0.3, (rel, rel4)
    # without the rotation on the activations the result is garbage
    a_bad = Q.int8_quantize(F.bf16_to_f32(d["x"]))
    yb, _ = G.qgemm_w4a8(a_bad[0], a_bad[1], wq, ws, wgs, out_dtype="f32")
    assert np.linalg.norm(yb - ref) / np.linalg.norm(ref) > 0.8


def test_bf16_fallback_is_rounded_transform():
    """The BF16 format is the transform output rounded to bf16: checked
    against torch's own bf16 cast of the oracle's fp32 transform."""
    import torch
    x = synth.laplace_activations(40, 256, 11, 12)
    for b in (16, 64, 128):
        r = Q.hadamard_quantize(x, b, "bf16")
        y = H.block_hadamard_bf16(x, b)
        want = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(r["q"], want)
        assert np.allclose(r["stats"], Q.activation_stats(x, y))
