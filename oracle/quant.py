"""Activation / weight quantization after the block Hadamard transform.

Test infrastructure only (see oracle/__init__.py).

[gist] §2.A: a stable block runs its linears with NVFP4 activations, a
volatile one with INT8; [yly] §一 says the same, likening NVFP4 to a low
flame and INT8 to a high one.  Neither page defines the encodings; the readings below are the
ones this project adopts, and the GPU path is bound to
them bit for bit.

NVFP4 (per tensor Y [M, K], K % 16 == 0):
  1. amax_T = max |Y| over the whole tensor (or a value the caller supplies).
     If amax_T is not finite or below 2^-100 the tensor is quantized to zero:
     gs = 1, every scale byte 0, every code 0.  (Below that level fp32 scales
     would turn subnormal; no bf16 activation of interest lives there.)
  2. gs = RN(amax_T / 2688)       (2688 = 6 * 448: largest E2M1 * largest E4M3)
  3. d  = RN(6 * gs)
  4. per 16-element group g:  a_g = max |y|;  s_raw = RN(a_g / d);
     s8 = E4M3(s_raw) (nearest-even, saturating at 448);
     s_dec = RN(e4m3(s8) * gs)
  5. s_dec == 0 -> the group's codes are 0.  Otherwise inv = RN(1 / s_dec)
     and each code is E2M1(RN(y * inv)) with y's sign bit.
  Codes are packed two per byte (even element in the low nibble), scales are
  one E4M3 byte per group in row-major [M, K/16] order, and the tensor scale
  pair is (amax_T, gs).  Dequantized value: e2m1(code) * e4m3(s8) * gs.
  (All "RN" are fp32 round-to-nearest-even.  Step 5 multiplies by the
  reciprocal of the group scale instead of dividing every element: one
  correctly rounded division per group, the same count as the scale itself.)

INT8 (per token row):
  a_m = max_k |y[m, k]|; rows with a_m not finite or below 2^-100 store
  scale 0 and all-zero codes.  Otherwise s_m = RN(a_m / 127),
  inv = RN(1 / s_m), q = clamp(rint_even(RN(y * inv)), -127, 127).
  Dequantized value: q * s_m.

MXFP4 / MXFP8 (the MX-native variant of the two activation formats; the
pages name NVFP4 as a Blackwell format, [gist] §2.A, and this variant keeps
the method on the block-scaled matrix instructions other hardware offers).
The encoding is the conversion of the OCP Microscaling Formats v1.0
specification (section 6.3), per block of 32 consecutive elements of a row
(K % 32 == 0):
  a = max |y| over the block (exact);
  e = floor(log2 a) - emax, emax = 2 for E2M1 elements, 8 for E4M3;
      clamped to [-127, 127]; a block of zeros takes e = -127;
  scale byte (E8M0) = e + 127;
  element = nearest-even encoding of y / 2^e (exact division by a power of
      two), saturating at the element format's largest finite value (6 or
      448), sign bit kept.
  Codes: E2M1 packed two per byte as for NVFP4; E4M3 one byte per element.
  Scales: one byte per block, row-major [M, K/32].  Dequantized value:
  element * 2^(byte - 127).  No tensor scale.

BF16 (the full-precision fallback of [gist] §2.C / [yly] §三):
  the rotated activations themselves, y rounded to bf16 (nearest even).  The
  weights exist only rotated, so the fallback multiplies rotated bf16
  activations by the dequantized 4-bit weights (W4A16).
"""
from __future__ import annotations

import math

import numpy as np

from .formats import (e2m1_to_float, e4m3_to_float, float_to_e2m1,
                      float_to_e4m3, pack_nibbles, unpack_nibbles, bf16_to_f32, f32_to_bf16)
from .hadamard import block_hadamard_f32

F32 = np.float32
GROUP = 16
MX_BLOCK = 32
MX_EMAX = {"e2m1": 2, "e4m3": 8}
ZERO_LIMIT = F32(2.0 ** -100)


def _amax_ok(a) -> bool:
    a = F32(a)
    return bool(np.isfinite(a) and a >= ZERO_LIMIT)


def nvfp4_quantize(y: np.ndarray, amax=None):
    """y: fp32 [M, K].  Returns (packed codes u8 [M, K/2], scales u8
    [M, K/16], (amax_T, gs) as float32)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    M, K = y.shape
    assert K % GROUP == 0
    if amax is None:
        amax_t = F32(np.max(np.abs(y))) if y.size else F32(0.0)
    else:
        amax_t = F32(amax)
    if M == 0 or not _amax_ok(amax_t):
        return (np.zeros((M, K // 2), np.uint8), np.zeros((M, K // GROUP), np.uint8),
                (amax_t, F32(1.0)))
    gs = F32(amax_t / F32(2688.0))
    d = F32(F32(6.0) * gs)
    yg = y.reshape(M, K // GROUP, GROUP)
    a_g = np.max(np.abs(yg), axis=-1)                       # exact
    s_raw = (a_g / d).astype(np.float32)                    # RN
    s8 = float_to_e4m3(s_raw)
    s_dec = (e4m3_to_float(s8).astype(np.float32) * gs).astype(np.float32)
    nz = s_dec != 0
    inv = np.where(nz, F32(1.0) / np.where(nz, s_dec, F32(1.0)), F32(0.0)).astype(np.float32)
    v = (yg * inv[..., None]).astype(np.float32)             # RN
    codes = float_to_e2m1(v)
    codes = np.where(nz[..., None], codes, np.uint8(0)).astype(np.uint8)
    return pack_nibbles(codes.reshape(M, K)), s8, (amax_t, gs)


def nvfp4_dequantize(packed: np.ndarray, scales: np.ndarray, gs=1.0) -> np.ndarray:
    """float64 [R, K] = e2m1(code) * e4m3(scale) * gs (exact in float64)."""
    codes = unpack_nibbles(packed)
    R, K = codes.shape
    vals = e2m1_to_float(codes).reshape(R, K // GROUP, GROUP)
    return (vals * e4m3_to_float(scales)[..., None]).reshape(R, K) * float(gs)


def int8_quantize(y: np.ndarray):
    """y: fp32 [M, K] -> (int8 codes [M, K], fp32 scales [M])."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    M, K = y.shape
    a = np.max(np.abs(y), axis=1) if K else np.zeros(M, np.float32)
    ok = np.isfinite(a) & (a >= ZERO_LIMIT)
    s = np.where(ok, (a / F32(127.0)).astype(np.float32), F32(0.0)).astype(np.float32)
    inv = np.where(ok, F32(1.0) / np.where(ok, s, F32(1.0)), F32(0.0)).astype(np.float32)
    v = (y * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(v), -127, 127).astype(np.int8)
    q[~ok] = 0
    return q, s


def int8_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return q.astype(np.float64) * s.astype(np.float64)[:, None]


def mx_quantize(y: np.ndarray, elem: str):
    """y: fp32 [M, K], K % 32 == 0; elem "e2m1" or "e4m3".  Returns (codes,
    E8M0 scale bytes u8 [M, K/32]): codes are packed E2M1 nibbles u8
    [M, K/2] or E4M3 bytes u8 [M, K]."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    M, K = y.shape
    assert K % MX_BLOCK == 0
    yb = y.astype(np.float64).reshape(M, K // MX_BLOCK, MX_BLOCK)
    a = np.max(np.abs(yb), axis=-1) if K else np.zeros((M, 0))
    # floor(log2 a) exactly: frexp gives a = f * 2^x with f in [0.5, 1)
    _, x = np.frexp(a)
    e = np.where(a > 0, x.astype(np.int64) - 1 - MX_EMAX[elem], -127)
    e = np.clip(e, -127, 127)
    t = yb / np.power(2.0, e)[..., None]                      # exact
    if elem == "e2m1":
        codes = pack_nibbles(float_to_e2m1(t).reshape(M, K))
    elif elem == "e4m3":
        codes = float_to_e4m3(t).reshape(M, K)
    else:
        raise ValueError(elem)
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, elem: str) -> np.ndarray:
    """float64 [R, K] = element value * 2^(scale byte - 127) (exact)."""
    if elem == "e2m1":
        vals = e2m1_to_float(unpack_nibbles(codes))
    elif elem == "e4m3":
        vals = e4m3_to_float(codes)
    else:
        raise ValueError(elem)
    R, K = vals.shape
    x = np.power(2.0, np.asarray(scales, dtype=np.int64) - 127)
    return (vals.reshape(R, K // MX_BLOCK, MX_BLOCK) * x[..., None]).reshape(R, K)


MX_ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}


# ---------------------------------------------------------------- GELU
# The DiT feed-forward applies GELU (tanh form) between FFN-up and FFN-down;
# fusing the FFN-down input quantization into FFN-up's epilogue puts it on
# this path.  The pages do not define it numerically; the reading here is an
# fp32 algorithm written out step by step, so that the GPU path can follow
# the same roundings (every step one fp32 operation, round to nearest even):
#   u = C0 * (y + C1 * ((y * y) * y))
#   z = clamp(-2 u, -80, 90)
#   GELU(y) = y / (1 + exp32(z))                    (= y * sigmoid(2u))
# with C0 = RN32(sqrt(2/pi)), C1 = RN32(0.044715).  exp32 is Cody-Waite range
# reduction, k = rint(z * RN32(1/ln 2)), r = (z - k ln2_hi) - k ln2_lo with
# ln2_hi = ln 2 truncated to 12 significant bits (k * ln2_hi is exact), the
# degree-7 Taylor polynomial of e^r in Horner form with coefficients
# RN32(1/n!), then two exact scalings by 2^floor(k/2) and 2^(k - floor(k/2)),
# so that z = 90 overflows to +inf (GELU -> -0 for large negative y) and
# z = -80 stays normal (GELU -> y for large positive y).
F32_C0 = np.float32(0.7978845608028654)
F32_C1 = np.float32(0.044715)
F32_LOG2E = np.float32(1.4426950408889634)
F32_LN2_HI = np.float32(0.693115234375)
F32_LN2_LO = np.float32(3.194618329871446e-05)
F32_TAYLOR = [np.float32(1.0 / math.factorial(n)) for n in range(8)]


def exp32(z: np.ndarray) -> np.ndarray:
    """e^z in fp32 by the steps above (z in [-80, 90])."""
    z = np.asarray(z, np.float32)
    k = np.rint((z * F32_LOG2E).astype(np.float32)).astype(np.float32)
    r = ((z - (k * F32_LN2_HI).astype(np.float32)).astype(np.float32) - (k * F32_LN2_LO).astype(np.float32)).astype(np.float32)
    p = F32_TAYLOR[7]
    for c in F32_TAYLOR[6::-1]:
        p = ((p * r).astype(np.float32) + c).astype(np.float32)
    ki = k.astype(np.int32)
    k1 = ki // 2                                     # floor
    with np.errstate(over="ignore"):
        return np.ldexp(np.ldexp(p, k1).astype(np.float32), ki - k1).astype(np.float32)


def gelu32(y: np.ndarray) -> np.ndarray:
    """GELU (tanh form) of fp32 values by the fp32 steps above."""
    y = np.asarray(y, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y3 = ((y * y).astype(np.float32) * y).astype(np.float32)
        w = (y + (F32_C1 * y3).astype(np.float32)).astype(np.float32)
        u = (F32_C0 * w).astype(np.float32)
        z = np.clip((np.float32(-2) * u).astype(np.float32), np.float32(-80), np.float32(90)).astype(np.float32)
        return (y / (np.float32(1) + exp32(z)).astype(np.float32)).astype(np.float32)


def activation_stats(x_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    """The outlier statistics fused into the quantize pass, in float64:
    [max|x|, sum|x|, max|y|, sum|y|] with x the bf16 input before the
    Hadamard transform and y after it.  The outlier ratio of [yly] §三 is
    max / (sum / n)."""
    x = np.abs(bf16_to_f32(x_bits).astype(np.float64))
    ya = np.abs(y.astype(np.float64))
    if x.size == 0:
        return np.zeros(4)
    return np.array([x.max(), x.sum(), ya.max(), ya.sum()])


def hadamard_quantize(x_bits: np.ndarray, had_block: int, fmt: str, amax=None, gelu: bool = False):
    """The full per-linear activation pass: block Hadamard of bf16 rows, then
    NVFP4 or INT8 quantization (or bf16 rounding for the full-precision
    fallback), plus the fused outlier statistics.
    fmt is "nvfp4", "int8", "bf16", "mxfp4" or "mxfp8".  gelu: the input is
    first mapped through gelu32 and rounded to bf16 (the FFN-down input as
    the model stores it); the statistics then describe that activation.
    Returns a dict."""
    if gelu:
        x_bits = f32_to_bf16(gelu32(bf16_to_f32(x_bits)))
    x = bf16_to_f32(x_bits)
    y = block_hadamard_f32(x, had_block)
    out = {"y": y, "stats": activation_stats(x_bits, y)}
    if fmt == "nvfp4":
        q, s, ts = nvfp4_quantize(y, amax)
        out.update(q=q, scales=s, amax=ts[0], gs=ts[1])
    elif fmt == "int8":
        q, s = int8_quantize(y)
        out.update(q=q, scales=s)
    elif fmt == "bf16":
        out.update(q=f32_to_bf16(y))
    elif fmt in MX_ELEM:
        q, s = mx_quantize(y, MX_ELEM[fmt])
        out.update(q=q, scales=s)
    else:
        raise ValueError(fmt)
    return out


def prepare_weight(w_bits: np.ndarray, had_block: int):
    """Offline weight preparation: W [N, K] is rotated along K by the same
    block Hadamard transform as the activations (so that the product of the
    two rotated operands equals X W^T, H being orthonormal and symmetric) and
    quantized to NVFP4 with its own tensor scale."""
    r = hadamard_quantize(w_bits, had_block, "nvfp4")
    return r["q"], r["scales"], r["gs"]


def prepare_weight_mx(w_bits: np.ndarray, had_block: int):
    """The MX variant of the weight preparation: the rotated weights in
    MXFP4 (E2M1 elements, one E8M0 scale per 32).  Returns (codes, scales)."""
    r = hadamard_quantize(w_bits, had_block, "mxfp4")
    return r["q"], r["scales"]
