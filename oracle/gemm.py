"""Quantized GEMMs: W4A4 (NVFP4 x NVFP4), W4A8 (INT8 x NVFP4), the
full-precision fallback W4A16 (bf16 x NVFP4), and the MX-native variant
(MXFP4 or MXFP8 activations x MXFP4 weights).

Test infrastructure only (see oracle/__init__.py).

[gist] §2.A / §3.1 and [yly] §四: every linear keeps 4-bit weights (the W4A6 and
W4A8 operating points) and runs with NVFP4 or INT8 activations.  Both operands are already
rotated by the same block Hadamard transform along K, so the product is the
linear layer's output without further correction.

The oracle is the plain definition: dequantize both operands exactly in
float64, multiply (numpy matmul as the library primitive), apply the tensor /
token scales and the optional bias, then round once to the output type.

W4A4:  Y = gs_a * gs_w * (A_hat @ W_hat^T) + bias
W4A8:  Y = s_a[m] * gs_w * (Q_a @ W_hat^T) + bias
MX:    Y = A_hat @ W_hat^T + bias with A_hat, W_hat the MX dequantized
       operands (element * 2^(E8M0 - 127) per 32-element block)
W4A16: Y = gs_w * (A @ W_hat^T) + bias, A the rotated activations in bf16
       ([gist] §2.C: a step flagged by the outlier check runs in FP16/BF16;
       the weights stay 4-bit, [gist] §4 memory figure)
with A_hat = e2m1 * e4m3, W_hat likewise (no tensor scale), Q_a the int8
codes.  For W4A8 every product and partial sum is exact in float64 (at most
29 bits of dynamic range plus log2(K) bits of growth), so Q_a @ W_hat^T is
the exact integer-scaled accumulator.
"""
from __future__ import annotations

import numpy as np

from .formats import unpack_nibbles, f32_to_bf16
from .quant import nvfp4_dequantize, mx_dequantize, MX_ELEM, GROUP


def _finish(y64: np.ndarray, bias, out_dtype: str):
    if bias is not None:
        y64 = y64 + np.asarray(bias, dtype=np.float64)[None, :]
    y32 = y64.astype(np.float32)
    if out_dtype == "f32":
        return y64, y32
    if out_dtype == "bf16":
        return y64, f32_to_bf16(y32)
    raise ValueError(out_dtype)


def qgemm_w4a4(a_q, a_s, a_gs, w_q, w_s, w_gs, bias=None, out_dtype="bf16"):
    """Returns (exact float64 Y, Y rounded to out_dtype: fp32 values or bf16
    bits).  The rounding goes float64 -> fp32 -> bf16 (both nearest-even)."""
    A = nvfp4_dequantize(a_q, a_s)
    W = nvfp4_dequantize(w_q, w_s)
    y = (float(np.float32(a_gs)) * float(np.float32(w_gs))) * (A @ W.T)
    return _finish(y, bias, out_dtype)


def qgemm_w4a8(a_q, a_s, w_q, w_s, w_gs, bias=None, out_dtype="bf16"):
    W = nvfp4_dequantize(w_q, w_s)
    acc = np.asarray(a_q, dtype=np.float64) @ W.T
    y = (np.asarray(a_s, dtype=np.float64)[:, None] * float(np.float32(w_gs))) * acc
    return _finish(y, bias, out_dtype)


def qgemm_w4a16(a_bits, w_q, w_s, w_gs, bias=None, out_dtype="bf16"):
    """a_bits: bf16 bit patterns [M, K] of the rotated activations."""
    from .formats import bf16_to_f32
    A = bf16_to_f32(a_bits).astype(np.float64)
    W = nvfp4_dequantize(w_q, w_s)
    y = float(np.float32(w_gs)) * (A @ W.T)
    return _finish(y, bias, out_dtype)


def qgemm_mx(a_q, a_s, a_fmt, w_q, w_s, bias=None, out_dtype="bf16"):
    """a_fmt "mxfp4" (packed E2M1 codes [M, K/2]) or "mxfp8" (E4M3 bytes
    [M, K]); a_s, w_s E8M0 bytes [rows, K/32]; w_q packed E2M1 [N, K/2].
    Returns (float64 Y, Y rounded to out_dtype)."""
    A = mx_dequantize(a_q, a_s, MX_ELEM[a_fmt])
    W = mx_dequantize(w_q, w_s, "e2m1")
    return _finish(A @ W.T, bias, out_dtype)


def w4a8_integer_accumulator(a_q, w_q) -> np.ndarray:
    """Exact int64 P[m, n] = sum_k q_a[m, k] * c[n, k] with c = 2 * e2m1(w)
    in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}: the integer accumulator of the
    W4A8 product when every weight scale is 1 (so Y = P / 2)."""
    codes = unpack_nibbles(w_q).astype(np.int64)
    mag2 = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)[codes & 7]
    c = np.where(codes & 8, -mag2, mag2)
    return np.asarray(a_q, dtype=np.int64) @ c.T


def w4a8_group_partials(a_q, w_q) -> np.ndarray:
    """Exact int64 P_g[m, n, g] per 16-element K group (the quantity an
    integer MFMA would hold per group before the weight scale)."""
    codes = unpack_nibbles(w_q).astype(np.int64)
    mag2 = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)[codes & 7]
    c = np.where(codes & 8, -mag2, mag2)
    a = np.asarray(a_q, dtype=np.int64)
    M, K = a.shape
    N = c.shape[0]
    ag = a.reshape(M, K // GROUP, GROUP)
    cg = c.reshape(N, K // GROUP, GROUP)
    return np.einsum("mgk,ngk->mng", ag, cg)
