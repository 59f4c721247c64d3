"""Online block Hadamard transform.

Test infrastructure only (see oracle/__init__.py).

[gist] §2.A (DMPQ, the outlier-smoothing item) and [yly] §一: an online
block Hadamard transform spreads activation outliers over the block before
quantization.  The pages give no normalisation, order or block size; the
readings adopted here (binding on the GPU path too):

* H_b is the Sylvester Hadamard matrix, H_b[i][j] = (-1)^popcount(i & j);
  it is symmetric, so x·H_b = H_b·x per block.
* The transform is orthonormal: y = x · blockdiag(H_b) / sqrt(b) along each
  row, block by block (b consecutive elements, b a power of two in [16, 256]).
* fp32 rounding is pinned by a fixed butterfly order: for h = 1, 2, 4, ...,
  b/2 and every index i with (i & h) == 0, the pair (v_i, v_{i+h}) becomes
  (v_i + v_{i+h}, v_i - v_{i+h}), each rounded to fp32 (round to nearest
  even).  The scaling is then exact (v * 2^-log2(b)/2) when log2(b) is even,
  otherwise one fp32 multiply by c_b = RN_fp32(1/sqrt(b)).
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_to_f32

VALID_BLOCKS = (16, 32, 64, 128, 256)


def sylvester(b: int) -> np.ndarray:
    """H_b as an int64 matrix, entry (-1)^popcount(i & j)."""
    i = np.arange(b)[:, None]
    j = np.arange(b)[None, :]
    parity = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(i & j)
    return np.where(parity == 1, -1, 1).astype(np.int64)


def rn_fp32_inv_sqrt(b: int) -> np.float32:
    """RN_fp32(1/sqrt(b)) for b = 2^(2k+1), computed exactly: 1/sqrt(2^(2k+1))
    = sqrt(2) * 2^-(k+1), and RN_fp32(sqrt(2)) is found with integer square
    roots (24-bit significand m with m^2 nearest 2 * 2^46)."""
    e = int(round(math.log2(b)))
    assert 1 << e == b and e % 2 == 1
    m = math.isqrt(2 << 46)              # floor(sqrt(2) * 2^23)
    if (2 * m + 1) ** 2 < (2 << 46) * 4:  # sqrt(2)*2^23 >= m + 1/2 -> round up
        m += 1
    return np.float32(m * 2.0 ** -23 * 2.0 ** -((e + 1) // 2))


def fwht_unscaled(x: np.ndarray, b: int) -> np.ndarray:
    """Blockwise butterflies along the last axis of an fp32 [M, K] array,
    in the pinned order, no normalisation.  Returns fp32 [M, K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    assert b in VALID_BLOCKS and K % b == 0
    v = x.reshape(M, K // b, b)
    h = 1
    while h < b:
        v = v.reshape(M, K // b, b // (2 * h), 2, h)
        lo = v[..., 0, :]
        hi = v[..., 1, :]
        v = np.stack((lo + hi, lo - hi), axis=-2)   # fp32 RNE adds
        h *= 2
    return v.reshape(M, K)


def scale_factor(b: int):
    """(factor, exact) with y = RN(v * factor); exact when log2(b) is even."""
    e = int(round(math.log2(b)))
    if e % 2 == 0:
        return np.float32(2.0 ** (-e // 2)), True
    return rn_fp32_inv_sqrt(b), False


def block_hadamard_f32(x: np.ndarray, b: int) -> np.ndarray:
    """y = x · blockdiag(H_b)/sqrt(b) for fp32 x [M, K] (pinned rounding)."""
    v = fwht_unscaled(x, b)
    f, _ = scale_factor(b)
    return (v * f).astype(np.float32)


def block_hadamard_bf16(x_bits: np.ndarray, b: int) -> np.ndarray:
    """Same transform for bf16 input bits [M, K]; returns fp32 [M, K]."""
    return block_hadamard_f32(bf16_to_f32(x_bits), b)
