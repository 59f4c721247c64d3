"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module draws random numbers and rounds them to bf16 (the storage type of
the activations and weights); it holds none of the quantization method's
arithmetic.  Both the CPU oracle and the GPU path consume the exact same bytes.

Shapes follow CogVideoX-2B/5B DiT blocks as the 6Bit-Diffusion write-ups
describe their test models (gist.science summary "6Bit-Diffusion:
Inference-Time Mixed-Precision Quantization for Video Diffusion Models",
§4 Resultados; youleyou.com article, §四): a 49-frame clip becomes 13 latent
frames, 30x45 latent patches at 480x720, plus 226 text tokens.  The activation
distribution (Laplace body with a few amplified channels) stands in for the
heavy-tailed DiT activations the jsqmd.com article on video-DiT quantization
describes in §1.1 (token heterogeneity, outlier channels).

All generators use numpy's PCG64 and return bf16 bit patterns as uint16
arrays (row-major), so the data is identical on every machine.
"""
from __future__ import annotations

import numpy as np
import torch

# ---------------------------------------------------------------- shapes
TEXT_TOKENS = 226
TOKENS_2B_5B = 13 * 30 * 45 + TEXT_TOKENS      # 17776
TOKENS_1080P = 13 * 68 * 120 + TEXT_TOKENS     # 106306
TOKENS_DYN = 4446                              # reduced-resolution schedule study

# (name, K, N) for the four linears of one DiT block, hidden size h, FFN 4h.
def block_linears(hidden: int):
    return [("qkv", hidden, 3 * hidden), ("out", hidden, hidden),
            ("ffn_up", hidden, 4 * hidden), ("ffn_down", 4 * hidden, hidden)]

# Layer ids used to derive seeds (X: 1000+id, W: 2000+id, outliers: 3000+id).
LAYER_IDS = {"qkv": 0, "out": 1, "ffn_up": 2, "ffn_down": 3}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to bf16 (round-to-nearest-even) and return
    the raw uint16 bit patterns.  Uses torch's cast as a library routine."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def outlier_channels(K: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.permutation(K)[:count])


def n_outliers(K: int, frac: float = 0.005) -> int:
    return int(round(frac * K))


def laplace_activations(M: int, K: int, seed: int, outlier_seed: int,
                        frac: float = 0.005, mult: float = 30.0,
                        chunk_rows: int = 4096) -> np.ndarray:
    """X ~ Laplace(0, 1) of shape [M, K] with round(frac*K) channels scaled by
    `mult`; returned as bf16 bits.  Laplace(0,1) is drawn as the difference of
    two independent Exp(1) variables, in float32, chunk by chunk."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ch = outlier_channels(K, n_outliers(K, frac), outlier_seed)
    out = np.empty((M, K), dtype=np.uint16)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        e1 = rng.standard_exponential((r1 - r0, K), dtype=np.float32)
        e2 = rng.standard_exponential((r1 - r0, K), dtype=np.float32)
        blk = e1 - e2
        if len(ch):
            blk[:, ch] *= np.float32(mult)
        out[r0:r1] = to_bf16_bits(blk)
    return out


def normal_matrix(rows: int, cols: int, std: float, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(a)


# ---------------------------------------------------------------- configs
def tiny_layer():
    """256x256 X ~ N(0,1) with 4 outlier channels x20; W ~ N(0, 0.02)."""
    M = K = N = 256
    rng = np.random.Generator(np.random.PCG64(1000))
    x = rng.standard_normal((M, K), dtype=np.float32)
    ch = outlier_channels(K, 4, 3000)
    x[:, ch] *= np.float32(20.0)
    return {"x": to_bf16_bits(x), "w": normal_matrix(N, K, 0.02, 2000),
            "M": M, "K": K, "N": N, "outlier_channels": ch}


def layer_inputs(M: int, name: str, K: int, N: int, frac=0.005, mult=30.0):
    lid = LAYER_IDS[name]
    x = laplace_activations(M, K, 1000 + lid, 3000 + lid, frac, mult)
    w = normal_matrix(N, K, 0.02, 2000 + lid)
    return x, w


def row_sample(M: int, count: int, seed: int = 7) -> np.ndarray:
    """Sorted, seeded sample of row indices that always includes the first
    and the last row (the ragged tail of a tiled kernel)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pick = rng.choice(M, size=min(count, M), replace=False)
    return np.unique(np.concatenate([pick, [0, M - 1]]))


def dyn_schedule(blocks: int = 30, steps: int = 50, M: int = TOKENS_DYN,
                 hidden: int = 1920, n_spikes: int = 3):
    """Parameters of the synthetic closed-loop schedule study: per block a
    smooth residual trajectory plus decaying noise, and a few (block, step)
    pairs whose input carries one channel amplified x300.

    Delta_{b,t} = a_b * (1 + 0.5 sin(pi t / steps + phi_b)) * U_b
                  + beta_b * exp(-t / 10) * Z_{b,t}
    The smooth part mirrors the PF-ODE smoothing argument of the youleyou.com
    article, §二 (adjacent-step differences shrink along the trajectory)."""
    par = []
    for b in range(blocks):
        rng = np.random.Generator(np.random.PCG64(6000 + b))
        a = rng.uniform(0.05, 0.5)
        beta = rng.uniform(0.01, 0.2)
        phi = rng.uniform(0.0, 2 * np.pi)
        par.append((a, beta, phi))
    rng = np.random.Generator(np.random.PCG64(7000))
    spikes = {}
    while len(spikes) < n_spikes:
        key = (int(rng.integers(0, blocks)), int(rng.integers(2, steps)))
        spikes[key] = int(rng.integers(0, hidden))
    return {"blocks": blocks, "steps": steps, "M": M, "hidden": hidden,
            "params": par, "spikes": spikes}


class DynWorkload:
    """Seeded inputs of the closed-loop schedule study (host, float32 / bf16
    bits).  Block 0's input at step t is Laplace(0, 1) with round(0.005 *
    hidden) channels x30 (seed 500 + t, channels from seed 3000); block b's
    input is block b-1's output.  U_b ~ Laplace (seed 4000 + b); the noise
    Z_{b,t} is a fixed N(0, 1) field per block (seed 5000 + b) rotated by
    7919 * t elements, so every step sees different noise without a fresh
    draw.  A spike multiplies one channel of the block input by 300 (fp32
    product, then bf16 round to nearest even)."""

    SPIKE_MULT = 300.0
    ROLL = 7919

    def __init__(self, blocks=30, steps=50, M=TOKENS_DYN, hidden=1920, n_spikes=3):
        self.sched = dyn_schedule(blocks, steps, M, hidden, n_spikes)
        self.blocks, self.steps, self.M, self.hidden = blocks, steps, M, hidden
        self._U, self._N = {}, {}

    def block0_input(self, t: int) -> np.ndarray:
        return to_bf16_bits(dyn_block_input(t, self.M, self.hidden))

    def spike_channel(self, b: int, t: int):
        return self.sched["spikes"].get((b, t))

    def coefficients(self, b: int, t: int):
        """(smooth, noise) fp32 multipliers of U_b and Z_{b,t}."""
        a, beta, phi = self.sched["params"][b]
        return (np.float32(a * (1.0 + 0.5 * np.sin(np.pi * t / self.steps + phi))),
                np.float32(beta * np.exp(-t / 10.0)))

    def U(self, b: int) -> np.ndarray:
        if b not in self._U:
            ru = np.random.Generator(np.random.PCG64(4000 + b))
            shape = (self.M, self.hidden)
            self._U[b] = (ru.standard_exponential(shape, dtype=np.float32)
                          - ru.standard_exponential(shape, dtype=np.float32))
        return self._U[b]

    def N(self, b: int) -> np.ndarray:
        if b not in self._N:
            rz = np.random.Generator(np.random.PCG64(5000 + b))
            self._N[b] = rz.standard_normal((self.M, self.hidden), dtype=np.float32)
        return self._N[b]

    def shift(self, t: int) -> int:
        return (self.ROLL * t) % (self.M * self.hidden)

    def delta(self, b: int, t: int) -> np.ndarray:
        """Delta_{b,t} in fp32: RN(RN(smooth * U_b) + RN(noise * Z_{b,t}))."""
        sm, nz = self.coefficients(b, t)
        Z = np.roll(self.N(b).reshape(-1), self.shift(t)).reshape(self.M, self.hidden)
        return (sm * self.U(b)).astype(np.float32) + (nz * Z).astype(np.float32)


def dyn_block_input(t: int, M: int, hidden: int) -> np.ndarray:
    """Input of block 0 at step t (float32, not yet rounded)."""
    rng = np.random.Generator(np.random.PCG64(500 + t))
    x = (rng.standard_exponential((M, hidden), dtype=np.float32)
         - rng.standard_exponential((M, hidden), dtype=np.float32))
    ch = outlier_channels(hidden, n_outliers(hidden), 3000)
    x[:, ch] *= np.float32(30.0)
    return x
