"""GPU parity of the GELU prologue of hadamard_quantize (the FFN-down input
quantized straight from FFN-up's bf16 output): codes, scales and the
rotated bf16 rows bit-exact against the oracle's fp32 GELU steps, for every
activation format.

The exhaustive case places each of the 65280 finite bf16 values alone in a
16-element Hadamard block, so that the rotated bf16 output holds
GELU(x) / 4 for each of them individually."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import quant as Q
from helpers import dev_bf16, host_bits, need_gpu, log

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(61))
FMTS = ["nvfp4", "int8", "bf16", "mxfp4", "mxfp8"]


def run_both(x_bits, b, fmt, ldx_pad=0, stats=True):
    M, K = x_bits.shape
    log(f"gelu quant M={M} K={K} b={b} fmt={fmt} pad={ldx_pad}")
    if ldx_pad:
        big = np.zeros((M, K + ldx_pad), np.uint16)
        big[:, :K] = x_bits
        xd = dev_bf16(big)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    r = V.hadamard_quantize(xd, b, fmt, stats=stats, gelu=True)
    torch.cuda.synchronize()
    ref = Q.hadamard_quantize(x_bits, b, fmt, gelu=True)
    q = host_bits(r.q) if fmt == "bf16" else r.q.cpu().numpy()
    assert np.array_equal(q, ref["q"]), np.argwhere(q != ref["q"])[:5]
    if fmt != "bf16":
        assert np.array_equal(r.scales.cpu().numpy(), ref["scales"])
    if fmt == "nvfp4":
        assert np.array_equal(r.ts.cpu().numpy(), np.array([ref["amax"], ref["gs"]], np.float32))
    if stats:
        st, want = r.stats.cpu().numpy(), ref["stats"]
        assert st[0] == want[0] and st[2] == want[2], (st, want)
        assert np.allclose(st[[1, 3]], want[[1, 3]], rtol=1e-5, atol=0), (st, want)


def test_gelu_every_bf16_value():
    need_gpu()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    x = np.zeros((len(finite) // 64, 1024), np.uint16)
    x.reshape(-1, 16)[:, 0] = finite
    run_both(x, 16, "bf16", stats=False)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("b", [16, 64, 256])
def test_gelu_quant_laplace(fmt, b):
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(300, 1280)).astype(np.float32) * 3)
    run_both(x, b, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_gelu_quant_ragged_strided(fmt):
    need_gpu()
    K = 96 if fmt != "int8" else 160
    x = synth.to_bf16_bits(RNG.standard_normal((257, K)).astype(np.float32) * 4)
    run_both(x, 32, fmt, ldx_pad=8)


def test_gelu_quant_tail_and_extremes():
    """The negative tail (GELU values down to the fp32 subnormal range and
    -0), large magnitudes (GELU = x or -0; small enough that the sums of
    64 of them stay finite) and bf16 subnormals."""
    need_gpu()
    K = 128
    rows = [np.linspace(-14, -3, K), np.linspace(-1e30, 1e30, K), np.full(K, 2.0 ** -130),
            np.linspace(-3e36, 3e36, K), RNG.standard_normal(K) * 2.0 ** -120]
    x = synth.to_bf16_bits(np.stack(rows).astype(np.float32))
    for fmt in ("bf16", "mxfp8", "mxfp4"):
        run_both(x, 64, fmt, stats=False)
