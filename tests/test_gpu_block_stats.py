"""GPU parity of block_stats against the oracle: Delta_new bit-exact, the
eight statistics within 1e-5 relative (maxima exact), run-to-run identical."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import stats as S
from helpers import dev_bf16, host_bits, need_gpu, log

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(23))


def check(inp, out, dprev):
    log(f"block_stats n={inp.size} dprev={dprev is not None}")
    dn, st = V.block_stats(dev_bf16(inp), dev_bf16(out), None if dprev is None else dev_bf16(dprev))
    torch.cuda.synchronize()
    dref, sref = S.block_stats(inp, out, dprev)
    assert np.array_equal(host_bits(dn), dref)
    got = st.cpu().numpy()
    assert got[4] == sref[4] and got[6] == sref[6]
    assert np.allclose(got, sref, rtol=1e-5, atol=0), (got, sref)
    return got


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 65536 + 3, 4446 * 1920])
@pytest.mark.parametrize("with_prev", [False, True])
def test_random(n, with_prev):
    need_gpu()
    inp = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32))
    out = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32) * 0.1 + F32(inp))
    dprev = synth.to_bf16_bits(RNG.standard_normal(n).astype(np.float32) * 0.1) if with_prev else None
    check(inp, out, dprev)


def F32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("n", [1000, 65536 + 3, 4446 * 1920])
@pytest.mark.parametrize("with_prev", [False, True])
def test_without_delta(n, with_prev):
    """No Delta_new buffer: nothing is written (the inputs keep their bits)
    and the eight statistics equal those of the call that writes Delta_new."""
    need_gpu()
    log(f"block_stats without Delta_new n={n} dprev={with_prev}")
    inp = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32))
    out = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32) * 0.1 + F32(inp))
    dprev = synth.to_bf16_bits(RNG.standard_normal(n).astype(np.float32) * 0.1) if with_prev else None
    di, do = dev_bf16(inp), dev_bf16(out)
    dp = dev_bf16(dprev) if with_prev else None
    _, st_ref = V.block_stats(di, do, dp)
    none, st = V.block_stats(di, do, dp, write_delta=False)
    torch.cuda.synchronize()
    assert none is None
    assert np.array_equal(host_bits(di), inp) and np.array_equal(host_bits(do), out)
    if with_prev:
        assert np.array_equal(host_bits(dp), dprev)
    assert np.array_equal(st.cpu().numpy(), st_ref.cpu().numpy())


def test_closed_forms_on_gpu():
    need_gpu()
    x = RNG.integers(-16, 17, size=(64, 96)).astype(np.float32).ravel() * 8
    inp = synth.to_bf16_bits(x)
    out = synth.to_bf16_bits(x * np.float32(1.125))
    d = RNG.choice([-8.0, -4.0, 4.0, 8.0], size=x.size).astype(np.float32)
    dprev = synth.to_bf16_bits(d * 1.25)
    out2 = synth.to_bf16_bits(x + d)
    got = check(inp, out, None)
    assert S.gamma(got) == 0.125
    got = check(inp, out2, dprev)
    assert abs(S.delta_change(got) - 0.2) < 1e-12


def test_repeatable():
    need_gpu()
    n = 4446 * 1920
    a = dev_bf16(synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32)))
    b = dev_bf16(synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32)))
    _, s1 = V.block_stats(a, b, a)
    _, s2 = V.block_stats(a, b, a)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


# ---- the delta cache in MXFP8

def check_mx8(inp, out, dprev):
    """dprev: None or (codes, scales) host arrays."""
    log(f"block_stats_mx8 n={inp.size} dprev={dprev is not None}")
    dp = None
    if dprev is not None:
        dp = V.MXTensor(torch.from_numpy(dprev[0]).cuda(), torch.from_numpy(dprev[1]).cuda(), "mxfp8")
    dn, st = V.block_stats_mx8(dev_bf16(inp), dev_bf16(out), dp)
    torch.cuda.synchronize()
    (qref, sref_s), sref = S.block_stats_mx8(inp, out, dprev)
    assert np.array_equal(dn.q.cpu().numpy(), qref)
    assert np.array_equal(dn.scales.cpu().numpy(), sref_s)
    got = st.cpu().numpy()
    assert got[4] == sref[4] and got[6] == sref[6]
    assert np.allclose(got, sref, rtol=1e-5, atol=0), (got, sref)
    return got, (qref, sref_s)


@pytest.mark.parametrize("n", [0, 32, 96, 1024, 65536 + 32, 4446 * 1920])
def test_mx8_random(n):
    need_gpu()
    inp = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32))
    out = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32) * 0.1 + F32(inp))
    _, first = check_mx8(inp, out, None)
    # the next step reads the cached delta back
    out2 = synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32) * 0.1 + F32(inp))
    check_mx8(inp, out2, first)


def test_mx8_extreme_blocks():
    """Zero deltas (exponent -127), bf16 subnormal deltas, deltas near 1e30,
    and blocks whose largest delta lands in the clipping band."""
    need_gpu()
    n = 32 * 6
    inp = np.zeros(n, np.float32)
    out = np.zeros(n, np.float32)
    out[32:64] = 2.0 ** -130
    out[64:96] = RNG.standard_normal(32).astype(np.float32) * 1e30
    out[96:128] = np.linspace(-15, 15, 32).astype(np.float32)
    out[128:160] = -0.0
    out[160:192] = RNG.standard_normal(32).astype(np.float32) * 3
    prev = (np.full(n, 0x38, np.uint8), np.full(n // 32, 120, np.uint8))
    check_mx8(synth.to_bf16_bits(inp), synth.to_bf16_bits(out), prev)


def test_mx8_repeatable():
    need_gpu()
    n = 4446 * 1920
    a = dev_bf16(synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32)))
    b = dev_bf16(synth.to_bf16_bits(RNG.laplace(size=n).astype(np.float32)))
    d1, s1 = V.block_stats_mx8(a, b)
    _, s2 = V.block_stats_mx8(a, b, d1)
    _, s3 = V.block_stats_mx8(a, b, d1)
    torch.cuda.synchronize()
    assert torch.equal(s2, s3)
    assert float(s2[2].cpu()) == 0.0      # the same delta read back

