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
