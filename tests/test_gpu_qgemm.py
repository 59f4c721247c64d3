"""GPU parity of qgemm_w4a4 / qgemm_w4a8 against the oracle: relative
Frobenius error <= 2e-3 (bf16 compared with the oracle's bf16 rounding; f32
with its exact value, where it must also be <= 1e-5), every element within
the fp32-summation bound of helpers.assert_elementwise, and the W4A8 integer
accumulator bit-exact."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import formats as F, gemm as G, quant as Q
from helpers import (assert_elementwise, bf16_values, dev_bf16, host_bits, need_gpu, rel_fro, log,
                     terms_w4a4, terms_w4a8)

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(22))
TOL = 2e-3


def nvfp4_dev(q, s, ts):
    return V.NVFP4Tensor(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(),
                         torch.tensor(ts, dtype=torch.float32).cuda())


def check_layer(x_bits, w_bits, b=64, bias=True, rows=None, out_dtypes=("bf16", "f32")):
    M, K = x_bits.shape
    N = w_bits.shape[0]
    log(f"gemm case M={M} N={N} K={K} rows={'all' if rows is None else len(rows)}")
    sel = np.arange(M) if rows is None else rows
    # weights: prepared on both sides, compared bit for bit
    wq_o, ws_o, wgs_o = Q.prepare_weight(w_bits, b)
    wd = V.hadamard_quantize(dev_bf16(w_bits), b, "nvfp4")
    assert np.array_equal(wd.q.cpu().numpy(), wq_o) and np.array_equal(wd.scales.cpu().numpy(), ws_o)
    assert wd.ts.cpu().numpy()[1] == wgs_o
    bias_h = RNG.standard_normal(N).astype(np.float32) if bias else None
    bias_d = torch.from_numpy(bias_h).cuda() if bias else None
    xd = dev_bf16(x_bits)
    # oracle activations on the sampled rows (NVFP4 amax over every row)
    amax = None
    if rows is not None:
        from oracle import hadamard as H
        amax = np.float32(0)
        for r0 in range(0, M, 4096):
            amax = max(amax, np.float32(np.abs(H.block_hadamard_bf16(x_bits[r0:r0 + 4096], b)).max()))
    a4 = Q.hadamard_quantize(x_bits[sel], b, "nvfp4", amax=amax)
    a8 = Q.hadamard_quantize(x_bits[sel], b, "int8")
    ad4 = V.hadamard_quantize(xd, b, "nvfp4")
    ad8 = V.hadamard_quantize(xd, b, "int8")
    # the activation codes themselves are checked bit for bit on the same rows
    assert np.array_equal(ad4.q.cpu().numpy()[sel], a4["q"]) and np.array_equal(ad4.scales.cpu().numpy()[sel], a4["scales"])
    assert np.array_equal(ad8.q.cpu().numpy()[sel], a8["q"])
    assert np.array_equal(ad8.scales.cpu().numpy()[sel].view(np.uint32), a8["scales"].view(np.uint32))
    t4 = terms_w4a4(a4["q"], a4["scales"], a4["gs"], wq_o, ws_o, wgs_o, bias_h)
    t8 = terms_w4a8(a8["q"], a8["scales"], wq_o, ws_o, wgs_o, bias_h)
    for od in out_dtypes:
        y4 = V.qgemm_w4a4(ad4, wd, bias_d, od)
        y8 = V.qgemm_w4a8(ad8, wd, bias_d, od)
        torch.cuda.synchronize()
        e4, r4 = G.qgemm_w4a4(a4["q"], a4["scales"], a4["gs"], wq_o, ws_o, wgs_o, bias_h, od)
        e8, r8 = G.qgemm_w4a8(a8["q"], a8["scales"], wq_o, ws_o, wgs_o, bias_h, od)
        if od == "bf16":
            g4 = bf16_values(host_bits(y4)[sel]); g8 = bf16_values(host_bits(y8)[sel])
            w4 = bf16_values(r4); w8 = bf16_values(r8)
        else:
            g4 = y4.cpu().numpy()[sel]; g8 = y8.cpu().numpy()[sel]
            w4, w8 = e4, e8
        err4, err8 = rel_fro(g4, w4), rel_fro(g8, w8)
        q4 = assert_elementwise(g4, e4, t4, K, od, f"w4a4 {od}")
        q8 = assert_elementwise(g8, e8, t8, K, od, f"w4a8 {od}")
        log(f"  {od}: w4a4 rel {err4:.2e} (max err/bound {q4:.3f})  w4a8 rel {err8:.2e} (max err/bound {q8:.3f})")
        assert err4 <= TOL and err8 <= TOL, (err4, err8)
        if od == "f32":
            assert err4 < 1e-5 and err8 < 1e-5   # only fp32 accumulation order differs


def test_tiny_layer():
    need_gpu()
    d = synth.tiny_layer()
    check_layer(d["x"], d["w"])
    check_layer(d["x"], d["w"], bias=False)


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (129, 33, 64), (300, 200, 320), (5, 130, 96),
                                   (64, 64, 48), (200, 257, 16), (1, 640, 1920), (131, 129, 256)])
def test_ragged(M, N, K):
    need_gpu()
    b = 16 if K % 64 else 64
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    check_layer(x, w, b=b)


def test_w4a8_integer_accumulator_exact():
    """Unit weight scales, gs_w = 1, s_a = 1: Y = sum_k q * e2m1(w) exactly."""
    need_gpu()
    M, N, K = 192, 160, 3072
    q = RNG.integers(-127, 128, size=(M, K)).astype(np.int8)
    codes = RNG.integers(0, 16, size=(N, K)).astype(np.uint8)
    wq = F.pack_nibbles(codes)
    ws = np.full((N, K // 16), 0x38, np.uint8)
    P = G.w4a8_integer_accumulator(q, wq)
    # every partial sum stays below 2^24 (bound: K * 127 * 12 / 2)
    assert K * 127 * 12 // 2 < 2 ** 24
    a = V.INT8Tensor(torch.from_numpy(q).cuda(), torch.ones(M, dtype=torch.float32, device="cuda"))
    w = nvfp4_dev(wq, ws, [1.0, 1.0])
    y = V.qgemm_w4a8(a, w, None, "f32")
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64) * 2, P.astype(np.float64))


def test_w4a4_unit_scale_exact_products():
    """Unit tensor scales and small exact sums: the fp32 result is exact."""
    need_gpu()
    M, N, K = 96, 64, 512
    ac = RNG.integers(0, 16, size=(M, K)).astype(np.uint8)
    wc = RNG.integers(0, 16, size=(N, K)).astype(np.uint8)
    as_ = RNG.integers(0x30, 0x40, size=(M, K // 16)).astype(np.uint8)   # 0.5 .. 1.875
    ws = RNG.integers(0x30, 0x40, size=(N, K // 16)).astype(np.uint8)
    a = nvfp4_dev(F.pack_nibbles(ac), as_, [2688.0, 1.0])
    w = nvfp4_dev(F.pack_nibbles(wc), ws, [2688.0, 1.0])
    y = V.qgemm_w4a4(a, w, None, "f32")
    torch.cuda.synchronize()
    want, _ = G.qgemm_w4a4(F.pack_nibbles(ac), as_, 1.0, F.pack_nibbles(wc), ws, 1.0, None, "f32")
    # products are multiples of 2^-8 below 2^7, sums below 2^16: all exact in fp32
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("lo,hi", [(0x01, 0x08), (0x00, 0x7F)])
def test_w4a4_full_scale_range_exact(lo, hi):
    """Scale bytes over the subnormal E4M3 range (and the whole range): the
    decoded operands are exact, so with sums that fit fp32 the result is
    bit-exact; over the whole range it agrees to fp32 accumulation."""
    need_gpu()
    M, N, K = 64, 96, 256
    ac = RNG.integers(0, 16, size=(M, K)).astype(np.uint8)
    wc = RNG.integers(0, 16, size=(N, K)).astype(np.uint8)
    as_ = RNG.integers(lo, hi, size=(M, K // 16)).astype(np.uint8)
    ws = RNG.integers(lo, hi, size=(N, K // 16)).astype(np.uint8)
    a = nvfp4_dev(F.pack_nibbles(ac), as_, [2688.0, 1.0])
    w = nvfp4_dev(F.pack_nibbles(wc), ws, [2688.0, 1.0])
    y = V.qgemm_w4a4(a, w, None, "f32")
    torch.cuda.synchronize()
    want, _ = G.qgemm_w4a4(F.pack_nibbles(ac), as_, 1.0, F.pack_nibbles(wc), ws, 1.0, None, "f32")
    got = y.cpu().numpy().astype(np.float64)
    if hi <= 0x08:
        # products are multiples of 2^-20 below 2^-7: sums of 256 are exact
        assert np.array_equal(got, want)
    else:
        assert rel_fro(got, want) < 1e-6
        t = terms_w4a4(F.pack_nibbles(ac), as_, 1.0, F.pack_nibbles(wc), ws, 1.0, None)
        assert_elementwise(got, want, t, K, "f32", "full scale range")


@pytest.mark.parametrize("name", ["qkv", "out", "ffn_up", "ffn_down"])
def test_cogvideox_5b_linears_sampled(name):
    need_gpu()
    M = synth.TOKENS_2B_5B
    K, N = {n: (k, nn) for n, k, nn in synth.block_linears(3072)}[name]
    x, w = synth.layer_inputs(M, name, K, N)
    check_layer(x, w, rows=synth.row_sample(M, 48), out_dtypes=("bf16", "f32"))


@pytest.mark.parametrize("name", ["qkv", "out", "ffn_up", "ffn_down"])
def test_cogvideox_2b_linears_sampled(name):
    """CogVideoX-2B-shaped block (hidden 1920): K = 1920 / 7680, N up to 7680."""
    need_gpu()
    M = synth.TOKENS_2B_5B
    K, N = {n: (k, nn) for n, k, nn in synth.block_linears(1920)}[name]
    x, w = synth.layer_inputs(M, name, K, N)
    check_layer(x, w, rows=synth.row_sample(M, 48), out_dtypes=("bf16", "f32"))


@pytest.mark.parametrize("M,N,K", [(1000, 700, 1024), (300, 260, 3072), (17, 2000, 2048), (4400, 4400, 1536)])
def test_split_k_repeatable(M, N, K):
    """Few tiles (or a partial last wave: 4400 x 4400 is 324 tiles) and long
    K: tiles are split into K slices whose fp32 partial sums a reduce pass
    adds in slice order.  The result matches the oracle and three calls give
    identical bits."""
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    check_layer(x, w, out_dtypes=("f32", "bf16"), rows=synth.row_sample(M, 64) if M > 2000 else None)
    wd = V.hadamard_quantize(dev_bf16(w), 64, "nvfp4")
    ad = V.hadamard_quantize(dev_bf16(x), 64, "nvfp4")
    a8 = V.hadamard_quantize(dev_bf16(x), 64, "int8")
    for fn, a in ((V.qgemm_w4a4, ad), (V.qgemm_w4a8, a8)):
        ys = [fn(a, wd, None, "f32") for _ in range(3)]
        torch.cuda.synchronize()
        assert all(torch.equal(ys[0], y) for y in ys[1:])


@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("fmt", ["nvfp4", "int8"])
def test_bf16_output_is_rounded_f32(fmt, with_bias):
    """The bf16 output (staged through LDS) is the fp32 output (stored
    directly, same accumulation) rounded to nearest even, bit for bit, with
    and without a bias (the NVFP4 epilogue has a copy for each), ragged M
    and a split tail."""
    need_gpu()
    M, N, K = 4000, 9216, 1024
    x = torch.from_numpy(RNG.laplace(size=(M, K)).astype(np.float32)).to(torch.bfloat16).cuda()
    w = (torch.from_numpy(RNG.standard_normal((N, K)).astype(np.float32)) * 0.02).to(torch.bfloat16).cuda()
    bias = torch.from_numpy(RNG.standard_normal(N).astype(np.float32)).cuda() if with_bias else None
    a = V.hadamard_quantize(x, 64, fmt)
    wd = V.hadamard_quantize(w, 64, "nvfp4")
    fn = V.qgemm_w4a4 if fmt == "nvfp4" else V.qgemm_w4a8
    yb = fn(a, wd, bias, "bf16")
    yf = fn(a, wd, bias, "f32")
    torch.cuda.synchronize()
    got, want = host_bits(yb), F.f32_to_bf16(yf.cpu().numpy())
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]

