"""GPU parity of the MX-native variant against the oracle: hadamard_quantize
in MXFP4 / MXFP8 (codes and E8M0 scales bit-exact, statistics as for the
other formats) and qgemm_mx (relative Frobenius error <= 2e-3 with bf16
output; with fp32 output only the accumulation inside the matrix
instruction differs; exact when every partial sum is representable)."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import formats as F, gemm as G, quant as Q
from helpers import assert_elementwise, bf16_values, dev_bf16, host_bits, need_gpu, rel_fro, log, terms_mx

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(51))
TOL = 2e-3


def check_quant(x_bits, b, fmt, ldx_pad=0, rows=None, stats=True):
    M, K = x_bits.shape
    log(f"mx quant M={M} K={K} b={b} fmt={fmt} pad={ldx_pad}")
    if ldx_pad:
        big = np.zeros((M, K + ldx_pad), np.uint16)
        big[:, :K] = x_bits
        xd = dev_bf16(big)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    r = V.hadamard_quantize(xd, b, fmt, stats=stats)
    torch.cuda.synchronize()
    sel = np.arange(M) if rows is None else rows
    ref = Q.hadamard_quantize(x_bits[sel], b, fmt)
    q = r.q.cpu().numpy()[sel]
    s = r.scales.cpu().numpy()[sel]
    bad = np.nonzero((q != ref["q"]).any(1) | (s != ref["scales"]).any(1))[0]
    assert len(bad) == 0, f"rows {sel[bad[:5]]} differ"
    if stats and rows is None:
        st = r.stats.cpu().numpy()
        want = ref["stats"]
        assert st[0] == want[0] and st[2] == want[2], (st, want)
        assert np.allclose(st[[1, 3]], want[[1, 3]], rtol=1e-5, atol=0), (st, want)
    return r, ref


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("b", [16, 32, 64, 128, 256])
def test_quant_tiny_layer_all_blocks(fmt, b):
    need_gpu()
    d = synth.tiny_layer()
    check_quant(d["x"], b, fmt)


@pytest.mark.parametrize("M,K,b,pad", [(1, 64, 64, 0), (3, 256, 64, 8), (257, 320, 64, 0), (65, 96, 32, 0),
                                       (7, 32, 16, 8), (129, 384, 128, 0), (5, 768, 256, 16), (300, 1920, 64, 0),
                                       (1000, 160, 32, 0)])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_quant_ragged_shapes(M, K, b, pad, fmt):
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32) * 2)
    check_quant(x, b, fmt, ldx_pad=pad)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_quant_extreme_magnitudes(fmt):
    """Zero rows, bf16 subnormals (block exponents clamped at -127), values
    near the bf16 maximum, and blocks whose top element lands in the
    saturating band."""
    need_gpu()
    K = 128
    rows = [np.zeros(K, np.float32),
            np.full(K, 2.0 ** -130, np.float32),
            RNG.standard_normal(K).astype(np.float32) * 2.0 ** -128,
            RNG.standard_normal(K).astype(np.float32) * 1e36,
            np.where(np.arange(K) % 2 == 0, -0.0, 0.0).astype(np.float32),
            RNG.standard_normal(K).astype(np.float32) * 7.9]
    x = synth.to_bf16_bits(np.stack(rows))
    for b in (16, 64):
        # the fused statistics sum |y| in fp32 within a thread's 64 elements:
        # checked on the rows where that sum stays finite
        check_quant(x, b, fmt, stats=False)
        check_quant(x[[0, 1, 2, 4, 5]], b, fmt)


def test_quant_5b_ffn_down_sampled():
    need_gpu()
    M = synth.TOKENS_2B_5B
    x, _ = synth.layer_inputs(M, "ffn_down", 12288, 3072)
    for fmt in ("mxfp4", "mxfp8"):
        check_quant(x, 64, fmt, rows=synth.row_sample(M, 64), stats=False)


def mx_dev(q, s, fmt):
    return V.MXTensor(torch.from_numpy(np.ascontiguousarray(q)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(s)).cuda(), fmt)


def check_gemm(x_bits, w_bits, b=64, bias=True, rows=None, out_dtypes=("bf16", "f32"), fmts=("mxfp4", "mxfp8")):
    M, K = x_bits.shape
    N = w_bits.shape[0]
    log(f"mx gemm case M={M} N={N} K={K} rows={'all' if rows is None else len(rows)}")
    sel = np.arange(M) if rows is None else rows
    wq_o, ws_o = Q.prepare_weight_mx(w_bits, b)
    wd = V.hadamard_quantize(dev_bf16(w_bits), b, "mxfp4")
    assert np.array_equal(wd.q.cpu().numpy(), wq_o) and np.array_equal(wd.scales.cpu().numpy(), ws_o)
    bias_h = RNG.standard_normal(N).astype(np.float32) if bias else None
    bias_d = torch.from_numpy(bias_h).cuda() if bias else None
    xd = dev_bf16(x_bits)
    for fmt in fmts:
        ref = Q.hadamard_quantize(x_bits[sel], b, fmt)
        ad = V.hadamard_quantize(xd, b, fmt)
        assert np.array_equal(ad.q.cpu().numpy()[sel], ref["q"]) and np.array_equal(ad.scales.cpu().numpy()[sel], ref["scales"])
        terms = terms_mx(ref["q"], ref["scales"], fmt, wq_o, ws_o, bias_h)
        for od in out_dtypes:
            y = V.qgemm_mx(ad, wd, bias_d, od)
            torch.cuda.synchronize()
            e64, r = G.qgemm_mx(ref["q"], ref["scales"], fmt, wq_o, ws_o, bias_h, od)
            if od == "bf16":
                got, want = bf16_values(host_bits(y)[sel]), bf16_values(r)
            else:
                got, want = y.cpu().numpy()[sel], e64
            err = rel_fro(got, want)
            qb = assert_elementwise(got, e64, terms, K, od, f"{fmt} {od}")
            log(f"  {fmt} {od}: rel {err:.2e} (max err/bound {qb:.3f})")
            assert err <= TOL, err
            if od == "f32":
                assert err < 1e-5, err


def test_gemm_tiny_layer():
    need_gpu()
    d = synth.tiny_layer()
    check_gemm(d["x"], d["w"])
    check_gemm(d["x"], d["w"], bias=False)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (129, 33, 128), (300, 200, 384), (5, 300, 256),
                                   (131, 257, 256), (600, 520, 1920), (257, 255, 640)])
def test_gemm_ragged(M, N, K):
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    check_gemm(x, w)


@pytest.mark.parametrize("a_fmt", ["mxfp4", "mxfp8"])
def test_gemm_exact_sums(a_fmt):
    """Random codes with scale bytes near 127: every product is a multiple of
    2^-16 below 2^20 and every partial sum fits fp32, so the result is the
    oracle's exact value."""
    need_gpu()
    M, N, K = 160, 96, 1024
    if a_fmt == "mxfp4":
        ac = RNG.integers(0, 16, size=(M, K)).astype(np.uint8)
        aq = F.pack_nibbles(ac)
    else:
        # E4M3 bytes with exponent field 4..10 (magnitudes 2^-3 .. 2^3 * 1.875)
        aq = RNG.integers(0, 256, size=(M, K)).astype(np.uint8)
        aq = (aq & 0x87) | ((((aq >> 3) & 7) + 4) << 3).astype(np.uint8)
    a_s = RNG.integers(124, 131, size=(M, K // 32)).astype(np.uint8)
    wc = RNG.integers(0, 16, size=(N, K)).astype(np.uint8)
    w_s = RNG.integers(124, 131, size=(N, K // 32)).astype(np.uint8)
    y = V.qgemm_mx(mx_dev(aq, a_s, a_fmt), mx_dev(F.pack_nibbles(wc), w_s, "mxfp4"), None, "f32")
    torch.cuda.synchronize()
    want, _ = G.qgemm_mx(aq, a_s, a_fmt, F.pack_nibbles(wc), w_s, None, "f32")
    got = y.cpu().numpy().astype(np.float64)
    if a_fmt == "mxfp4":
        assert np.array_equal(got, want)
    else:
        assert rel_fro(got, want) < 1e-6


@pytest.mark.parametrize("M,N,K", [(1000, 700, 1024), (300, 260, 3072), (17, 2000, 2048), (4400, 4400, 1536)])
def test_gemm_split_k_repeatable(M, N, K):
    """Few tiles or a partial last wave: K slices and the reduce pass; three
    calls give identical bits."""
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    check_gemm(x, w, out_dtypes=("f32", "bf16"), rows=synth.row_sample(M, 64) if M > 2000 else None)
    wd = V.hadamard_quantize(dev_bf16(w), 64, "mxfp4")
    for fmt in ("mxfp4", "mxfp8"):
        a = V.hadamard_quantize(dev_bf16(x), 64, fmt)
        ys = [V.qgemm_mx(a, wd, None, "f32") for _ in range(3)]
        torch.cuda.synchronize()
        assert all(torch.equal(ys[0], y) for y in ys[1:])


@pytest.mark.parametrize("name", ["qkv", "out", "ffn_up", "ffn_down"])
def test_gemm_cogvideox_5b_sampled(name):
    need_gpu()
    M = synth.TOKENS_2B_5B
    K, N = {n: (k, nn) for n, k, nn in synth.block_linears(3072)}[name]
    x, w = synth.layer_inputs(M, name, K, N)
    check_gemm(x, w, rows=synth.row_sample(M, 48), out_dtypes=("bf16", "f32"))


def test_gemm_two_waves_and_split_tail():
    """Two waves of data-parallel tiles (512 of 600) plus a split tail of 88
    tiles in 2 K slices, ragged M, bias."""
    need_gpu()
    M, N, K = 2000, 19200, 1024
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    check_gemm(x, w, rows=synth.row_sample(M, 96), out_dtypes=("bf16", "f32"))


@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_gemm_bf16_output_is_rounded_f32(fmt, with_bias):
    """The bf16 output is the fp32 output (same accumulation order) rounded
    to nearest even, bit for bit: pins the epilogue's bf16 conversion, with
    and without a bias (the epilogue has a copy for each)."""
    need_gpu()
    M, N, K = 4096, 9216, 1024
    x = torch.from_numpy(RNG.laplace(size=(M, K)).astype(np.float32)).to(torch.bfloat16).cuda()
    w = (torch.from_numpy(RNG.standard_normal((N, K)).astype(np.float32)) * 0.02).to(torch.bfloat16).cuda()
    bias = torch.from_numpy(RNG.standard_normal(N).astype(np.float32)).cuda() if with_bias else None
    a = V.hadamard_quantize(x, 64, fmt)
    wd = V.hadamard_quantize(w, 64, "mxfp4")
    yb = V.qgemm_mx(a, wd, bias, "bf16")
    yf = V.qgemm_mx(a, wd, bias, "f32")
    torch.cuda.synchronize()
    want = F.f32_to_bf16(yf.cpu().numpy())
    got = host_bits(yb)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_ragged_edges_padded_output(fmt, with_bias):
    """561 tiles with ragged M and N (17 x 33 tiles of 4100 x 8200): 512 in
    the data-parallel kernel, 49 in K slices.  The bf16 output, written into
    a row-padded buffer whose padding must stay untouched, equals the RNE of
    the fp32 output bit for bit, and rows of the first and last tile rows
    meet the element-wise bar against the oracle."""
    need_gpu()
    M, N, K = 4100, 8200, 1024
    x_bits = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w_bits = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    bias_h = RNG.standard_normal(N).astype(np.float32) if with_bias else None
    log(f"mx ragged edges fmt={fmt} bias={with_bias}")
    a = V.hadamard_quantize(dev_bf16(x_bits), 64, fmt)
    wd = V.hadamard_quantize(dev_bf16(w_bits), 64, "mxfp4")
    bias_d = torch.from_numpy(bias_h).cuda() if with_bias else None
    big = torch.full((M, N + 24), -7.0, dtype=torch.bfloat16, device="cuda")
    yb = V.qgemm_mx(a, wd, bias_d, "bf16", y=big[:, :N])
    yf = V.qgemm_mx(a, wd, bias_d, "f32")
    torch.cuda.synchronize()
    got = host_bits(big)
    assert np.array_equal(got[:, :N], F.f32_to_bf16(yf.cpu().numpy())), "bf16 != RNE(f32)"
    assert (got[:, N:] == F.f32_to_bf16(np.float32(-7.0))).all(), "padding written"
    rows = np.r_[0:3, 255:258, M - 4:M]
    ref = Q.hadamard_quantize(x_bits[rows], 64, fmt)
    wq_o, ws_o = Q.prepare_weight_mx(w_bits, 64)
    e64, _ = G.qgemm_mx(ref["q"], ref["scales"], fmt, wq_o, ws_o, bias_h, "f32")
    terms = terms_mx(ref["q"], ref["scales"], fmt, wq_o, ws_o, bias_h)
    assert_elementwise(yf.cpu().numpy()[rows], e64, terms, K, "f32", f"ragged edges {fmt}")


def test_gemm_rejects_unsupported_k():
    need_gpu()
    a = V.MXTensor(torch.zeros((4, 48), dtype=torch.uint8, device="cuda"),
                   torch.zeros((4, 3), dtype=torch.uint8, device="cuda"), "mxfp4")
    w = V.MXTensor(torch.zeros((8, 48), dtype=torch.uint8, device="cuda"),
                   torch.zeros((8, 3), dtype=torch.uint8, device="cuda"), "mxfp4")
    with pytest.raises(V.VdtqError) as e:
        V.qgemm_mx(a, w)
    assert e.value.code == 2
