"""GPU parity of hadamard_quantize against the oracle: codes, scales and the
tensor scale bit-exact; fused statistics within 1e-5 relative (maxima exact)."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import formats as F, hadamard as H, quant as Q
from helpers import dev_bf16, need_gpu, log

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(21))


def oracle_every_row(x_bits, b, chunk=2048):
    """The tensor amax and the four outlier statistics over every row of a
    large input, from the oracle's transform chunk by chunk (the maxima
    combine exactly, the fp64 sums in row-chunk order)."""
    M = x_bits.shape[0]
    amax = np.float32(0)
    st = np.zeros(4)
    for r0 in range(0, M, chunk):
        xc = x_bits[r0:r0 + chunk]
        y = H.block_hadamard_bf16(xc, b)
        amax = max(amax, np.float32(np.abs(y).max()) if y.size else np.float32(0))
        c = Q.activation_stats(xc, y)
        st = np.array([max(st[0], c[0]), st[1] + c[1], max(st[2], c[2]), st[3] + c[3]])
    return amax, st


def check_stats(got, want):
    assert got[0] == want[0] and got[2] == want[2], (got, want)
    assert np.allclose(got[[1, 3]], want[[1, 3]], rtol=1e-5, atol=0), (got, want)


def run_and_compare(x_bits, b, fmt, amax=None, stats=True, ldx_pad=0, rows=None):
    M, K = x_bits.shape
    log(f"hq case M={M} K={K} b={b} fmt={fmt} amax={amax} pad={ldx_pad} stats={stats} "
        f"rows={'all' if rows is None else len(rows)}")
    if ldx_pad:
        big = np.zeros((M, K + ldx_pad), np.uint16)
        big[:, :K] = x_bits
        xd = dev_bf16(big)[:, :K]
    else:
        xd = dev_bf16(x_bits)
    r = V.hadamard_quantize(xd, had_block=b, fmt=fmt, amax=amax, stats=stats)
    torch.cuda.synchronize()
    sel = np.arange(M) if rows is None else rows
    # the tensor amax and the statistics need every row; the codes are row-local
    full = oracle_every_row(x_bits, b) if rows is not None else None
    if fmt == "nvfp4":
        ya = None
        if amax is None:
            ya = full[0] if full is not None else oracle_every_row(x_bits, b)[0]
        ref = Q.hadamard_quantize(x_bits[sel], b, "nvfp4", amax=ya if amax is None else amax)
        ts = r.ts.cpu().numpy()
        assert ts[0] == ref["amax"] or (np.isnan(ts[0]) and np.isnan(ref["amax"])), (ts, ref["amax"])
        assert ts[1] == ref["gs"], (ts, ref["gs"])
        q = r.q.cpu().numpy()[sel]
        s = r.scales.cpu().numpy()[sel]
        bad = np.nonzero((q != ref["q"]).any(1) | (s != ref["scales"]).any(1))[0]
        assert len(bad) == 0, f"rows {sel[bad[:5]]} differ"
    else:
        ref = Q.hadamard_quantize(x_bits[sel], b, "int8")
        q = r.q.cpu().numpy()[sel]
        s = r.scales.cpu().numpy()[sel]
        assert np.array_equal(s.view(np.uint32), ref["scales"].view(np.uint32))
        assert np.array_equal(q, ref["q"])
    if stats:
        check_stats(r.stats.cpu().numpy(), ref["stats"] if rows is None else full[1])
    return r


@pytest.mark.parametrize("fmt", ["nvfp4", "int8"])
@pytest.mark.parametrize("b", [16, 32, 64, 128, 256])
def test_tiny_layer_all_blocks(fmt, b):
    need_gpu()
    d = synth.tiny_layer()
    run_and_compare(d["x"], b, fmt)


@pytest.mark.parametrize("M,K,b,pad", [(1, 64, 64, 0), (3, 256, 64, 8), (257, 320, 64, 0), (1000, 192, 64, 0),
                                       (33, 80, 16, 0), (7, 48, 16, 8), (65, 96, 32, 0), (129, 384, 128, 0),
                                       (5, 768, 256, 16), (300, 1920, 64, 0), (2, 16, 16, 0)])
@pytest.mark.parametrize("fmt", ["nvfp4", "int8"])
def test_ragged_shapes(M, K, b, pad, fmt):
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32) * 2)
    run_and_compare(x, b, fmt, ldx_pad=pad)


def test_degenerate_inputs():
    need_gpu()
    K = 128
    z = np.zeros((5, K), np.uint16)
    for fmt in ("nvfp4", "int8"):
        run_and_compare(z, 64, fmt)                               # all zero
    x = synth.to_bf16_bits(RNG.standard_normal((6, K)).astype(np.float32))
    x[2] = 0                                                      # a zero row
    x[4, :64] = 0x8000                                            # -0.0 block
    for fmt in ("nvfp4", "int8"):
        run_and_compare(x, 64, fmt)
    # huge dynamic range: subnormal E4M3 scales and groups that round to 0
    y = RNG.standard_normal((4, 256)).astype(np.float32)
    y[0, 0] = 3.0e4
    y[1] *= 2.0 ** -14
    y[2] *= 2.0 ** -24
    run_and_compare(synth.to_bf16_bits(y), 64, "nvfp4")
    # values near the bf16 maximum / minimum normal
    y = RNG.standard_normal((2, 64)).astype(np.float32) * 1e30
    run_and_compare(synth.to_bf16_bits(y), 64, "nvfp4")
    run_and_compare(synth.to_bf16_bits(y), 64, "int8")
    y = RNG.standard_normal((2, 64)).astype(np.float32) * 1e-36
    run_and_compare(synth.to_bf16_bits(y), 16, "int8")
    run_and_compare(synth.to_bf16_bits(y), 16, "nvfp4")


@pytest.mark.parametrize("scale", [1.0, 0.25, 0.0, float("inf"), float("nan"), 2.0 ** -101, 4.0])
def test_given_amax(scale):
    need_gpu()
    d = synth.tiny_layer()
    true = np.float32(np.abs(H.block_hadamard_bf16(d["x"], 64)).max())
    run_and_compare(d["x"], 64, "nvfp4", amax=float(true * np.float32(scale)))


def test_empty_rows():
    need_gpu()
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    r = V.hadamard_quantize(x, 64, "nvfp4", stats=True)
    assert r.q.shape == (0, 64) and r.ts.cpu().tolist() == [0.0, 1.0]
    assert r.stats.cpu().tolist() == [0, 0, 0, 0]
    r = V.hadamard_quantize(x, 64, "int8")
    assert r.q.shape == (0, 128)


def test_repeatable():
    need_gpu()
    x = dev_bf16(synth.laplace_activations(2048, 3072, 1, 2))
    a = V.hadamard_quantize(x, 64, "nvfp4", stats=True)
    b = V.hadamard_quantize(x, 64, "nvfp4", stats=True)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.scales, b.scales) and torch.equal(a.stats, b.stats)


@pytest.mark.parametrize("fmt,K", [("nvfp4", 3072), ("int8", 3072), ("nvfp4", 12288), ("int8", 12288)])
def test_cogvideox_5b_shapes_sampled(fmt, K):
    """Full 5B-shaped activations (M = 17776); codes compared on sampled rows
    (first and last row included), the tensor amax over every row."""
    need_gpu()
    M = synth.TOKENS_2B_5B
    name = "ffn_down" if K == 12288 else "qkv"
    x, _ = synth.layer_inputs(M, name, K, 16)
    run_and_compare(x, 64, fmt, rows=synth.row_sample(M, 256), stats=True)


@pytest.mark.parametrize("fmt,K", [("nvfp4", 1920), ("int8", 1920), ("nvfp4", 7680), ("int8", 7680)])
def test_cogvideox_2b_shapes_sampled(fmt, K):
    """CogVideoX-2B-shaped activations (M = 17776, hidden 1920, FFN 7680)."""
    need_gpu()
    M = synth.TOKENS_2B_5B
    name = "ffn_down" if K == 7680 else "qkv"
    x, _ = synth.layer_inputs(M, name, K, 16)
    run_and_compare(x, 64, fmt, rows=synth.row_sample(M, 256), stats=True)


@pytest.mark.parametrize("K", [3072, 12288])
def test_fused_stats_5b_every_format(K):
    """The fused statistics at the 5B shapes in every activation format
    (NVFP4, INT8, BF16, MXFP4, MXFP8), against the oracle over every row.
    These grids hold 4444 to 26664 workgroup partials, more than one pass of
    the final reduction's 4096-partial loop; the codes of the BF16 and MX
    formats are compared on sampled rows as well.  NVFP4 runs twice: with
    the tensor amax computed (the statistics come from the amax pre-pass)
    and with it supplied (from the quantize pass)."""
    need_gpu()
    M = synth.TOKENS_2B_5B
    name = "ffn_down" if K == 12288 else "qkv"
    x, _ = synth.layer_inputs(M, name, K, 16)
    amax_o, want = oracle_every_row(x, 64)
    rows = synth.row_sample(M, 64)
    xd = dev_bf16(x)
    for fmt in ("nvfp4", "int8", "bf16", "mxfp4", "mxfp8"):
        log(f"stats 5B K={K} fmt={fmt}")
        r = V.hadamard_quantize(xd, 64, fmt, stats=True)
        torch.cuda.synchronize()
        check_stats(r.stats.cpu().numpy(), want)
        if fmt == "nvfp4":
            assert r.ts.cpu().numpy()[0] == amax_o
            log(f"stats 5B K={K} fmt=nvfp4, amax supplied")
            rg = V.hadamard_quantize(xd, 64, fmt, amax=float(amax_o), stats=True)
            torch.cuda.synchronize()
            check_stats(rg.stats.cpu().numpy(), want)
            assert torch.equal(rg.q, r.q) and torch.equal(rg.scales, r.scales)
        if fmt in ("bf16", "mxfp4", "mxfp8"):
            ref = Q.hadamard_quantize(x[rows], 64, fmt)
            if fmt == "bf16":
                assert np.array_equal(r.q.view(torch.int16).cpu().numpy().view(np.uint16)[rows], ref["q"])
            else:
                assert np.array_equal(r.q.cpu().numpy()[rows], ref["q"])
                assert np.array_equal(r.scales.cpu().numpy()[rows], ref["scales"])


def test_fused_stats_more_partials_than_one_pass_all_rows():
    """M = 12000, K = 3072: 4500 NVFP4 and 3000 INT8 workgroup partials;
    codes and statistics compared on every row."""
    need_gpu()
    x = synth.laplace_activations(12000, 3072, 77, 78)
    for fmt in ("nvfp4", "int8"):
        run_and_compare(x, 64, fmt, stats=True)
