"""GPU parity of qgemm_mx_quant, the MX GEMM whose epilogue emits the next
linear's MX activation (bias, optional GELU, 64-point Hadamard, MX
encoding).

  * against the unfused GPU chain qgemm_mx (bf16) -> hadamard_quantize:
    codes and scales bit-exact wherever the unfused GEMM keeps its tiles
    whole (it splits a partial last wave along K, summing in another
    order; those tile rows are left out, found by the same work split);
  * against the oracle chain: bit-exact when every partial sum of the
    product is exact (the GEMM result then has one correct value); at the
    FFN-up shape of the 5B block, on sampled rows, the share of differing
    codes and the dequantized error stay at the level that bf16 rounding
    flips of the GEMM output explain."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import formats as F, gemm as G, quant as Q
from helpers import dev_bf16, host_bits, need_gpu, rel_fro, log

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(71))


def mx_dev(q, s, fmt):
    return V.MXTensor(torch.from_numpy(np.ascontiguousarray(q)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(s)).cuda(), fmt)


def split_tile_rows(M, N, K):
    """Tile rows (256 tokens each) holding a tile that qgemm_mx splits along K:
    the host work split of the MX GEMM (whole waves of 256 x 256 tiles run
    data-parallel, a partial last wave is cut into K slices when that is
    estimated to finish sooner), with tiles numbered in groups of 8 tile
    rows, column-major inside a group."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm_n, tn_n, nk = -(-M // 256), -(-N // 256), K // 128
    tiles, G_ = tm_n * tn_n, max(1, min(cus, 256))
    left = tiles % G_
    slices = min(G_ // left, nk) if left else 0
    slice_nk = -(-nk // slices) if slices else 0
    if slices:
        slices = -(-nk // slice_nk)
    split = slices >= 2 and slice_nk + 3 < nk
    rows = set()
    for t in range(left if split else 0):
        g = t // (8 * tn_n)
        gsz = min(tm_n - 8 * g, 8)
        rows.add(8 * g + (t - g * 8 * tn_n) % gsz)
    return rows


def unfused(a, w, bias, out_fmt, gelu):
    y = V.qgemm_mx(a, w, bias, "bf16")
    return V.hadamard_quantize(y, 64, out_fmt, gelu=gelu)


def compare_rows(got, want, rows):
    gq, gs = got.q.cpu().numpy()[rows], got.scales.cpu().numpy()[rows]
    wq, ws = want.q.cpu().numpy()[rows], want.scales.cpu().numpy()[rows]
    bad = np.nonzero((gq != wq).any(1) | (gs != ws).any(1))[0]
    assert len(bad) == 0, f"rows {np.asarray(rows)[bad[:5]]} differ"


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (257, 320, 256), (300, 640, 512), (64, 4096, 384)])
@pytest.mark.parametrize("a_fmt,out_fmt", [("mxfp4", "mxfp4"), ("mxfp8", "mxfp4"), ("mxfp4", "mxfp8"),
                                           ("mxfp8", "mxfp8")])
def test_matches_unfused_chain(M, N, K, a_fmt, out_fmt):
    need_gpu()
    log(f"mx_quant vs chain M={M} N={N} K={K} {a_fmt}->{out_fmt}")
    x = dev_bf16(synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32)))
    w = dev_bf16(synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.05))
    a = V.hadamard_quantize(x, 64, a_fmt)
    wq = V.hadamard_quantize(w, 64, "mxfp4")
    bias = torch.from_numpy(RNG.standard_normal(N).astype(np.float32)).cuda()
    assert not split_tile_rows(M, N, K)
    for gelu in (True, False):
        for b in (bias, None):
            got = V.qgemm_mx_quant(a, wq, b, out_fmt, gelu=gelu)
            want = unfused(a, wq, b, out_fmt, gelu)
            torch.cuda.synchronize()
            assert torch.equal(got.q, want.q) and torch.equal(got.scales, want.scales), (gelu, b is None)


@pytest.mark.parametrize("out_fmt", ["mxfp4", "mxfp8"])
def test_exact_sums_match_oracle(out_fmt):
    """Random MXFP4 codes with scale bytes 121..124 and a dyadic bias: every
    product is a multiple of 2^-14 and every partial sum stays below 2^10,
    so acc + bias is exact; the fused output must equal the oracle chain's
    bit for bit (GELU, Hadamard and MX encoding included)."""
    need_gpu()
    M, N, K = 300, 640, 1024
    ac = RNG.integers(0, 16, size=(M, K)).astype(np.uint8)
    a_s = RNG.integers(121, 125, size=(M, K // 32)).astype(np.uint8)
    wc = RNG.integers(0, 16, size=(N, K)).astype(np.uint8)
    w_s = RNG.integers(121, 125, size=(N, K // 32)).astype(np.uint8)
    bias = (RNG.integers(-512, 512, size=N) / 256.0).astype(np.float32)
    aq, wq = F.pack_nibbles(ac), F.pack_nibbles(wc)
    y_bits = G.qgemm_mx(aq, a_s, "mxfp4", wq, w_s, bias, "bf16")[1]
    vals = F.bf16_to_f32(y_bits)
    log(f"  GEMM output range {vals.min():.3g} .. {vals.max():.3g}, "
        f"{np.mean((vals > -10) & (vals < 2.75)):.2f} in GELU's non-trivial band")
    for gelu in (True, False):
        ref = Q.hadamard_quantize(y_bits, 64, out_fmt, gelu=gelu)
        got = V.qgemm_mx_quant(mx_dev(aq, a_s, "mxfp4"), mx_dev(wq, w_s, "mxfp4"), torch.from_numpy(bias).cuda(),
                               out_fmt, gelu=gelu)
        torch.cuda.synchronize()
        assert np.array_equal(got.q.cpu().numpy(), ref["q"]), gelu
        assert np.array_equal(got.scales.cpu().numpy(), ref["scales"]), gelu


def test_ffn_up_5b():
    """FFN-up of the 5B block (17776 x 3072 -> 12288, MXFP8 activations in,
    MXFP4 FFN-down activations out, GELU): bit-exact against the unfused
    GPU chain on every row of the tiles it keeps whole; against the oracle
    chain on sampled rows."""
    need_gpu()
    M = synth.TOKENS_2B_5B
    K, N = 3072, 12288
    x, w = synth.layer_inputs(M, "ffn_up", K, N)
    bias_h = (RNG.standard_normal(N) * 0.1).astype(np.float32)
    bias = torch.from_numpy(bias_h).cuda()
    a = V.hadamard_quantize(dev_bf16(x), 64, "mxfp8")
    wq = V.hadamard_quantize(dev_bf16(w), 64, "mxfp4")
    got = V.qgemm_mx_quant(a, wq, bias, "mxfp4", gelu=True)
    want = unfused(a, wq, bias, "mxfp4", True)
    again = V.qgemm_mx_quant(a, wq, bias, "mxfp4", gelu=True)
    torch.cuda.synchronize()
    assert torch.equal(got.q, again.q) and torch.equal(got.scales, again.scales)
    skip = split_tile_rows(M, N, K)
    rows = np.array([r for r in range(M) if r // 256 not in skip])
    log(f"ffn_up 5B: {len(rows)} of {M} rows outside split tile rows {sorted(skip)}")
    compare_rows(got, want, rows)

    sel = synth.row_sample(M, 16)
    ra = Q.hadamard_quantize(x[sel], 64, "mxfp8")
    wo_q, wo_s = Q.prepare_weight_mx(w, 64)
    y_bits = G.qgemm_mx(ra["q"], ra["scales"], "mxfp8", wo_q, wo_s, bias_h, "bf16")[1]
    ref = Q.hadamard_quantize(y_bits, 64, "mxfp4", gelu=True)
    gq, gs = got.q.cpu().numpy()[sel], got.scales.cpu().numpy()[sel]
    code_diff = np.mean(F.unpack_nibbles(gq) != F.unpack_nibbles(ref["q"]))
    scale_diff = np.mean(gs != ref["scales"])
    deq_got = Q.mx_dequantize(gq, gs, "e2m1")
    deq_ref = Q.mx_dequantize(ref["q"], ref["scales"], "e2m1")
    err = rel_fro(deq_got, deq_ref)
    log(f"  vs oracle chain: codes differ {code_diff:.2e}, scales {scale_diff:.2e}, dequantized rel {err:.2e}")
    assert code_diff < 1e-2 and scale_diff < 1e-2 and err < 2e-2
