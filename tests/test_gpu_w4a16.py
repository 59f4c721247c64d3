"""GPU parity of the full-precision fallback: the BF16 output of
hadamard_quantize (bit-exact against the oracle's bf16 rounding of its fp32
transform) and qgemm_w4a16 (relative Frobenius error <= 2e-3 with bf16
output, <= 1e-5 with fp32 output, where only the fp32 accumulation order
differs)."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import gemm as G, hadamard as H, quant as Q
from helpers import assert_elementwise, bf16_values, dev_bf16, host_bits, need_gpu, rel_fro, log, terms_w4a16

pytestmark = pytest.mark.gpu
RNG = np.random.Generator(np.random.PCG64(31))
TOL = 2e-3


def check_bf16_pass(x_bits, b, stats=False, rows=None):
    M, K = x_bits.shape
    log(f"bf16 pass M={M} K={K} b={b} stats={stats}")
    r = V.hadamard_quantize(dev_bf16(x_bits), b, "bf16", stats=stats)
    torch.cuda.synchronize()
    sel = np.arange(M) if rows is None else rows
    ref = Q.hadamard_quantize(x_bits[sel], b, "bf16")
    got = host_bits(r.q)[sel]
    bad = np.nonzero((got != ref["q"]).any(1))[0]
    assert len(bad) == 0, f"rows {sel[bad[:5]]} differ"
    if stats and rows is None:
        st = r.stats.cpu().numpy()
        want = ref["stats"]
        assert st[0] == want[0] and st[2] == want[2], (st, want)
        assert np.allclose(st[[1, 3]], want[[1, 3]], rtol=1e-5, atol=0)
    return r


def check_w4a16(x_bits, w_bits, b=64, bias=True, rows=None, out_dtypes=("bf16", "f32")):
    M, K = x_bits.shape
    N = w_bits.shape[0]
    log(f"w4a16 case M={M} N={N} K={K} rows={'all' if rows is None else len(rows)}")
    sel = np.arange(M) if rows is None else rows
    wq_o, ws_o, wgs_o = Q.prepare_weight(w_bits, b)
    wd = V.hadamard_quantize(dev_bf16(w_bits), b, "nvfp4")
    bias_h = RNG.standard_normal(N).astype(np.float32) if bias else None
    bias_d = torch.from_numpy(bias_h).cuda() if bias else None
    a = check_bf16_pass(x_bits, b, rows=rows)
    a_ref = Q.hadamard_quantize(x_bits[sel], b, "bf16")["q"]
    terms = terms_w4a16(a_ref, wq_o, ws_o, wgs_o, bias_h)
    for od in out_dtypes:
        y = V.qgemm_w4a16(a, wd, bias_d, od)
        torch.cuda.synchronize()
        e64, r = G.qgemm_w4a16(a_ref, wq_o, ws_o, wgs_o, bias_h, od)
        if od == "bf16":
            got, want = bf16_values(host_bits(y)[sel]), bf16_values(r)
        else:
            got, want = y.cpu().numpy()[sel], e64
        err = rel_fro(got, want)
        qb = assert_elementwise(got, e64, terms, K, od, f"w4a16 {od}")
        log(f"  {od}: rel {err:.2e} (max err/bound {qb:.3f})")
        assert err <= TOL, err
        if od == "f32":
            assert err < 1e-5


@pytest.mark.parametrize("b", [16, 64, 256])
def test_bf16_pass_tiny(b):
    need_gpu()
    d = synth.tiny_layer()
    check_bf16_pass(d["x"], b, stats=True)


@pytest.mark.parametrize("M,K,b", [(1, 64, 64), (257, 320, 64), (33, 80, 16), (5, 768, 256), (1000, 192, 64)])
def test_bf16_pass_ragged(M, K, b):
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32) * 3)
    check_bf16_pass(x, b, stats=True)


def test_w4a16_tiny_layer():
    need_gpu()
    d = synth.tiny_layer()
    check_w4a16(d["x"], d["w"])
    check_w4a16(d["x"], d["w"], bias=False)


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (129, 33, 64), (300, 200, 320), (5, 300, 128),
                                   (131, 257, 256), (600, 520, 1920), (300, 260, 768)])
def test_w4a16_ragged(M, N, K):
    need_gpu()
    x = synth.to_bf16_bits(RNG.laplace(size=(M, K)).astype(np.float32))
    w = synth.to_bf16_bits(RNG.standard_normal((N, K)).astype(np.float32) * 0.02)
    check_w4a16(x, w)


def test_w4a16_integer_inputs_exact():
    """Small-integer bf16 activations, unit weight scales: fp32 sums exact."""
    need_gpu()
    M, N, K = 96, 80, 512
    a = RNG.integers(-20, 21, size=(M, K)).astype(np.float32)
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    codes = RNG.integers(0, 16, size=(N, K)).astype(np.uint8)
    from oracle import formats as F
    wq = F.pack_nibbles(codes)
    ws = np.full((N, K // 16), 0x38, np.uint8)
    w = V.NVFP4Tensor(torch.from_numpy(wq).cuda(), torch.from_numpy(ws).cuda(),
                      torch.tensor([2688.0, 1.0], dtype=torch.float32).cuda())
    y = V.qgemm_w4a16(V.BF16Tensor(dev_bf16(a_bits)), w, None, "f32")
    torch.cuda.synchronize()
    want, _ = G.qgemm_w4a16(a_bits, wq, ws, np.float32(1.0), None, "f32")
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)


def test_w4a16_rejects_k_not_multiple_of_64():
    need_gpu()
    a = V.BF16Tensor(torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda"))
    w = V.NVFP4Tensor(torch.zeros((8, 48), dtype=torch.uint8, device="cuda"),
                      torch.zeros((8, 6), dtype=torch.uint8, device="cuda"),
                      torch.tensor([0.0, 1.0], dtype=torch.float32, device="cuda"))
    with pytest.raises(V.VdtqError):
        V.qgemm_w4a16(a, w)


@pytest.mark.parametrize("name", ["qkv", "out", "ffn_up", "ffn_down"])
def test_w4a16_cogvideox_5b_sampled(name):
    need_gpu()
    M = synth.TOKENS_2B_5B
    K, N = {n: (k, nn) for n, k, nn in synth.block_linears(3072)}[name]
    x, w = synth.layer_inputs(M, name, K, N)
    check_w4a16(x, w, rows=synth.row_sample(M, 48), out_dtypes=("bf16", "f32"))
