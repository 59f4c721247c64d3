"""Maximum sizes: activation operands of 4 GB and more.

A 540000 x 16384 bf16 input (17.7 GB) quantizes to 8.8 GB of INT8 codes
and 4.4 GB of NVFP4 codes.  Both are past the 32-bit byte offsets of the
pipelined GEMM, so qgemm_w4a8 and qgemm_w4a4 take the general kernel with
64-bit row offsets; the quantize pass addresses the input through
per-workgroup bases.  The input is a seeded 2048-row block (the Laplace
recipe with outlier channels) repeated down the rows, so the oracle knows
every row: the tensor amax is the block's, and the sampled rows include the
ones on both sides of each 4 GB boundary.  qgemm_w4a16 and qgemm_mx refuse
such operands with VDTQ_EUNSUPPORTED before any launch."""
import numpy as np
import pytest
import torch

import synth
import video_diffusion_transformer_block_amd as V
from oracle import gemm as G, hadamard as H, quant as Q
from helpers import assert_elementwise, log, need_gpu, rel_fro, terms_w4a4, terms_w4a8

pytestmark = pytest.mark.gpu
B = 64
M, K, N, R = 540000, 16384, 64, 2048


def test_operands_beyond_4gb():
    need_gpu()
    assert M * K >= 2 ** 32 and M * K // 2 >= 2 ** 32
    block = synth.laplace_activations(R, K, 1950, 3950)
    w = synth.normal_matrix(N, K, 0.02, 2950)
    rows = np.unique(np.concatenate([
        [0, 1, R - 1, R, 2 ** 32 // K - 1, 2 ** 32 // K, 2 ** 32 // (K // 2) - 1, 2 ** 32 // (K // 2),
         2 ** 32 // (K // 2) + 1, M - 1], synth.row_sample(M, 12, seed=29)]))
    log(f"large operands: M={M} K={K} N={N}, {M * K * 2 / 2 ** 30:.1f} GiB of bf16 input")
    xb = torch.from_numpy(np.ascontiguousarray(block).view(np.int16)).view(torch.bfloat16).cuda()
    x = xb.repeat((M + R - 1) // R, 1)[:M]
    del xb
    wq_o, ws_o, wgs_o = Q.prepare_weight(w, B)
    wd = V.NVFP4Tensor(torch.from_numpy(wq_o).cuda(), torch.from_numpy(ws_o).cuda(),
                       torch.tensor(np.array([np.float32(0), wgs_o], np.float32)).cuda())
    a8 = V.hadamard_quantize(x, B, "int8")
    a4 = V.hadamard_quantize(x, B, "nvfp4")
    sel = torch.from_numpy(rows).cuda()
    y8 = V.qgemm_w4a8(a8, wd, None, "f32")[sel]
    y4 = V.qgemm_w4a4(a4, wd, None, "f32")[sel]
    torch.cuda.synchronize()
    log("  library done; oracle on the block and the sampled rows")

    # the tensor amax: every row repeats a row of the block
    amax_o = np.float32(np.abs(H.block_hadamard_bf16(block, B)).max())
    assert a4.ts.cpu().numpy()[0] == amax_o
    hb = block[rows % R]
    r4 = Q.hadamard_quantize(hb, B, "nvfp4", amax=amax_o)
    r8 = Q.hadamard_quantize(hb, B, "int8")
    assert a4.ts.cpu().numpy()[1] == r4["gs"]
    assert np.array_equal(a4.q[sel].cpu().numpy(), r4["q"])
    assert np.array_equal(a4.scales[sel].cpu().numpy(), r4["scales"])
    assert np.array_equal(a8.q[sel].cpu().numpy(), r8["q"])
    assert np.array_equal(a8.scales[sel].cpu().numpy().view(np.uint32), r8["scales"].view(np.uint32))

    x4, _ = G.qgemm_w4a4(r4["q"], r4["scales"], r4["gs"], wq_o, ws_o, wgs_o, None, "f32")
    x8, _ = G.qgemm_w4a8(r8["q"], r8["scales"], wq_o, ws_o, wgs_o, None, "f32")
    h4, h8 = y4.cpu().numpy(), y8.cpu().numpy()
    q4 = assert_elementwise(h4, x4, terms_w4a4(r4["q"], r4["scales"], r4["gs"], wq_o, ws_o, wgs_o, None), K,
                            "f32", "w4a4 f32")
    q8 = assert_elementwise(h8, x8, terms_w4a8(r8["q"], r8["scales"], wq_o, ws_o, wgs_o, None), K,
                            "f32", "w4a8 f32")
    e4, e8 = rel_fro(h4, x4), rel_fro(h8, x8)
    log(f"  w4a4 f32 rel {e4:.2e} (err/bound {q4:.3f}), w4a8 f32 rel {e8:.2e} (err/bound {q8:.3f})")
    assert e4 < 1e-5 and e8 < 1e-5

    # the W4A16 and MX GEMMs keep 32-bit offsets and refuse such operands
    with pytest.raises(V.VdtqError, match="4 GB"):
        V.qgemm_w4a16(V.BF16Tensor(x), wd)
    wm = V.MXTensor(torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda"),
                    torch.zeros((N, K // 32), dtype=torch.uint8, device="cuda"), "mxfp4")
    am = V.MXTensor(a4.q, torch.zeros((M, K // 32), dtype=torch.uint8, device="cuda"), "mxfp4")
    with pytest.raises(V.VdtqError, match="4 GB"):
        V.qgemm_mx(am, wm)
