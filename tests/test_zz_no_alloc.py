"""hadamard_quantize_noalloc (the entry point for callers that cannot
allocate) against hadamard_quantize with a caller-given workspace, through
the C ABI: codes, scales, tensor scale and statistics bit for bit, on two
calls in a row, the second with a smaller input, in every format that uses
the scratch array (NVFP4 with the tensor amax computed, statistics, the
GELU table)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from video_diffusion_transformer_block_amd import _lib as L
from helpers import dev_bf16, need_gpu, log

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _outputs(M, K, fmt, dev):
    if fmt == L.FMT_NVFP4:
        return (torch.full((M, K // 2), 0xAA, dtype=torch.uint8, device=dev),
                torch.full((M, K // 16), 0xAA, dtype=torch.uint8, device=dev),
                torch.full((2,), -1.0, dtype=torch.float32, device=dev))
    if fmt == L.FMT_INT8:
        return (torch.full((M, K), 99, dtype=torch.int8, device=dev),
                torch.full((M,), -1.0, dtype=torch.float32, device=dev), None)
    if fmt == L.FMT_BF16:
        return torch.full((M, K), 7.0, dtype=torch.bfloat16, device=dev), None, None
    width = K // 2 if fmt == L.FMT_MXFP4 else K
    return (torch.full((M, width), 0xAA, dtype=torch.uint8, device=dev),
            torch.full((M, K // 32), 0xAA, dtype=torch.uint8, device=dev), None)


def _call(x, fmt, flags, noalloc):
    M, K = x.shape
    dev = x.device
    q, s, ts = _outputs(M, K, fmt, dev)
    st = torch.full((4,), -1.0, dtype=torch.float64, device=dev) if flags & L.STATS else None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = L.lib()
    if noalloc:
        rc = lib.hadamard_quantize_noalloc(_p(x), M, K, x.stride(0), 64, fmt, flags, _p(q), _p(s), _p(ts), _p(st),
                                           stream)
    else:
        nbytes = lib.vdtq_workspace_bytes(L.OP_HADAMARD_QUANTIZE, M, K)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        rc = lib.hadamard_quantize(_p(x), M, K, x.stride(0), 64, fmt, flags, _p(q), _p(s), _p(ts), _p(st),
                                   _p(ws), ws.numel(), stream)
    assert rc == L.OK, lib.vdtq_last_error()
    return [t for t in (q, s, ts, st) if t is not None]


CASES = [(L.FMT_NVFP4, L.STATS), (L.FMT_NVFP4, 0), (L.FMT_INT8, L.STATS), (L.FMT_BF16, L.STATS | L.GELU),
         (L.FMT_MXFP4, L.STATS | L.GELU), (L.FMT_MXFP8, L.GELU)]


@pytest.mark.parametrize("fmt,flags", CASES)
def test_noalloc_matches_workspace_call(fmt, flags):
    need_gpu()
    big = dev_bf16(synth.laplace_activations(17776, 3072, 1000, 3000))       # 5B QKV input
    small = dev_bf16(synth.laplace_activations(300, 1024, 1001, 3001))
    for x in (big, small):                                                     # second call smaller
        log(f"noalloc fmt={fmt} flags={flags} M={x.shape[0]} K={x.shape[1]}")
        got = _call(x, fmt, flags, noalloc=True)
        want = _call(x, fmt, flags, noalloc=False)
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert torch.equal(g.view(torch.uint8), w.view(torch.uint8))

