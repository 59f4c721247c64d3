"""CPU tests of the binding's checks on caller-given buffers: a buffer of the
wrong dtype, shape, stride or device raises ValueError before the library is
called, so no kernel can read or write past it.  The library is replaced by
a stub that fails the test if a launching entry point is reached, and the
binding's device type is set to "cpu" so that host tensors stand in for
device memory."""
import pytest
import torch

from video_diffusion_transformer_block_amd import _lib as L
from video_diffusion_transformer_block_amd import ops as O

class _StubLib:
    """vdtq_workspace_bytes answers; every other entry point records its
    call and returns VDTQ_OK without doing anything."""

    def __init__(self):
        self.calls = []

    def vdtq_workspace_bytes(self, op, m, k):
        return 4096

    def __getattr__(self, name):
        def call(*args):
            self.calls.append(name)
            return 0
        return call


@pytest.fixture
def stub(monkeypatch):
    s = _StubLib()
    monkeypatch.setattr(O, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(L, "lib", lambda: s)
    monkeypatch.setattr(O, "_stream", lambda dev: None)
    monkeypatch.setattr(O, "_ws", {})
    monkeypatch.setattr(O, "_gemm_ws", {})
    monkeypatch.setattr(O, "_bs_ws", {})
    return s


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def nv(R, K):
    return O.NVFP4Tensor(u8(R, K // 2), u8(R, K // 16), torch.zeros(2, dtype=torch.float32))


def mx(R, K, fmt="mxfp4"):
    return O.MXTensor(u8(R, K // 2 if fmt == "mxfp4" else K), u8(R, K // 32), fmt)


M, N, K = 8, 64, 128


def test_valid_buffers_reach_the_library(stub):
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    O.hadamard_quantize(x, 64, "nvfp4", out=nv(M, K))
    O.hadamard_quantize(x, 64, "int8")
    O.qgemm_w4a4(nv(M, K), nv(N, K), torch.zeros(N), "bf16", y=torch.zeros((M, N), dtype=torch.bfloat16))
    O.qgemm_w4a4(nv(M, K), nv(N, K), None, "f32", y=torch.zeros((M, 2 * N))[:, :N])    # ldy = 2N
    O.qgemm_w4a8(O.INT8Tensor(torch.zeros((M, K), dtype=torch.int8), torch.zeros(M)), nv(N, K))
    O.qgemm_w4a16(O.BF16Tensor(torch.zeros((M, K), dtype=torch.bfloat16)), nv(N, K))
    O.qgemm_mx(mx(M, K, "mxfp8"), mx(N, K))
    O.qgemm_mx_quant(mx(M, K), mx(N, K), out=mx(M, N))
    d = torch.zeros((M, N), dtype=torch.bfloat16)
    O.block_stats(d, d.clone(), d.clone(), d.clone())
    O.block_stats_mx8(d, d.clone(), _mx_flat(M * N), None)
    assert stub.calls == ["hadamard_quantize", "hadamard_quantize", "qgemm_w4a4", "qgemm_w4a4", "qgemm_w4a8",
                          "qgemm_w4a16", "qgemm_mx", "qgemm_mx_quant", "block_stats", "block_stats_mx8"]


def _mx_flat(n):
    return O.MXTensor(u8(n), u8(n // 32), "mxfp8")


BAD_GEMM = {
    "y too few rows": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K), y=torch.zeros((M - 1, N), dtype=torch.bfloat16)),
    "y wrong dtype": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K), None, "f32", y=torch.zeros((M, N), dtype=torch.bfloat16)),
    "y bf16 for f32": lambda: O.qgemm_w4a8(O.INT8Tensor(torch.zeros((M, K), dtype=torch.int8), torch.zeros(M)),
                                          nv(N, K), None, "f32", y=torch.zeros((M, N), dtype=torch.bfloat16)),
    "y column stride": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K), y=torch.zeros((N, M), dtype=torch.bfloat16).t()),
    "bad out_dtype": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K), None, "fp8"),
    "a scales short": lambda: O.qgemm_w4a4(O.NVFP4Tensor(u8(M, K // 2), u8(M, K // 32), torch.zeros(2)), nv(N, K)),
    "a ts short": lambda: O.qgemm_w4a4(O.NVFP4Tensor(u8(M, K // 2), u8(M, K // 16), torch.zeros(1)), nv(N, K)),
    "w K mismatch": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K // 2)),
    "w scales short": lambda: O.qgemm_w4a4(nv(M, K), O.NVFP4Tensor(u8(N, K // 2), u8(N - 1, K // 16), torch.zeros(2))),
    "bias short": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K), torch.zeros(N - 1)),
    "bias dtype": lambda: O.qgemm_w4a4(nv(M, K), nv(N, K), torch.zeros(N, dtype=torch.float64)),
    "int8 scales short": lambda: O.qgemm_w4a8(O.INT8Tensor(torch.zeros((M, K), dtype=torch.int8), torch.zeros(M - 1)),
                                              nv(N, K)),
    "int8 codes dtype": lambda: O.qgemm_w4a8(O.INT8Tensor(u8(M, K), torch.zeros(M)), nv(N, K)),
    "a16 not contiguous": lambda: O.qgemm_w4a16(
        O.BF16Tensor(torch.zeros((K, M), dtype=torch.bfloat16).t()), nv(N, K)),
    "mx scales short": lambda: O.qgemm_mx(O.MXTensor(u8(M, K // 2), u8(M, K // 64), "mxfp4"), mx(N, K)),
    "mx codes for mxfp8 short": lambda: O.qgemm_mx(O.MXTensor(u8(M, K // 2), u8(M, K // 32), "mxfp8"), mx(N, K)),
    "mx quant out short": lambda: O.qgemm_mx_quant(mx(M, K), mx(N, K), out=mx(M - 1, N)),
    "mx quant out fmt": lambda: O.qgemm_mx_quant(mx(M, K), mx(N, K), out_fmt="mxfp4", out=mx(M, N, "mxfp8")),
}

BAD_QUANT = {
    "nvfp4 out codes short": lambda x: O.hadamard_quantize(
        x, 64, "nvfp4", out=O.NVFP4Tensor(u8(M - 1, K // 2), u8(M, K // 16), torch.zeros(2))),
    "nvfp4 out scales short": lambda x: O.hadamard_quantize(
        x, 64, "nvfp4", out=O.NVFP4Tensor(u8(M, K // 2), u8(M, K // 32), torch.zeros(2))),
    "int8 out scales short": lambda x: O.hadamard_quantize(
        x, 64, "int8", out=O.INT8Tensor(torch.zeros((M, K), dtype=torch.int8), torch.zeros(M - 1))),
    "int8 out codes dtype": lambda x: O.hadamard_quantize(x, 64, "int8", out=O.INT8Tensor(u8(M, K), torch.zeros(M))),
    "bf16 out short": lambda x: O.hadamard_quantize(
        x, 64, "bf16", out=O.BF16Tensor(torch.zeros((M, K // 2), dtype=torch.bfloat16))),
    "mx out short": lambda x: O.hadamard_quantize(x, 64, "mxfp8", out=mx(M, K, "mxfp4")),
    "stats short": lambda x: O.hadamard_quantize(
        x, 64, "nvfp4", stats=True, out=O.NVFP4Tensor(u8(M, K // 2), u8(M, K // 16), torch.zeros(2),
                                                     torch.zeros(2, dtype=torch.float64))),
    "K not a multiple of 16": lambda x: O.hadamard_quantize(x[:, :120], 8, "int8"),
    "x wrong dtype": lambda x: O.hadamard_quantize(x.float(), 64, "int8"),
}


@pytest.mark.parametrize("case", sorted(BAD_GEMM))
def test_gemm_rejects_bad_buffers(stub, case):
    with pytest.raises(ValueError):
        BAD_GEMM[case]()
    assert stub.calls == []


@pytest.mark.parametrize("case", sorted(BAD_QUANT))
def test_quantize_rejects_bad_buffers(stub, case):
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        BAD_QUANT[case](x)
    assert stub.calls == []


def test_block_stats_rejects_bad_buffers(stub):
    d = torch.zeros((M, N), dtype=torch.bfloat16)
    bad = [
        lambda: O.block_stats(d, d, torch.zeros((M, N - 8), dtype=torch.bfloat16)),      # dprev short
        lambda: O.block_stats(d, d, None, torch.zeros((M, N), dtype=torch.float32)),     # dnew dtype
        lambda: O.block_stats(d, d, d, d),                                                # dnew aliases dprev
        lambda: O.block_stats(d, d[:, :N // 2]),                                          # out shape
        lambda: O.block_stats_mx8(d, d, _mx_flat(M * N // 2)),                            # dprev short
        lambda: O.block_stats_mx8(d, d, None, O.MXTensor(u8(M * N), u8(M * N // 64), "mxfp8")),   # scales short
        lambda: O.block_stats_mx8(d, d, mx(M, N)),                                        # not mxfp8
        lambda: O.block_stats_mx8(d[:, :8], d[:, :8].clone()),                            # n % 32 (not contiguous)
    ]
    for f in bad:
        with pytest.raises(ValueError):
            f()
    assert stub.calls == []


def test_cpu_tensors_are_refused_without_the_stub():
    """With the real device type, host tensors never reach the library."""
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        O.hadamard_quantize(x, 64, "int8")
    with pytest.raises(ValueError, match="device tensor"):
        O.qgemm_w4a4(nv(M, K), nv(N, K))
