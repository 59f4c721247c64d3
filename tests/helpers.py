"""Shared helpers for the GPU parity tests (host <-> device marshalling and
comparison metrics).  No method arithmetic lives here."""
import numpy as np
import torch

import video_diffusion_transformer_block_amd as V
from oracle import formats as F


def need_gpu():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    V.lib()  # raises if the library is missing: no fallback path exists


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_fro(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return F.bf16_to_f32(bits).astype(np.float64)


def log(msg: str):
    print(msg, flush=True)


# ------------------------------------------------- element-wise GEMM bound
# Both sides form the same exact products; the library adds them in fp32 in
# some order (MFMA tree, K slices, a reduce pass), then applies the fp32
# scale product and the bias, each one rounding.  Any order of K - 1 fp32
# additions errs by at most (K - 1) u sum|products| (u = 2^-24), and the
# scale product, the scaling and the bias add contribute a few u of
# sum|products| + |bias|.  The bound used is 2 (K + 4) u T with
# T = |scale| sum_k |a_k w_k| + |bias|; bf16 output adds its own rounding,
# at most 2^-8 of the value.  A misplaced or dropped term of ordinary size
# breaks it: T is about sqrt(K) |y|, so the bound is about 2 K^1.5 u |y|
# (2 % of |y| at K = 3072).
U32 = 2.0 ** -24


def _bias_abs(bias, N):
    return np.zeros(N) if bias is None else np.abs(np.asarray(bias, np.float64))


def terms_w4a4(a_q, a_s, a_gs, w_q, w_s, w_gs, bias):
    from oracle import quant as Q
    A = np.abs(Q.nvfp4_dequantize(a_q, a_s))
    W = np.abs(Q.nvfp4_dequantize(w_q, w_s))
    sc = abs(float(np.float32(a_gs)) * float(np.float32(w_gs)))
    return sc * (A @ W.T) + _bias_abs(bias, W.shape[0])[None, :]


def terms_w4a8(a_q, a_s, w_q, w_s, w_gs, bias):
    from oracle import quant as Q
    A = np.abs(np.asarray(a_q, np.float64))
    W = np.abs(Q.nvfp4_dequantize(w_q, w_s))
    sc = np.abs(np.asarray(a_s, np.float64))[:, None] * abs(float(np.float32(w_gs)))
    return sc * (A @ W.T) + _bias_abs(bias, W.shape[0])[None, :]


def terms_w4a16(a_bits, w_q, w_s, w_gs, bias):
    from oracle import quant as Q
    A = np.abs(F.bf16_to_f32(a_bits).astype(np.float64))
    W = np.abs(Q.nvfp4_dequantize(w_q, w_s))
    return abs(float(np.float32(w_gs))) * (A @ W.T) + _bias_abs(bias, W.shape[0])[None, :]


def terms_mx(a_q, a_s, a_fmt, w_q, w_s, bias):
    from oracle import quant as Q
    A = np.abs(Q.mx_dequantize(a_q, a_s, Q.MX_ELEM[a_fmt]))
    W = np.abs(Q.mx_dequantize(w_q, w_s, "e2m1"))
    return A @ W.T + _bias_abs(bias, W.shape[0])[None, :]


def assert_elementwise(got, exact, terms, K, out_dtype, label=""):
    """got: the library's output values (fp32, or bf16 decoded) on the
    compared rows; exact: the oracle's float64 result; terms: T above."""
    got = np.asarray(got, np.float64)
    exact = np.asarray(exact, np.float64)
    fb = 2.0 * (K + 4) * U32 * np.asarray(terms, np.float64)
    if out_dtype == "bf16":
        bound = 1.01 * fb + 2.0 ** -8 * (np.abs(exact) + fb)
    else:
        bound = fb
    err = np.abs(got - exact)
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, (f"{label}: {len(bad)} elements outside the bound, first {bad[:4].tolist()}: "
                           f"got {got[tuple(bad[0])]} want {exact[tuple(bad[0])]} bound {bound[tuple(bad[0])]}")
    nz = bound > 0
    return float((err[nz] / bound[nz]).max()) if nz.any() else 0.0
