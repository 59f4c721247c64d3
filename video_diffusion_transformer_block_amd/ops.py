"""Torch-facing binding of the C ABI: the same five calls, argument
marshalling only.  torch provides device memory and the current HIP stream;
every step of the computation runs in libvdtq.so."""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


# Device type every tensor handed to the library must have (the CPU tests of
# the argument checks below substitute "cpu" and a library stub).
_DEVICE_TYPE = "cuda"


def _require(t: torch.Tensor, dtype, name: str):
    if not torch.is_tensor(t) or t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _buf(t, name: str, dtype, shape, dev: torch.device):
    """A caller-given buffer the library reads or writes as a dense row-major
    array: it must be a contiguous tensor of exactly `shape` and `dtype` on
    `dev`, or the kernel would read or write past it."""
    _require(t, dtype, name)
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _flat(t, name: str, dtype, n: int, dev: torch.device):
    """A caller-given buffer read or written as n consecutive elements."""
    _require(t, dtype, name)
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of {n} elements, got shape {tuple(t.shape)}")
    return t


def _nvfp4(t: "NVFP4Tensor", name: str, R: int, K: int, dev: torch.device):
    _buf(t.q, f"{name}.q", torch.uint8, (R, K // 2), dev)
    _buf(t.scales, f"{name}.scales", torch.uint8, (R, K // 16), dev)
    _buf(t.ts, f"{name}.ts", torch.float32, (2,), dev)


def _mx(t: "MXTensor", name: str, R: int, K: int, dev: torch.device):
    if t.fmt not in ("mxfp4", "mxfp8"):
        raise ValueError(f"{name}.fmt {t.fmt!r}")
    _buf(t.q, f"{name}.q", torch.uint8, (R, K // 2 if t.fmt == "mxfp4" else K), dev)
    _buf(t.scales, f"{name}.scales", torch.uint8, (R, K // 32), dev)


def _bias(bias, N: int, dev: torch.device):
    if bias is not None:
        _buf(bias, "bias", torch.float32, (N,), dev)


def _ws_key(device: torch.device):
    """Workspaces are kept per (device, current stream): calls on one stream
    run in order and may share one; calls on different streams never do."""
    s = _stream(device)
    return torch.device(device).index, (None if s is None else s.value)


_ws = {}


def workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """Scratch buffer of the calls on the current stream of `device`."""
    key = _ws_key(device)
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf


_bs_ws = {}


def stats_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """Workspace of block_stats / block_stats_mx8 on the current stream,
    zero-filled when allocated: it holds the calls' completion counter, which
    must be zero before the first call and which every call leaves at zero
    (so it is not shared with the other entry points' workspace)."""
    key = _ws_key(device)
    buf = _bs_ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _bs_ws[key] = buf
    return buf


_gemm_ws = {}


def gemm_workspace(device: torch.device, M: int, N: int) -> torch.Tensor:
    """GEMM workspace (fp32 partial tiles of K slices) of the calls on the
    current stream of `device`."""
    key = _ws_key(device)
    nbytes = L.lib().vdtq_workspace_bytes(L.OP_QGEMM, M, N)
    buf = _gemm_ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _gemm_ws[key] = buf
    return buf


@dataclass
class NVFP4Tensor:
    """Packed codes [R, K/2] u8, E4M3 scales [R, K/16] u8, {amax, gs} f32[2]."""
    q: torch.Tensor
    scales: torch.Tensor
    ts: torch.Tensor
    stats: Optional[torch.Tensor] = None


@dataclass
class BF16Tensor:
    """The rotated activations in bf16 [M, K] (full-precision fallback)."""
    q: torch.Tensor
    stats: Optional[torch.Tensor] = None


@dataclass
class INT8Tensor:
    """Codes [M, K] int8 and per-row fp32 scales [M]."""
    q: torch.Tensor
    scales: torch.Tensor
    stats: Optional[torch.Tensor] = None


@dataclass
class MXTensor:
    """MX operand: codes (MXFP4: packed E2M1 [R, K/2] u8; MXFP8: E4M3 [R, K]
    u8) and E8M0 scales [R, K/32] u8; fmt is "mxfp4" or "mxfp8"."""
    q: torch.Tensor
    scales: torch.Tensor
    fmt: str
    stats: Optional[torch.Tensor] = None


def hadamard_quantize(x: torch.Tensor, had_block: int = 64, fmt: str = "nvfp4", amax=None,
                      stats: bool = False, out=None, gelu: bool = False):
    """Block Hadamard transform of bf16 rows + NVFP4, INT8, MXFP4 or MXFP8
    quantization (or bf16 rounding).  gelu: the rows are first mapped
    through the feed-forward's GELU (fp32, rounded to bf16).
    amax (NVFP4 only): a float or a 1-element device tensor to use as the
    tensor amax instead of computing it, or the string "given" to use the
    value already in out.ts[0].  out: a previously returned NVFP4Tensor /
    INT8Tensor of the same shape whose buffers are reused."""
    _require(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    M, K = x.shape
    dev = x.device
    if K % 16:
        raise ValueError(f"K = {K} is not a multiple of 16")
    if out is not None and stats and out.stats is not None:
        _buf(out.stats, "out.stats", torch.float64, (4,), dev)
    flags = (L.STATS if stats else 0) | (L.GELU if gelu else 0)
    st = torch.empty(4, dtype=torch.float64, device=dev) if stats else None
    nbytes = L.lib().vdtq_workspace_bytes(L.OP_HADAMARD_QUANTIZE, M, K)
    ws = workspace(dev, nbytes)
    if out is not None and stats and out.stats is not None:
        st = out.stats
    if fmt == "nvfp4":
        if out is not None:
            _nvfp4(out, "out", M, K, dev)
            q, s, ts = out.q, out.scales, out.ts
        else:
            q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            s = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
            ts = torch.empty(2, dtype=torch.float32, device=dev)
            if isinstance(amax, str) and amax == "given":
                raise ValueError('amax="given" reuses out.ts[0]: pass out=')
        if amax is not None:
            flags |= L.AMAX_GIVEN
            if not (isinstance(amax, str) and amax == "given"):
                ts[0] = amax if not torch.is_tensor(amax) else amax.reshape(-1)[0]
        fcode = L.FMT_NVFP4
    elif fmt == "int8":
        if amax is not None:
            raise ValueError("amax applies to nvfp4 only")
        if out is not None:
            _buf(out.q, "out.q", torch.int8, (M, K), dev)
            _buf(out.scales, "out.scales", torch.float32, (M,), dev)
            q, s = out.q, out.scales
        else:
            q = torch.empty((M, K), dtype=torch.int8, device=dev)
            s = torch.empty((M,), dtype=torch.float32, device=dev)
        ts = None
        fcode = L.FMT_INT8
    elif fmt == "bf16":
        if amax is not None:
            raise ValueError("amax applies to nvfp4 only")
        if out is not None:
            _buf(out.q, "out.q", torch.bfloat16, (M, K), dev)
        q = out.q if out is not None else torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        s = ts = None
        fcode = L.FMT_BF16
    elif fmt in ("mxfp4", "mxfp8"):
        if amax is not None:
            raise ValueError("amax applies to nvfp4 only")
        if out is not None:
            if getattr(out, "fmt", fmt) != fmt:
                raise ValueError(f"out holds {out.fmt}, asked for {fmt}")
            _mx(MXTensor(out.q, out.scales, fmt), "out", M, K, dev)
            q, s = out.q, out.scales
        else:
            q = torch.empty((M, K // 2 if fmt == "mxfp4" else K), dtype=torch.uint8, device=dev)
            s = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        ts = None
        fcode = L.FMT_MXFP4 if fmt == "mxfp4" else L.FMT_MXFP8
    else:
        raise ValueError(fmt)
    L.check(L.lib().hadamard_quantize(_p(x), M, K, x.stride(0), had_block, fcode, flags, _p(q), _p(s),
                                      _p(ts), _p(st), _p(ws), ws.numel(), _stream(dev)))
    if fcode == L.FMT_NVFP4:
        return NVFP4Tensor(q, s, ts, st)
    if fcode == L.FMT_BF16:
        return BF16Tensor(q, st)
    if fcode in (L.FMT_MXFP4, L.FMT_MXFP8):
        return MXTensor(q, s, fmt, st)
    return INT8Tensor(q, s, st)


def _out(M, N, out_dtype, dev, y):
    """The GEMM output: a caller-given y must be [M, N] of the output dtype
    on `dev` with unit column stride (its row stride is passed as ldy)."""
    if out_dtype not in ("bf16", "f32"):
        raise ValueError(f"out_dtype {out_dtype!r}")
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    if y is None:
        return torch.empty((M, N), dtype=dt, device=dev)
    _require(y, dt, "y")
    if y.device != dev:
        raise ValueError(f"y is on {y.device}, expected {dev}")
    if tuple(y.shape) != (M, N) or (M > 0 and N > 0 and (y.stride(1) != 1 or y.stride(0) < N)):
        raise ValueError(f"y must be [{M}, {N}] with unit column stride, got shape {tuple(y.shape)} "
                         f"strides {tuple(y.stride())}")
    return y


def qgemm_w4a4(a: NVFP4Tensor, w: NVFP4Tensor, bias: Optional[torch.Tensor] = None,
               out_dtype: str = "bf16", y: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, K = a.q.shape[0], a.q.shape[1] * 2
    N = w.q.shape[0]
    dev = a.q.device
    _nvfp4(a, "a", M, K, dev)
    _nvfp4(w, "w", N, K, dev)
    _bias(bias, N, dev)
    y = _out(M, N, out_dtype, dev, y)
    ws = gemm_workspace(a.q.device, M, N)
    L.check(L.lib().qgemm_w4a4(_p(a.q), _p(a.scales), _p(a.ts), _p(w.q), _p(w.scales), _p(w.ts), _p(bias),
                               _p(y), y.stride(0), L.OUT_BF16 if out_dtype == "bf16" else L.OUT_F32,
                               M, N, K, _p(ws), ws.numel(), _stream(a.q.device)))
    return y


def qgemm_w4a8(a: INT8Tensor, w: NVFP4Tensor, bias: Optional[torch.Tensor] = None,
               out_dtype: str = "bf16", y: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, K = a.q.shape
    N = w.q.shape[0]
    dev = a.q.device
    _buf(a.q, "a.q", torch.int8, (M, K), dev)
    _buf(a.scales, "a.scales", torch.float32, (M,), dev)
    _nvfp4(w, "w", N, K, dev)
    _bias(bias, N, dev)
    y = _out(M, N, out_dtype, dev, y)
    ws = gemm_workspace(a.q.device, M, N)
    L.check(L.lib().qgemm_w4a8(_p(a.q), _p(a.scales), _p(w.q), _p(w.scales), _p(w.ts), _p(bias),
                               _p(y), y.stride(0), L.OUT_BF16 if out_dtype == "bf16" else L.OUT_F32,
                               M, N, K, _p(ws), ws.numel(), _stream(a.q.device)))
    return y


def qgemm_w4a16(a: BF16Tensor, w: NVFP4Tensor, bias: Optional[torch.Tensor] = None,
                out_dtype: str = "bf16", y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Full-precision fallback: rotated bf16 activations x NVFP4 weights."""
    _require(a.q, torch.bfloat16, "a.q")
    if a.q.dim() != 2 or not a.q.is_contiguous():
        raise ValueError("a.q must be a contiguous [M, K] tensor")
    M, K = a.q.shape
    N = w.q.shape[0]
    dev = a.q.device
    _nvfp4(w, "w", N, K, dev)
    _bias(bias, N, dev)
    y = _out(M, N, out_dtype, dev, y)
    ws = gemm_workspace(dev, M, N)
    L.check(L.lib().qgemm_w4a16(_p(a.q), _p(w.q), _p(w.scales), _p(w.ts), _p(bias), _p(y), y.stride(0),
                                L.OUT_BF16 if out_dtype == "bf16" else L.OUT_F32, M, N, K, _p(ws), ws.numel(),
                                _stream(a.q.device)))
    return y


def qgemm_mx(a: MXTensor, w: MXTensor, bias: Optional[torch.Tensor] = None,
             out_dtype: str = "bf16", y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MX-native product: MXFP4 or MXFP8 activations x MXFP4 weights."""
    if w.fmt != "mxfp4":
        raise ValueError("MX weights must be mxfp4")
    M = a.q.shape[0]
    K = a.q.shape[1] * (2 if a.fmt == "mxfp4" else 1)
    N = w.q.shape[0]
    dev = a.q.device
    _mx(a, "a", M, K, dev)
    _mx(w, "w", N, K, dev)
    _bias(bias, N, dev)
    y = _out(M, N, out_dtype, dev, y)
    ws = gemm_workspace(a.q.device, M, N)
    L.check(L.lib().qgemm_mx(L.FMT_MXFP4 if a.fmt == "mxfp4" else L.FMT_MXFP8, _p(a.q), _p(a.scales), _p(w.q),
                             _p(w.scales), _p(bias), _p(y), y.stride(0),
                             L.OUT_BF16 if out_dtype == "bf16" else L.OUT_F32, M, N, K, _p(ws), ws.numel(),
                             _stream(a.q.device)))
    return y


def qgemm_mx_quant(a: MXTensor, w: MXTensor, bias: Optional[torch.Tensor] = None, out_fmt: str = "mxfp4",
                   had_block: int = 64, gelu: bool = True, out: Optional[MXTensor] = None) -> MXTensor:
    """qgemm_mx with a quantizing epilogue: the bf16 product (plus bias),
    optionally through GELU, Hadamard-transformed in blocks of had_block and
    MX-encoded as the next linear's activation (FFN-up feeding FFN-down)."""
    if w.fmt != "mxfp4":
        raise ValueError("MX weights must be mxfp4")
    if out_fmt not in ("mxfp4", "mxfp8"):
        raise ValueError(f"out_fmt {out_fmt!r}")
    M = a.q.shape[0]
    K = a.q.shape[1] * (2 if a.fmt == "mxfp4" else 1)
    N = w.q.shape[0]
    dev = a.q.device
    _mx(a, "a", M, K, dev)
    _mx(w, "w", N, K, dev)
    if bias is not None:
        _bias(bias, N, dev)
    if out is not None:
        if out.fmt != out_fmt:
            raise ValueError(f"out holds {out.fmt}, asked for {out_fmt}")
        _mx(out, "out", M, N, dev)
    if out is None:
        q = torch.empty((M, N // 2 if out_fmt == "mxfp4" else N), dtype=torch.uint8, device=dev)
        s = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
        out = MXTensor(q, s, out_fmt)
    L.check(L.lib().qgemm_mx_quant(L.FMT_MXFP4 if a.fmt == "mxfp4" else L.FMT_MXFP8, _p(a.q), _p(a.scales),
                                   _p(w.q), _p(w.scales), _p(bias), had_block,
                                   L.FMT_MXFP4 if out_fmt == "mxfp4" else L.FMT_MXFP8, L.GELU if gelu else 0,
                                   _p(out.q), _p(out.scales), M, N, K, _stream(dev)))
    return out


def block_stats(inp: torch.Tensor, out: torch.Tensor, dprev: Optional[torch.Tensor] = None,
                dnew: Optional[torch.Tensor] = None, write_delta: bool = True):
    """Returns (dnew or None, stats f64[8] device tensor)."""
    _require(inp, torch.bfloat16, "inp")
    _require(out, torch.bfloat16, "out")
    if inp.shape != out.shape or not inp.is_contiguous() or not out.is_contiguous():
        raise ValueError("inp/out must be contiguous tensors of one shape")
    n = inp.numel()
    dev = inp.device
    if out.device != dev:
        raise ValueError("inp and out must be on one device")
    if dprev is not None:
        _flat(dprev, "dprev", torch.bfloat16, n, dev)
    if dnew is not None:
        _flat(dnew, "dnew", torch.bfloat16, n, dev)
        if dprev is not None and n > 0 and dnew.data_ptr() == dprev.data_ptr():
            raise ValueError("dnew must not alias dprev")
    if dnew is None and write_delta:
        dnew = torch.empty_like(inp)
    st = torch.empty(8, dtype=torch.float64, device=dev)
    ws = stats_workspace(dev, L.lib().vdtq_workspace_bytes(L.OP_BLOCK_STATS, n, 1))
    L.check(L.lib().block_stats(_p(inp), _p(out), _p(dprev), _p(dnew), n, _p(st), _p(ws), ws.numel(),
                                _stream(dev)))
    return dnew, st


def block_stats_mx8(inp: torch.Tensor, out: torch.Tensor, dprev: Optional[MXTensor] = None,
                    dnew: Optional[MXTensor] = None, write_delta: bool = True):
    """block_stats with the delta cache in MXFP8 (codes u8 [n], E8M0 scales
    u8 [n/32], as an MXTensor of fmt "mxfp8" over the flattened tensor).
    Returns (dnew or None, stats f64[8] device tensor)."""
    _require(inp, torch.bfloat16, "inp")
    _require(out, torch.bfloat16, "out")
    if inp.shape != out.shape or not inp.is_contiguous() or not out.is_contiguous():
        raise ValueError("inp/out must be contiguous tensors of one shape")
    n = inp.numel()
    dev = inp.device
    if out.device != dev:
        raise ValueError("inp and out must be on one device")
    if n % 32:
        raise ValueError(f"n = {n} is not a multiple of 32")
    for name, d in (("dprev", dprev), ("dnew", dnew)):
        if d is not None:
            if d.fmt != "mxfp8":
                raise ValueError(f"{name} must be an mxfp8 MXTensor")
            _flat(d.q, f"{name}.q", torch.uint8, n, dev)
            _flat(d.scales, f"{name}.scales", torch.uint8, n // 32, dev)
    if dprev is not None and dnew is not None and n > 0 and dnew.q.data_ptr() == dprev.q.data_ptr():
        raise ValueError("dnew must not alias dprev")
    if dnew is None and write_delta:
        dnew = MXTensor(torch.empty(n, dtype=torch.uint8, device=dev),
                        torch.empty(n // 32, dtype=torch.uint8, device=dev), "mxfp8")
    st = torch.empty(8, dtype=torch.float64, device=dev)
    ws = stats_workspace(dev, L.lib().vdtq_workspace_bytes(L.OP_BLOCK_STATS, n, 1))
    L.check(L.lib().block_stats_mx8(_p(inp), _p(out), _p(dprev.q if dprev else None),
                                    _p(dprev.scales if dprev else None), _p(dnew.q if dnew else None),
                                    _p(dnew.scales if dnew else None), n, _p(st), _p(ws), ws.numel(),
                                    _stream(dev)))
    return dnew, st


def dmpq_budget_gamma(gammas, avg_bits: float = 6.0) -> float:
    """Host call: the Gamma threshold of a step in bit-budget mode (the k-th
    largest of the blocks' Gamma_{t-1}, k = floor(n (avg_bits - 4) / 4))."""
    g = [float(x) for x in gammas]
    arr = (ctypes.c_double * max(1, len(g)))(*g)
    return float(L.lib().dmpq_budget_gamma(arr, len(g), float(avg_bits)))


def dmpq_depth_params(base: L.DmpqParams, depth: int, n_blocks: int, s_shallow: float,
                      s_deep: float) -> L.DmpqParams:
    """Host call: block `depth` of `n_blocks`' parameters under a depth-aware
    caching profile (tau and tau_acc scaled linearly with relative depth,
    from s_shallow at the first block to s_deep at the last)."""
    out = L.DmpqParams()
    L.check(L.lib().dmpq_depth_params(ctypes.byref(base), int(depth), int(n_blocks), float(s_shallow),
                                      float(s_deep), ctypes.byref(out)))
    return out


def dmpq_params(gamma=0.1, tau=0.05, tau_acc=0.15, rho=50.0, tau_u=math.inf, warmup=2) -> L.DmpqParams:
    return L.DmpqParams(gamma, tau, tau_acc, rho, tau_u, warmup, 0)


def dmpq_state() -> L.DmpqState:
    s = L.DmpqState()
    L.lib().dmpq_state_init(ctypes.byref(s))
    return s


def dmpq_step(params: L.DmpqParams, state: L.DmpqState, last_stats, in_ratio: float) -> int:
    """Host call.  last_stats: 8 floats (host) or None.  Returns VDTQ_ACT_*."""
    act = ctypes.c_int(-1)
    ptr = None
    if last_stats is not None:
        arr = (ctypes.c_double * 8)(*[float(v) for v in last_stats])
        ptr = ctypes.cast(arr, ctypes.POINTER(ctypes.c_double))
    L.check(L.lib().dmpq_step(ctypes.byref(params), ctypes.byref(state), ptr, float(in_ratio),
                              ctypes.byref(act)))
    return act.value


def outlier_ratio(max_abs: float, sum_abs: float, n: int) -> float:
    return L.lib().vdtq_outlier_ratio(float(max_abs), float(sum_abs), int(n))
