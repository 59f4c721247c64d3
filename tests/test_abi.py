"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, rejects bad arguments before touching a device, and the host
scheduler follows the hand-derived sequence and the oracle."""
import ctypes
import json
import math
import os
import re
import subprocess

import numpy as np
import pytest

import video_diffusion_transformer_block_amd as V
from video_diffusion_transformer_block_amd import _lib as L
from oracle import dmpq as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vdtq.h")
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: every call
FAKE8 = ctypes.c_void_p(0x10008)         # below fails validation before a launch


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|void|size_t|double|char)\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_and_exports_agree():
    decl = declared_functions()
    assert sorted(L.EXPORTED) == decl
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in decl:
        assert name in syms, name
        assert getattr(V.lib(), name) is not None


def test_version_and_workspace_sizes():
    assert V.lib().vdtq_version().startswith(b"vdtq")
    lib = V.lib()
    assert lib.vdtq_workspace_bytes(L.OP_HADAMARD_QUANTIZE, 17776, 3072) >= 4 * 8 * (17776 * 48 // 256)
    assert lib.vdtq_workspace_bytes(L.OP_BLOCK_STATS, 4446 * 1920, 1) >= 8 * 8
    assert lib.vdtq_workspace_bytes(99, 1, 1) == 0


def _hq(**kw):
    a = dict(x=FAKE, M=4, K=64, ldx=64, b=64, fmt=0, flags=0, q=FAKE, s=FAKE, ts=FAKE, st=None,
             ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return V.lib().hadamard_quantize(a["x"], a["M"], a["K"], a["ldx"], a["b"], a["fmt"], a["flags"], a["q"],
                                     a["s"], a["ts"], a["st"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=15), L.EINVAL), (dict(K=0), L.EINVAL), (dict(M=-1), L.EINVAL),
    (dict(b=48), L.EINVAL), (dict(b=512), L.EINVAL), (dict(K=96, ldx=96, b=64), L.EINVAL),
    (dict(ldx=60), L.EINVAL), (dict(ldx=68), L.EINVAL), (dict(fmt=5), L.EINVAL), (dict(fmt=-1), L.EINVAL),
    (dict(flags=8), L.EINVAL), (dict(fmt=1, flags=1), L.EINVAL), (dict(fmt=1, flags=2, ws=None), L.EINVAL),
    (dict(fmt=3, flags=2, wsb=64), L.EINVAL),
    (dict(fmt=1, K=16384 + 64, ldx=16448), L.EUNSUPPORTED),
    (dict(x=None), L.EINVAL), (dict(q=None), L.EINVAL), (dict(x=FAKE8), L.EINVAL),
    (dict(ts=None), L.EINVAL), (dict(flags=2, st=None), L.EINVAL),
    (dict(ws=None), L.EINVAL), (dict(wsb=8), L.EINVAL),
    (dict(fmt=2, flags=1), L.EINVAL), (dict(fmt=2, q=None), L.EINVAL),
    (dict(fmt=3, K=48, ldx=48, b=16), L.EINVAL), (dict(fmt=4, K=80, ldx=80, b=16), L.EINVAL),
    (dict(fmt=3, flags=1), L.EINVAL), (dict(fmt=4, s=None), L.EINVAL), (dict(fmt=3, q=FAKE8), L.EINVAL),
    (dict(fmt=2, q=FAKE8), L.EINVAL), (dict(fmt=2, flags=2, st=None), L.EINVAL),
])
def test_hadamard_quantize_rejects(kw, code):
    assert _hq(**kw) == code
    assert V.lib().vdtq_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(K=15), L.EINVAL), (dict(b=48), L.EINVAL), (dict(x=None), L.EINVAL), (dict(x=FAKE8), L.EINVAL),
    (dict(fmt=1, flags=1), L.EINVAL), (dict(ts=None), L.EINVAL), (dict(flags=2, st=None), L.EINVAL),
    (dict(fmt=1, K=16384 + 64, ldx=16448), L.EUNSUPPORTED),
])
def test_hadamard_quantize_noalloc_rejects_like_the_workspace_call(kw, code):
    """The allocation-free entry point shares hadamard_quantize's checks."""
    a = dict(x=FAKE, M=4, K=64, ldx=64, b=64, fmt=0, flags=0, q=FAKE, s=FAKE, ts=FAKE, st=None)
    a.update(kw)
    rc = V.lib().hadamard_quantize_noalloc(a["x"], a["M"], a["K"], a["ldx"], a["b"], a["fmt"], a["flags"], a["q"],
                                           a["s"], a["ts"], a["st"], None)
    assert rc == code and V.lib().vdtq_last_error()


@pytest.mark.parametrize("M,K,fmt", [(250000, 3072, 1), (240000, 64, 0), (17776 * 12, 12288, 0)])
def test_hadamard_quantize_noalloc_rejects_beyond_its_scratch(M, K, fmt):
    """Sizes whose partials exceed the static scratch array are refused
    before anything runs (no device is needed to see it)."""
    lib = V.lib()
    assert lib.vdtq_workspace_bytes(L.OP_HADAMARD_QUANTIZE, M, K) > L.NOALLOC_SCRATCH_BYTES
    rc = lib.hadamard_quantize_noalloc(FAKE, M, K, K, 64, fmt, 0, FAKE, FAKE, FAKE, None, None)
    assert rc == L.EUNSUPPORTED and b"maximum" in lib.vdtq_last_error()


def test_noalloc_scratch_bound_is_the_header_constant():
    src = open(HEADER).read()
    m = re.search(r"#define VDTQ_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES
    # the 5B and 1080p shapes of the block fit
    for M, K in ((17776, 3072), (17776, 12288), (106306, 3072), (106306, 12288)):
        assert V.lib().vdtq_workspace_bytes(L.OP_HADAMARD_QUANTIZE, M, K) <= L.NOALLOC_SCRATCH_BYTES


def _gemm(fn, **kw):
    a = dict(aq=FAKE, as_=FAKE, ats=FAKE, wq=FAKE, ws=FAKE, wts=FAKE, bias=None, y=FAKE, ldy=64, od=0,
             M=8, N=64, K=64, gws=FAKE, gwsb=1 << 28)
    a.update(kw)
    if fn == "w4a4":
        return V.lib().qgemm_w4a4(a["aq"], a["as_"], a["ats"], a["wq"], a["ws"], a["wts"], a["bias"], a["y"],
                                  a["ldy"], a["od"], a["M"], a["N"], a["K"], a["gws"], a["gwsb"], None)
    return V.lib().qgemm_w4a8(a["aq"], a["as_"], a["wq"], a["ws"], a["wts"], a["bias"], a["y"], a["ldy"],
                              a["od"], a["M"], a["N"], a["K"], a["gws"], a["gwsb"], None)


@pytest.mark.parametrize("fn", ["w4a4", "w4a8"])
@pytest.mark.parametrize("kw", [dict(K=0), dict(K=40), dict(M=-2), dict(ldy=10), dict(od=3),
                                dict(aq=None), dict(wq=None), dict(wts=None), dict(y=None),
                                dict(aq=FAKE8), dict(M=1 << 31), dict(gws=None), dict(gwsb=4096),
                                dict(gws=FAKE8)])
def test_qgemm_rejects(fn, kw):
    assert _gemm(fn, **kw) == L.EINVAL


def test_qgemm_workspace_size():
    """One fp32 256 x 256 partial tile per K slice, at most one slice per CU
    (256 on MI355X) in flight."""
    slots = 256 * 256 * 256 * 4
    assert V.lib().vdtq_workspace_bytes(L.OP_QGEMM, 17776, 3072) == slots
    assert V.lib().vdtq_workspace_bytes(L.OP_QGEMM, 1, 1) == slots
    assert V.lib().vdtq_workspace_bytes(L.OP_QGEMM, 0, 64) == 0


def test_qgemm_empty_is_noop():
    assert _gemm("w4a4", M=0) == L.OK
    assert _gemm("w4a8", N=0, aq=None, y=None) == L.OK


def _a16(**kw):
    a = dict(a=FAKE, wq=FAKE, ws=FAKE, wts=FAKE, bias=None, y=FAKE, ldy=64, od=0, M=8, N=64, K=128, gws=FAKE,
             gwsb=1 << 28)
    a.update(kw)
    return V.lib().qgemm_w4a16(a["a"], a["wq"], a["ws"], a["wts"], a["bias"], a["y"], a["ldy"], a["od"],
                               a["M"], a["N"], a["K"], a["gws"], a["gwsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), L.EINVAL), (dict(K=40), L.EINVAL), (dict(M=-1), L.EINVAL), (dict(ldy=10), L.EINVAL),
    (dict(od=2), L.EINVAL), (dict(a=None), L.EINVAL), (dict(wq=None), L.EINVAL), (dict(wts=None), L.EINVAL),
    (dict(y=None), L.EINVAL), (dict(a=FAKE8), L.EINVAL), (dict(K=96), L.EUNSUPPORTED),
    (dict(M=1 << 20, K=1 << 11), L.EUNSUPPORTED), (dict(gws=None), L.EINVAL), (dict(gwsb=4096), L.EINVAL),
    (dict(gws=FAKE8), L.EINVAL),
])
def test_qgemm_w4a16_rejects(kw, code):
    assert _a16(**kw) == code
    assert V.lib().vdtq_last_error()


def test_qgemm_w4a16_empty_is_noop():
    assert _a16(M=0, a=None) == L.OK
    assert _a16(N=0, y=None) == L.OK


def _mx(**kw):
    a = dict(fmt=L.FMT_MXFP4, aq=FAKE, as_=FAKE, wq=FAKE, ws=FAKE, bias=None, y=FAKE, ldy=64, od=0, M=8, N=64,
             K=128, gws=FAKE, gwsb=1 << 28)
    a.update(kw)
    return V.lib().qgemm_mx(a["fmt"], a["aq"], a["as_"], a["wq"], a["ws"], a["bias"], a["y"], a["ldy"], a["od"],
                            a["M"], a["N"], a["K"], a["gws"], a["gwsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=L.FMT_NVFP4), L.EINVAL), (dict(fmt=L.FMT_INT8), L.EINVAL), (dict(fmt=7), L.EINVAL),
    (dict(K=0), L.EINVAL), (dict(K=48), L.EINVAL), (dict(M=-1), L.EINVAL), (dict(ldy=10), L.EINVAL),
    (dict(od=2), L.EINVAL), (dict(aq=None), L.EINVAL), (dict(as_=None), L.EINVAL), (dict(wq=None), L.EINVAL),
    (dict(ws=None), L.EINVAL), (dict(y=None), L.EINVAL), (dict(aq=FAKE8), L.EINVAL),
    (dict(gws=None), L.EINVAL), (dict(gwsb=4096), L.EINVAL), (dict(gws=FAKE8), L.EINVAL),
    (dict(K=96), L.EUNSUPPORTED), (dict(fmt=L.FMT_MXFP8, K=160), L.EUNSUPPORTED),
    (dict(fmt=L.FMT_MXFP8, M=1 << 21, K=1 << 11), L.EUNSUPPORTED),
])
def test_qgemm_mx_rejects(kw, code):
    assert _mx(**kw) == code
    assert V.lib().vdtq_last_error()


def test_qgemm_mx_empty_is_noop():
    assert _mx(M=0, aq=None) == L.OK
    assert _mx(N=0, y=None, gws=None) == L.OK


def _mxq(**kw):
    a = dict(fmt=L.FMT_MXFP4, aq=FAKE, as_=FAKE, wq=FAKE, ws=FAKE, bias=None, b=64, of=L.FMT_MXFP8, fl=L.GELU,
             q=FAKE, s=FAKE, M=8, N=64, K=128)
    a.update(kw)
    return V.lib().qgemm_mx_quant(a["fmt"], a["aq"], a["as_"], a["wq"], a["ws"], a["bias"], a["b"], a["of"],
                                  a["fl"], a["q"], a["s"], a["M"], a["N"], a["K"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=L.FMT_INT8), L.EINVAL), (dict(of=L.FMT_NVFP4), L.EINVAL), (dict(of=5), L.EINVAL),
    (dict(fl=1), L.EINVAL), (dict(fl=8), L.EINVAL), (dict(b=32), L.EUNSUPPORTED), (dict(b=128), L.EUNSUPPORTED),
    (dict(N=96), L.EINVAL), (dict(N=32), L.EINVAL), (dict(K=48), L.EINVAL), (dict(K=96), L.EUNSUPPORTED),
    (dict(M=-1), L.EINVAL), (dict(q=None), L.EINVAL), (dict(s=None), L.EINVAL), (dict(ws=None), L.EINVAL),
    (dict(q=FAKE8), L.EINVAL), (dict(s=ctypes.c_void_p(0x10002)), L.EINVAL),
    (dict(bias=ctypes.c_void_p(0x10004)), L.EINVAL), (dict(aq=FAKE8), L.EINVAL), (dict(M=1 << 26, K=1 << 7, fmt=L.FMT_MXFP8), L.EUNSUPPORTED),
])
def test_qgemm_mx_quant_rejects(kw, code):
    assert _mxq(**kw) == code
    assert V.lib().vdtq_last_error()


def test_qgemm_mx_quant_empty_is_noop():
    assert _mxq(M=0, aq=None, q=None) == L.OK
    assert _mxq(N=0, wq=None, s=None) == L.OK


@pytest.mark.parametrize("kw", [dict(n=-1), dict(st=None), dict(inp=None), dict(dnew=FAKE, dprev=FAKE),
                                dict(ws=None), dict(wsb=0), dict(inp=FAKE8)])
def test_block_stats_rejects(kw):
    a = dict(inp=FAKE, out=FAKE, dprev=None, dnew=None, n=64, st=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    rc = V.lib().block_stats(a["inp"], a["out"], a["dprev"], a["dnew"], a["n"], a["st"], a["ws"], a["wsb"], None)
    assert rc == L.EINVAL


FAKE4 = ctypes.c_void_p(0x10004)


@pytest.mark.parametrize("kw", [dict(n=-32), dict(n=48), dict(st=None), dict(inp=None), dict(pq=FAKE, ps=None),
                                dict(nq=None), dict(nq=FAKE, pq=FAKE, ps=FAKE), dict(ws=None), dict(wsb=0),
                                dict(inp=FAKE8), dict(nq=FAKE4)])
def test_block_stats_mx8_rejects(kw):
    a = dict(inp=FAKE, out=FAKE, pq=None, ps=None, nq=FAKE, ns=FAKE8, n=64, st=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    rc = V.lib().block_stats_mx8(a["inp"], a["out"], a["pq"], a["ps"], a["nq"], a["ns"], a["n"], a["st"], a["ws"],
                                 a["wsb"], None)
    assert rc == L.EINVAL
    assert V.lib().vdtq_last_error()


def test_dmpq_step_hand_sequence():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "dmpq_sequence.json")))
    p = V.dmpq_params(**g["params"])
    s = V.dmpq_state()
    names = {L.ACT_SKIP: "skip", L.ACT_NVFP4: "nvfp4", L.ACT_INT8: "int8", L.ACT_BF16: "bf16"}
    got = [names[V.dmpq_step(p, s, None if n is None else g["stats"][n], r)] for n, r, _ in g["calls"]]
    assert got == [c[2] for c in g["calls"]]


def test_dmpq_step_matches_oracle_random():
    rng = np.random.Generator(np.random.PCG64(99))
    for trial in range(20):
        kw = dict(gamma=rng.uniform(0.02, 0.3), tau=rng.uniform(0.01, 0.2), tau_acc=rng.uniform(0.05, 0.6),
                  rho=rng.uniform(2, 20), tau_u=(math.inf if trial % 2 else rng.uniform(0.2, 1.0)),
                  warmup=int(rng.integers(0, 4)))
        p_c, s_c = V.dmpq_params(**kw), V.dmpq_state()
        p_o, s_o = D.Params(**kw), D.State()
        last = None
        for t in range(200):
            ratio = float(rng.uniform(1, 25))
            a_c = V.dmpq_step(p_c, s_c, last, ratio)
            a_o = D.dmpq_step(p_o, s_o, None if last is None else np.array(last), ratio)
            assert a_c == a_o, (trial, t)
            if a_c == L.ACT_SKIP:
                last = None
            else:
                z = rng.uniform(0, 1, 4)
                last = [z[0] * 0.05, 1.0, (z[1] * 0.2) ** 2, 1.0 if z[2] > 0.05 else 0.0, 1, 1, 1, 1]
        assert s_c.step == s_o.step and s_c.acc == s_o.acc and s_c.r_last == s_o.r_last


def test_dmpq_step_null_args():
    assert V.lib().dmpq_step(None, None, None, 1.0, None) == L.EINVAL


def test_outlier_ratio_c():
    assert V.outlier_ratio(4.0, 100.0, 100) == 4.0
    assert V.outlier_ratio(0.0, 0.0, 100) == 1.0


def test_dmpq_budget_gamma_matches_oracle():
    rng = np.random.Generator(np.random.PCG64(78))
    for trial in range(300):
        n = int(rng.integers(0, 80))
        g = rng.uniform(0, 0.3, n)
        if trial % 5 == 0 and n:
            g[rng.integers(0, n, size=max(1, n // 3))] = 0.1          # ties
        if trial % 7 == 0 and n:
            g[0] = math.inf
        bits = float(rng.uniform(3, 9))
        assert V.dmpq_budget_gamma(g, bits) == D.budget_gamma(g, bits), (trial, n, bits)
    assert V.dmpq_budget_gamma([0.2, 0.1], math.nan) == math.inf
    assert V.lib().dmpq_budget_gamma(None, 4, 6.0) == math.inf


def test_dmpq_depth_params_matches_oracle():
    """The C depth profile equals the oracle's bit for bit (same float64
    steps), for random bases, depths and factors, and rejects bad input."""
    rng = np.random.Generator(np.random.PCG64(91))
    for _ in range(500):
        n = int(rng.integers(1, 64))
        depth = int(rng.integers(0, n))
        s0, s1 = (float(v) for v in rng.uniform(0, 3, 2))
        base = dict(gamma=float(rng.uniform(0, 1)), tau=float(rng.uniform(0, 0.2)),
                    tau_acc=float(rng.uniform(0, 0.5)), rho=float(rng.uniform(1, 500)),
                    tau_u=float(rng.choice([math.inf, rng.uniform(0, 1)])), warmup=int(rng.integers(0, 5)))
        got = V.dmpq_depth_params(V.dmpq_params(**base), depth, n, s0, s1)
        want = D.depth_params(D.Params(**base), depth, n, s0, s1)
        assert (got.gamma, got.tau, got.tau_acc, got.rho, got.tau_u, got.warmup) == \
               (want.gamma, want.tau, want.tau_acc, want.rho, want.tau_u, want.warmup)
    base = V.dmpq_params()
    out = L.DmpqParams()
    for args in ((-1, 4, 1.0, 1.0), (4, 4, 1.0, 1.0), (0, 0, 1.0, 1.0), (0, 4, -0.5, 1.0),
                 (0, 4, 1.0, math.inf), (0, 4, math.nan, 1.0)):
        assert V.lib().dmpq_depth_params(ctypes.byref(base), *args, ctypes.byref(out)) == L.EINVAL
    assert V.lib().dmpq_depth_params(None, 0, 1, 1.0, 1.0, ctypes.byref(out)) == L.EINVAL
