"""Pins for oracle/gemm.py: brute-force loops, one-hot rows, exact integer
accumulators."""
import numpy as np

from oracle import formats as F, gemm as G, quant as Q

RNG = np.random.Generator(np.random.PCG64(14))


def _rand_nvfp4(rows, K):
    codes = RNG.integers(0, 16, size=(rows, K)).astype(np.uint8)
    scales = RNG.integers(0, 0x7F, size=(rows, K // 16)).astype(np.uint8)
    return F.pack_nibbles(codes), scales, codes


def _loop_dot(a_vals, w_vals):
    M, K = a_vals.shape
    N = w_vals.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(a_vals[m][k]) * float(w_vals[n][k])
            out[m, n] = s
    return out


def test_w4a4_brute_force():
    M, N, K = 4, 5, 48
    aq, as_, ac = _rand_nvfp4(M, K)
    wq, ws, wc = _rand_nvfp4(N, K)
    a_gs, w_gs = np.float32(0.37), np.float32(1.9)
    # decode each element straight from the definitions
    av = [[F.E2M1_VALUES[ac[m, k] & 7] * (-1 if ac[m, k] & 8 else 1)
           * F.e4m3_to_float(as_[m, k // 16]) for k in range(K)] for m in range(M)]
    wv = [[F.E2M1_VALUES[wc[n, k] & 7] * (-1 if wc[n, k] & 8 else 1)
           * F.e4m3_to_float(ws[n, k // 16]) for k in range(K)] for n in range(N)]
    want = _loop_dot(np.array(av), np.array(wv)) * float(a_gs) * float(w_gs)
    bias = RNG.standard_normal(N).astype(np.float32)
    y64, y32 = G.qgemm_w4a4(aq, as_, a_gs, wq, ws, w_gs, bias=bias, out_dtype="f32")
    assert np.allclose(y64, want + bias, rtol=1e-12, atol=1e-9)
    _, yb = G.qgemm_w4a4(aq, as_, a_gs, wq, ws, w_gs, bias=bias, out_dtype="bf16")
    assert np.array_equal(yb, F.f32_to_bf16(y32))


def test_w4a8_brute_force_and_integer_accumulator():
    M, N, K = 3, 6, 64
    aq = RNG.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_s = np.abs(RNG.standard_normal(M)).astype(np.float32)
    wq, ws, wc = _rand_nvfp4(N, K)
    wv = [[F.E2M1_VALUES[wc[n, k] & 7] * (-1 if wc[n, k] & 8 else 1)
           * F.e4m3_to_float(ws[n, k // 16]) for k in range(K)] for n in range(N)]
    w_gs = np.float32(0.5)
    want = _loop_dot(aq.astype(np.float64), np.array(wv)) * a_s[:, None].astype(np.float64) * 0.5
    y64, _ = G.qgemm_w4a8(aq, a_s, wq, ws, w_gs, out_dtype="f32")
    assert np.allclose(y64, want, rtol=1e-12)
    # unit scales: Y == P / 2 exactly, P the integer accumulator
    ones = np.full_like(ws, 0x38)
    y_unit, y32 = G.qgemm_w4a8(aq, np.ones(M, np.float32), wq, ones, np.float32(1.0), out_dtype="f32")
    P = G.w4a8_integer_accumulator(aq, wq)
    brute = np.array([[sum(int(aq[m, k]) * int(round(2 * F.E2M1_VALUES[wc[n, k] & 7]))
                           * (-1 if wc[n, k] & 8 else 1) for k in range(K))
                       for n in range(N)] for m in range(M)])
    assert np.array_equal(P, brute)
    assert np.array_equal(y_unit, P / 2.0) and np.array_equal(y32, (P / 2.0).astype(np.float32))
    Pg = G.w4a8_group_partials(aq, wq)
    assert np.array_equal(Pg.sum(-1), P)
    assert np.abs(Pg).max() <= 16 * 127 * 12


def test_one_hot_rows_pick_weight_columns():
    N, K = 8, 64
    wq, ws, _ = _rand_nvfp4(N, K)
    W = Q.nvfp4_dequantize(wq, ws)
    # A = e_k scaled to exactly 1.0: code 2 (1.0) with scale byte 0x38 (1.0)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2
    aq = F.pack_nibbles(codes)
    as_ = np.full((K, K // 16), 0x38, np.uint8)
    y64, _ = G.qgemm_w4a4(aq, as_, np.float32(1), wq, ws, np.float32(1), out_dtype="f32")
    assert np.array_equal(y64, W.T)
