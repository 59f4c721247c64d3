"""Pins for oracle/gemm.py: brute-force loops, one-hot rows, exact integer
accumulators."""
import numpy as np

from oracle import formats as F, gemm as G, hadamard as H, quant as Q

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


def test_w4a16_brute_force():
    """bf16 activations straight from their bits, weights from the format
    definitions, products summed in a Python loop."""
    M, N, K = 3, 5, 48
    # random signs, mantissas and exponents 2^-27 .. 2^24 (no overflow)
    a_bits = ((RNG.integers(0, 2, size=(M, K)) << 15) | (RNG.integers(100, 151, size=(M, K)) << 7)
              | RNG.integers(0, 128, size=(M, K))).astype(np.uint16)
    wq, ws, wc = _rand_nvfp4(N, K)
    w_gs = np.float32(0.75)
    av = [[struct_bf16(a_bits[m, k]) for k in range(K)] for m in range(M)]
    wv = [[F.E2M1_VALUES[wc[n, k] & 7] * (-1 if wc[n, k] & 8 else 1)
           * F.e4m3_to_float(ws[n, k // 16]) for k in range(K)] for n in range(N)]
    want = _loop_dot(np.array(av), np.array(wv)) * 0.75
    y64, _ = G.qgemm_w4a16(a_bits, wq, ws, w_gs, out_dtype="f32")
    assert np.allclose(y64, want, rtol=1e-12, atol=0)


def struct_bf16(bits):
    """bf16 bits -> float through the IEEE single layout (struct module)."""
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_w4a16_integer_inputs_exact():
    """Small-integer activations and unit weight scales: Y is the exact
    integer sum of a * e2m1(w)."""
    M, N, K = 4, 6, 64
    a = RNG.integers(-20, 21, size=(M, K)).astype(np.float32)
    a_bits = (a.view(np.uint32) >> 16).astype(np.uint16)      # exact in bf16
    wq, _, wc = _rand_nvfp4(N, K)
    ones = np.full((N, K // 16), 0x38, np.uint8)
    y64, y32 = G.qgemm_w4a16(a_bits, wq, ones, np.float32(1.0), out_dtype="f32")
    c = np.array([[F.E2M1_VALUES[wc[n, k] & 7] * (-1 if wc[n, k] & 8 else 1) for k in range(K)]
                  for n in range(N)])
    assert np.array_equal(y64, a.astype(np.float64) @ c.T)


def test_w4a16_rotation_cancels():
    """bf16 fallback of a whole linear: rotating activations and weights by
    the same block Hadamard transform leaves X W^T, up to the weights'
    4-bit error and the bf16 rounding of the rotated activations."""
    M, N, K = 32, 24, 128
    x = RNG.standard_normal((M, K)).astype(np.float32)
    w = (RNG.standard_normal((N, K)) * 0.02).astype(np.float32)
    xb, wb = F.f32_to_bf16(x), F.f32_to_bf16(w)
    wq, ws, wgs = Q.prepare_weight(wb, 64)
    a = Q.hadamard_quantize(xb, 64, "bf16")["q"]
    y64, _ = G.qgemm_w4a16(a, wq, ws, wgs, out_dtype="f32")
    ref = F.bf16_to_f32(xb).astype(np.float64) @ F.bf16_to_f32(wb).astype(np.float64).T
    rel = np.linalg.norm(y64 - ref) / np.linalg.norm(ref)
    assert rel < 0.15            # NVFP4 weights: ~10% relative error per element
    # the bf16 activations alone (weights exact) reproduce X W^T to bf16 precision
    Wrot = H.block_hadamard_f32(F.bf16_to_f32(wb), 64).astype(np.float64)
    y_exact_w = F.bf16_to_f32(a).astype(np.float64) @ Wrot.T
    assert np.linalg.norm(y_exact_w - ref) / np.linalg.norm(ref) < 1e-2
