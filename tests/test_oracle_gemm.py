"""Pins of the oracle's GEMM references and INT8 quantizers (CPU only).

W4A16 reference: exact rational brute force on tiny shapes, one-hot inputs
(Y = a column of the dequantized weight), all codes at the zero-point (Y = 0).
INT8: exhaustive argmin code search with the +-127 clip (Quantization
operators guide §2.1/§2.2), the max element mapping to +-127, exact integer
brute force of the accumulator, the closed form 127 * 127 * K, and the
epilogue C * scale_X * scale_W (§2.3) against NumPy float32 arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

from test_oracle_q4 import unpack_nibbles


def _dequant_np(codes, scales, zeros, K, g):
    u = unpack_nibbles(codes, K)
    G = K // g
    zp = np.full((codes.shape[0], G), 8) if zeros is None else unpack_nibbles(zeros, G)
    return [[Fraction(int(u[n, k] - zp[n, k // g])) * Fraction(float(scales[n, k // g]))
             for k in range(K)] for n in range(codes.shape[0])]


@pytest.mark.parametrize("sym", [False, True])
def test_w4a16_ref_exact_bruteforce(orc, sym):
    rng = np.random.default_rng(21)
    M, N, K, g = 3, 4, 96, 32
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=sym)
    Y, B = orc.w4a16_ref(X, codes, scales, zeros, g=g)
    wh = _dequant_np(codes, scales, zeros, K, g)
    for m in range(M):
        xs = [Fraction(float(v)) for v in X[m]]
        for n in range(N):
            exact = sum(x * w for x, w in zip(xs, wh[n]))
            bound = sum(abs(x) * abs(w) for x, w in zip(xs, wh[n]))
            assert abs(Fraction(Y[m, n]) - exact) <= K * Fraction(2) ** -53 * bound
            assert abs(Fraction(B[m, n]) - bound) <= K * Fraction(2) ** -53 * bound


def test_w4a16_ref_one_hot_and_zero(orc):
    rng = np.random.default_rng(22)
    N, K, g = 16, 256, 128
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=False)
    w_hat = orc.q4_dequant(codes, scales, zeros, K, g)
    X = np.eye(K, dtype=np.float16)
    Y, _ = orc.w4a16_ref(X, codes, scales, zeros, g=g)
    assert np.array_equal(Y, w_hat.T)
    # sampled rows give the same values as the full call
    rows = [3, 200, 17]
    Ys, _ = orc.w4a16_ref(X, codes, scales, zeros, g=g, rows=rows)
    assert np.array_equal(Ys, Y[rows])
    # every code at its zero-point: the product is exactly zero
    zeros5 = np.full_like(zeros, 0x55)
    codes5 = np.full_like(codes, 0x55)
    Xr = rng.standard_normal((4, K)).astype(np.float16)
    Y0, _ = orc.w4a16_ref(Xr, codes5, scales, zeros5, g=g)
    assert np.all(Y0 == 0)


def brute_q8(t):
    """argmin over q in [-127, 127] of |t - q|, ties to even q."""
    levels = np.arange(-127, 128)
    d = np.abs(t.astype(np.float64)[:, None] - levels[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = (levels % 2 == 0)[None, :]
    tie = cand.sum(axis=1) > 1
    return levels[np.where(tie, np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))]


def test_q8_weight_codes_exhaustive(orc):
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    vals = np.unique(allh[np.isfinite(allh) & (np.abs(allh.astype(np.float32)) <= 2.0)])
    K = 512
    rows = -(-vals.size // K)
    W = np.zeros(rows * K, np.float16)
    W[: vals.size] = vals
    W = W.reshape(rows, K)
    rng = np.random.default_rng(23)
    s = rng.uniform(0.3, 3.0, K).astype(np.float32)
    for smooth in (None, s):
        Wq, sw = orc.q8_quantize_weight(W, smooth)
        wp = W.astype(np.float32) * (np.float32(1) if smooth is None else smooth[None, :])
        a = np.maximum(np.abs(wp).max(1), np.float32(1e-8))
        assert np.array_equal(sw, a / np.float32(127))
        for n in range(rows):
            t = wp[n] / sw[n]
            assert np.array_equal(Wq[n].astype(np.int64), brute_q8(t)), n
            # the largest |w'| maps to +-127
            k = np.argmax(np.abs(wp[n]))
            assert abs(int(Wq[n, k])) == 127


def test_q8_act_codes(orc):
    rng = np.random.default_rng(24)
    M, K = 16, 1024
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, :10] *= 30
    X[3] = 0                                  # an all-zero token
    X = X.astype(np.float16)
    s = rng.uniform(0.5, 8.0, K).astype(np.float32)
    for smooth in (None, s):
        Xq, sx = orc.q8_quantize_act(X, smooth)
        xp = X.astype(np.float32) if smooth is None else X.astype(np.float32) / smooth[None, :]
        a = np.maximum(np.abs(xp).max(1), np.float32(1e-8))
        assert np.array_equal(sx, a / np.float32(127))
        for m in range(M):
            assert np.array_equal(Xq[m].astype(np.int64), brute_q8(xp[m] / sx[m]))
        assert np.all(Xq[3] == 0)


def test_int8_gemm_bruteforce_and_closed_form(orc):
    rng = np.random.default_rng(25)
    M, N, K = 5, 7, 300
    Xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    acc, aacc, ovf = orc.int8_gemm(Xq, Wq)
    assert ovf == 0
    for m in range(M):
        for n in range(N):
            prods = [int(a) * int(b) for a, b in zip(Xq[m], Wq[n])]
            assert acc[m, n] == sum(prods)
            assert aacc[m, n] == sum(abs(p) for p in prods)
    K = 8192
    acc, _, ovf = orc.int8_gemm(np.full((2, K), 127, np.int8), np.full((3, K), 127, np.int8))
    assert ovf == 0 and np.all(acc == 16129 * K) and 16129 * K == 132_128_768
    acc, _, ovf = orc.int8_gemm(np.full((1, 140000), 127, np.int8),
                                np.full((1, 140000), -127, np.int8))
    assert ovf == 1


def test_w8a8_epilogue(orc):
    rng = np.random.default_rng(26)
    M, N, K = 6, 9, 512
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    Xq, sx = orc.q8_quantize_act(X)
    Wq, sw = orc.q8_quantize_weight(W)
    acc, aacc, _ = orc.int8_gemm(Xq, Wq)
    Y, B, y16 = orc.w8a8_epilogue(acc, aacc, sx, sw)
    for m in range(M):
        for n in range(N):
            exact = Fraction(float(sx[m])) * Fraction(float(sw[n])) * int(acc[m, n])
            assert abs(Fraction(Y[m, n]) - exact) <= Fraction(2) ** -51 * abs(exact)
    ref16 = ((acc.astype(np.float32) * sx[:, None]) * sw[None, :]).astype(np.float16)
    assert np.array_equal(y16, ref16.view(np.uint16))
    # the fp32 expression is evaluated left to right, (acc * sx) * sw; on a
    # larger sample the other association differs in some fp16 results
    acc2 = rng.integers(-2 ** 27, 2 ** 27, (256, 256)).astype(np.int64)
    sx2 = rng.uniform(1e-3, 1.0, 256).astype(np.float32)
    sw2 = rng.uniform(1e-5, 1e-3, 256).astype(np.float32)
    _, _, y2 = orc.w8a8_epilogue(acc2, np.abs(acc2), sx2, sw2)
    ref2 = ((acc2.astype(np.float32) * sx2[:, None]) * sw2[None, :]).astype(np.float16)
    assert np.array_equal(y2, ref2.view(np.uint16))
    # sampled rows
    rows = [4, 1]
    acc_s, aacc_s, _ = orc.int8_gemm(Xq, Wq, rows=rows)
    assert np.array_equal(acc_s, acc[rows])
    Ys, _, _ = orc.w8a8_epilogue(acc_s, aacc_s, sx, sw, rows=rows)
    assert np.array_equal(Ys, Y[rows])
