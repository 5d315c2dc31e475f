"""Pins of the oracle's MXFP4 weight path (Quantization operators guide §4.3:
E2M1 elements, an E8M0 scale per block of 32, FP8 activations): the E2M1
encoder against the value set the pages print and a brute-force nearest
search, the block-scale choice against its defining inequality, the
dequantized weight against the format's error bound, and the W4A8 GEMM
reference against exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from golden_io import load, num

F = load("formats.txt")


def test_e2m1_round_trip_and_value_set(orc):
    vals = [orc.e2m1_decode(c) for c in range(16)]
    assert sorted(set(vals)) == sorted(set(num(F["e2m1_values"])))
    for c in range(16):
        assert orc.e2m1_encode(vals[c]) == c


def brute_e2m1(x):
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = abs(Fraction(float(x)))
    best = min(range(8), key=lambda c: (abs(Fraction(mags[c]) - a), c & 1))
    return best | (8 if np.signbit(np.float32(x)) else 0)


def test_e2m1_brute_force(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = h[np.isfinite(h)].astype(np.float32)
    f = f[np.abs(f) <= 16]
    sample = np.concatenate([f[::7], np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, -5.0, -0.0])])
    for x in sample:
        assert orc.e2m1_encode(float(x)) == brute_e2m1(x), x


def test_scale_choice_and_error_bound(orc):
    W, _ = workloads.small_case(31, 1, 48, 512)
    W[3, :32] = 0                       # an all-zero block
    W[4, 32:64] = np.float16(0.75)      # amax = 6 * 2^-3 exactly
    s = (np.abs(np.random.default_rng(8).standard_normal(512)) + 0.5).astype(np.float32)
    for smooth in (None, s):
        codes, sc = orc.mxfp4_quantize_weight(W, smooth)
        v = W.astype(np.float32) * (1 if smooth is None else smooth)
        amax = np.abs(v.reshape(48, 16, 32)).max(axis=2).astype(np.float64)
        e = sc.astype(np.int64) - 127
        nz = amax > 0
        # the smallest power of two with amax <= 6 * 2^e
        assert np.all(amax[nz] <= 6 * np.ldexp(1.0, e[nz]))
        assert np.all(amax[nz] > 6 * np.ldexp(1.0, e[nz] - 1))
        assert np.all(sc[~nz] == 0)
        what = orc.mxfp4_dequant(codes, sc)
        scale = np.repeat(np.ldexp(1.0, e), 32, axis=1)
        assert np.all(np.abs(what - v) <= 0.25 * np.maximum(np.abs(v), scale))
    codes, sc = orc.mxfp4_quantize_weight(W)
    assert sc[4, 1] == 127 - 3 and np.all(codes[4, 16:32] == 0x77)   # every element -> 6


def test_gemm_exact_against_fractions(orc):
    rng = np.random.default_rng(9)
    K = 64
    Xq = rng.integers(0, 256, (3, K)).astype(np.uint8)
    Xq[(Xq & 0x7F) == 0x7F] = 0x38
    codes = rng.integers(0, 256, (4, K // 2)).astype(np.uint8)
    scales = rng.integers(110, 140, (4, K // 32)).astype(np.uint8)
    acc, aacc = orc.mxfp4_gemm(Xq, codes, scales)
    for m in range(3):
        for n in range(4):
            exact = Fraction(0)
            absum = Fraction(0)
            for k in range(K):
                c4 = (int(codes[n, k // 2]) >> (4 * (k & 1))) & 0xF
                w = Fraction(orc.e2m1_decode(c4)) * Fraction(2) ** (int(scales[n, k // 32]) - 127)
                p = Fraction(orc.e4m3_decode(int(Xq[m, k]))) * w
                exact += p
                absum += abs(p)
            assert Fraction(acc[m, n]) == exact and Fraction(aacc[m, n]) == absum


def test_w4a8_product_approximates_the_layer(orc):
    """FP4 weights keep one mantissa bit: the W4A8 product is a coarse but
    unbiased approximation of X W^T (relative L2 of a few tens of percent at
    most on Gaussian data)."""
    W, X = workloads.small_case(32, 16, 64, 1024, x_outlier_mult=1.0)
    Xq, sx = orc.fp8_quantize_act(X)
    codes, sc = orc.mxfp4_quantize_weight(W)
    acc, aacc = orc.mxfp4_gemm(Xq, codes, sc)
    Y, B = orc.mxfp4_reference(acc, aacc, sx)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(Y - exact) / np.linalg.norm(exact)
    assert 0.02 < rel < 0.3, rel
