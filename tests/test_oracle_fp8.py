"""Pins of the oracle's FP8 E4M3 path (Quantization operators guide §4.1,
§4.2; Core ideas §2.1): the encoder against a brute-force nearest search
over the 254 finite codes and, independently, PyTorch's float8_e4m3fn cast;
the per-row quantizers against closed forms and the format's error bound;
the GEMM reference against exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def table(orc):
    return {c: orc.e4m3_decode(c) for c in FINITE}


def brute_encode(vals, x):
    """Nearest finite E4M3 value with the sign of x, ties to the even code."""
    neg = np.signbit(np.float32(x))
    best = None
    for c, v in vals.items():
        if bool(c & 0x80) != bool(neg):
            continue
        d = abs(Fraction(float(v)) - Fraction(float(x)))
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_decode_encode_round_trip(orc):
    for c in FINITE:
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c, hex(c)


def test_midpoints_and_neighbours(orc):
    vals = table(orc)
    pos = sorted((v, c) for c, v in vals.items() if c < 0x80)
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (v0 + v1) / 2          # exact in fp32 (both are short binary fractions)
        even = c0 if c0 % 2 == 0 else c1
        assert orc.e4m3_encode(mid) == even
        assert orc.e4m3_encode(-mid) == even | 0x80
        assert orc.e4m3_encode(np.nextafter(np.float32(mid), np.float32(0))) == c0
        assert orc.e4m3_encode(np.nextafter(np.float32(mid), np.float32(1e9))) == c1


def test_brute_force_nearest(orc):
    vals = table(orc)
    rng = np.random.default_rng(3)
    xs = list(rng.standard_normal(400).astype(np.float32) * np.float32(60))
    xs += list((rng.standard_normal(200) * 0.01).astype(np.float32))
    xs += [np.float32(v) for v in (0.0, -0.0, 447.9, 448.0, 455.9, 464.0, 500.0, -1e6, 2.0 ** -10,
                                   3 * 2.0 ** -11, 2.0 ** -6 - 2.0 ** -12)]
    for x in xs:
        assert orc.e4m3_encode(float(x)) == brute_encode(vals, x), x


def test_every_fp16_against_torch(orc):
    """All finite fp16 values (and their products by 1/64 and 300) that lie
    within the range where both encoders are defined alike (|x| <= 464)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = h[np.isfinite(h)].astype(np.float32)
    for mult in (1.0, 1.0 / 64, 300.0):
        x = (f * np.float32(mult)).astype(np.float32)
        x = x[np.abs(x) <= 464]
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = np.array([orc.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
        assert np.array_equal(got, ref), mult


def test_saturation(orc):
    # the guide clamps to the format maximum before casting: beyond 448 -> +-448
    for x in (449.0, 480.0, 1e4, 3.0e38):
        assert orc.e4m3_encode(x) == 0x7E and orc.e4m3_encode(-x) == 0xFE


@pytest.mark.parametrize("which", ["weight", "act"])
def test_row_quantizer_closed_forms(orc, which):
    quant = orc.fp8_quantize_weight if which == "weight" else orc.fp8_quantize_act
    # a constant row: every code is the maximum, scale = v / 448
    X = np.full((2, 64), 3.5, np.float16)
    X[1] = -3.5
    q, sc = quant(X)
    assert np.all(q[0] == 0x7E) and np.all(q[1] == 0xFE)
    assert np.all(sc == np.float32(3.5) / np.float32(448))
    # an all-zero row: codes 0, scale floored at 1e-8 / 448
    q, sc = quant(np.zeros((1, 32), np.float16))
    assert np.all(q == 0) and sc[0] == np.float32(1e-8) / np.float32(448)


@pytest.mark.parametrize("which", ["weight", "act"])
def test_row_quantizer_error_bound(orc, which):
    W, X = workloads.small_case(21, 40, 30, 512)
    A = W if which == "weight" else X
    s = (np.abs(np.random.default_rng(4).standard_normal(512)) + 0.5).astype(np.float32)
    quant = orc.fp8_quantize_weight if which == "weight" else orc.fp8_quantize_act
    q, sc = quant(A, s)
    v = A.astype(np.float32) * s if which == "weight" else A.astype(np.float32) / s
    dec = np.vectorize(orc.e4m3_decode)(q).astype(np.float64) * sc[:, None]
    # the largest |v| of each row is coded as +-448 (its quotient rounds to 448)
    amax_idx = np.argmax(np.abs(v), axis=1)
    assert np.all(np.isin(q[np.arange(len(q)), amax_idx], (0x7E, 0xFE)))
    # E4M3: half a quantum, 2^-4 relative for normals, 2^-10 * scale below 2^-6 * scale
    err = np.abs(dec - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * sc[:, None]) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_gemm_exact_against_fractions(orc):
    rng = np.random.default_rng(5)
    Xq = rng.integers(0, 256, (3, 37)).astype(np.uint8)
    Wq = rng.integers(0, 256, (4, 37)).astype(np.uint8)
    Xq[Xq == 0x7F] = 0x7E
    Xq[Xq == 0xFF] = 0xFE
    Wq[Wq == 0x7F] = 0x01
    Wq[Wq == 0xFF] = 0x81
    acc, aacc = orc.fp8_gemm(Xq, Wq)
    for m in range(3):
        for n in range(4):
            exact = sum(Fraction(orc.e4m3_decode(int(a))) * Fraction(orc.e4m3_decode(int(b)))
                        for a, b in zip(Xq[m], Wq[n]))
            absum = sum(abs(Fraction(orc.e4m3_decode(int(a))) * Fraction(orc.e4m3_decode(int(b))))
                        for a, b in zip(Xq[m], Wq[n]))
            assert Fraction(acc[m, n]) == exact and Fraction(aacc[m, n]) == absum
    acc_r, _ = orc.fp8_gemm(Xq, Wq, rows=[2, 0])
    assert np.array_equal(acc_r, acc[[2, 0]])


def test_gemm_closed_form(orc):
    K = 8192
    acc, aacc = orc.fp8_gemm(np.full((2, K), 0x7E, np.uint8), np.full((3, K), 0xFE, np.uint8))
    assert np.all(acc == -448.0 * 448.0 * K) and np.all(aacc == 448.0 * 448.0 * K)


def test_scaled_product_approximates_the_layer(orc):
    """The guide's C = scale_A scale_B (A_fp8 @ B_fp8) stays close to X W^T:
    E4M3 carries 3 mantissa bits, so the relative L2 error is a few percent."""
    W, X = workloads.small_case(22, 16, 64, 1024, x_outlier_mult=1.0)
    Xq, sx = orc.fp8_quantize_act(X)
    Wq, sw = orc.fp8_quantize_weight(W)
    acc, aacc = orc.fp8_gemm(Xq, Wq)
    Y, B = orc.fp8_reference(acc, aacc, sx, sw)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(Y - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 0.06, rel
