"""Pins of the oracle's NVFP4 weight path (Quantization notes, FP4 item: E2M1
values with one FP8 E4M3 scale per block of 16, 4.5 bits per weight; the
sketch there: scale = E4M3(amax / 6), codes = the E2M1 value of w / scale).
The block scale is checked against torch's own float8_e4m3fn conversion, the
codes against a brute-force nearest search over the E2M1 value set, the ties
and the degenerate blocks against their closed forms, the storage cost against
the figure the page prints, and the reference product against exact sums."""
import math

import numpy as np
import pytest
import torch

import workloads
from golden_io import load, num

BITS = load("bits_per_weight.txt")
F = load("formats.txt")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def brute_code(x):
    """Nearest E2M1 magnitude by exhaustive search (ties to the even code), sign from x."""
    a = abs(float(x))
    best = min(range(8), key=lambda c: (abs(E2M1[c] - a), c & 1))
    return best | (8 if np.signbit(np.float32(x)) else 0)


def weights(seed, n, k, sigma):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, k)) * sigma).astype(np.float16)


def test_storage_cost_matches_the_page(orc):
    N, K = 3, 256
    codes, scales = orc.nvfp4_quantize(weights(1, N, K, 1.0))
    bits = (codes.nbytes + scales.nbytes) * 8 / (N * K)
    assert bits == num(BITS["nvfp4_block16"])
    assert max(orc.e2m1_decode(c) for c in range(16)) == num(BITS["nvfp4_e2m1_max"])


@pytest.mark.parametrize("sigma", [1e-3, 2e-2, 1.0, 60.0])
def test_block_scale_is_torchs_e4m3_of_amax_over_6(orc, sigma):
    W = weights(2, 16, 512, sigma)
    _, scales = orc.nvfp4_quantize(W)
    amax = np.abs(W.astype(np.float32).reshape(16, 32, 16)).max(axis=2)
    q = (amax / np.float32(6)).astype(np.float32)            # fl32(amax / 6)
    inside = q < 448
    ref = torch.from_numpy(q[inside]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales[inside], ref)
    assert np.all(scales[~inside] == 0x7E)                    # saturated at 448


def test_saturation_and_degenerate_blocks(orc):
    W = np.zeros((4, 64), np.float16)
    W[1, :16] = np.float16(60000.0)                           # amax / 6 > 448
    W[2, 16] = np.float16(6 * 2.0 ** -10)                     # amax / 6 = 2^-10: the tie rounds to 0
    W[2, 32] = np.float16(6 * 2.0 ** -10) * np.float16(1.001)  # just above: the smallest subnormal
    W[3, 48:64] = -np.float16(0.0)
    codes, scales = orc.nvfp4_quantize(W)
    assert scales[0, 0] == 0 and np.all(codes[0] == 0)        # all-zero block
    assert scales[1, 0] == 0x7E and np.all(codes[1, :8] == 0x77)   # 60000 / 448 > 6: clipped to 6
    assert scales[2, 1] == 0 and np.all(codes[2, 8:16] == 0)
    assert scales[2, 2] == 0x01 and codes[2, 16] & 0xF == 0x5  # w / 2^-9 = 3.003: the E2M1 value 3
    assert scales[3, 3] == 0 and np.all(codes[3, 24:32] == 0)  # -0 blocks: scale 0, codes 0


def test_ties_go_to_the_even_code(orc):
    # amax = 6 gives the scale 1.0 exactly, so w / scale = w
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    row = np.zeros(16, np.float16)
    row[0] = 6
    row[1:8] = mids
    row[8:15] = [-m for m in mids]
    codes, scales = orc.nvfp4_quantize(row[None, :])
    assert orc.e4m3_decode(int(scales[0, 0])) == 1.0
    what = orc.nvfp4_dequant(codes, scales)[0]
    assert list(what[1:8]) == want and list(what[8:15]) == [-w for w in want]


@pytest.mark.parametrize("sigma", [2e-2, 1.0])
def test_codes_are_the_nearest_e2m1_value(orc, sigma):
    W = weights(3, 24, 256, sigma)
    W[5, :16] = W[5, :16] * np.float16(0)                     # a zero block among them
    codes, scales = orc.nvfp4_quantize(W)
    u = np.empty((24, 256), np.uint8)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    sc = np.array([[orc.e4m3_decode(int(c)) for c in r] for r in scales], np.float32)
    for n in range(24):
        for k in range(256):
            s = sc[n, k // 16]
            want = 0 if s == 0 else brute_code(np.float32(W[n, k]) / s)
            assert u[n, k] == want, (n, k)


def test_dequantized_weight_is_exact_in_fp16_and_bounded(orc):
    W = weights(4, 32, 512, 0.5)
    codes, scales = orc.nvfp4_quantize(W)
    what = orc.nvfp4_dequant(codes, scales)
    assert np.array_equal(what.astype(np.float16).astype(np.float64), what)
    s = np.repeat(np.array([[orc.e4m3_decode(int(c)) for c in r] for r in scales]), 16, axis=1)
    w = W.astype(np.float64)
    # within half the widest E2M1 gap (1.0) times the scale, or clipped at 6 * scale
    assert np.all(np.abs(what - w) <= np.maximum(s * 1.0, np.abs(w) - 6 * s) + 1e-12)
    assert np.all(np.abs(what) <= 6 * s)


def test_reference_one_hot_and_exact_sums(orc):
    N, K = 20, 128
    W = weights(5, N, K, 0.3)
    codes, scales = orc.nvfp4_quantize(W)
    what = orc.nvfp4_dequant(codes, scales)
    ks = [0, 15, 16, 77, 127]
    X = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1
    Y, B = orc.nvfp4_ref(X, codes, scales)
    for i, k in enumerate(ks):
        assert np.array_equal(Y[i], what[:, k]) and np.array_equal(B[i], np.abs(what[:, k]))
    _, X2 = workloads.small_case(6, 3, N, K)
    Y2, B2 = orc.nvfp4_ref(X2, codes, scales, rows=[2, 0])
    for i, m in enumerate([2, 0]):
        for n in range(N):
            terms = [float(X2[m, k]) * what[n, k] for k in range(K)]
            assert math.isclose(Y2[i, n], math.fsum(terms), rel_tol=0, abs_tol=1e-12 * (1 + B2[i, n]))
            assert math.isclose(B2[i, n], math.fsum(abs(t) for t in terms), rel_tol=1e-14)
