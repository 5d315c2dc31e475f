"""Pins of the oracle's group-wise INT4 quantizer (CPU only).

What fixes the quantizer, independently of the oracle's own code:
  * an exhaustive search over the 16 code levels (argmin of the distance to
    the fp32 quotient, ties to the even level) for every fp16 value inside a
    set of group ranges -- a different formulation of round + clip;
  * the code is the nearest representable level in exact arithmetic;
  * closed forms: x = 0 maps to zp; |x| = max|x| maps to +-7 (symmetric);
  * the worked example of the Quantization schemes notes (step 0.427 over
    [-3.2, 3.2]; w = 0.21 -> 0);
  * the error table of Core ideas §2.3 (256 x 512, seed 0);
  * bits per weight from Quantization operators guide §3.3 / Quantization
    notes item (1).
"""
import numpy as np
import pytest

from golden_io import load, num

ALL_H = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_H = np.unique(ALL_H[np.isfinite(ALL_H)].astype(np.float32))


def unpack_nibbles(packed, count):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int64)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out[..., :count]


def brute_codes(x32, sf, zp):
    """argmin over u in [0, 15] of |fl32(x / sf) - (u - zp)|, ties to the even
    level (u - zp). Returns u."""
    t = (x32.astype(np.float32) / np.float32(sf)).astype(np.float64)
    levels = np.arange(16) - zp
    d = np.abs(t[:, None] - levels[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = (levels % 2 == 0)[None, :]
    tie = cand.sum(axis=1) > 1
    return np.where(tie, np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))


def groups_from_values(vals, ends, g=128):
    """Rows of g fp16 values: the two range ends first, then the values."""
    body = g - len(ends)
    n = -(-len(vals) // body)
    padded = np.zeros(n * body, np.float32)
    padded[: len(vals)] = vals
    rows = np.empty((n, g), np.float32)
    rows[:, : len(ends)] = ends
    rows[:, len(ends):] = padded.reshape(n, body)
    return rows.astype(np.float16)


ASYM_RANGES = [(-1.0, 1.0), (-0.3, 2.5), (-3.2, 3.2), (0.001, 1.0), (-2.0, -0.5),
               (-2.0 ** -12, 3 * 2.0 ** -13), (-6e-7, 5e-7), (-60000.0, 65504.0),
               (-0.02, 0.08)]


@pytest.mark.parametrize("lo,hi", ASYM_RANGES)
def test_asym_codes_exhaustive(orc, lo, hi):
    lo16, hi16 = np.float32(np.float16(lo)), np.float32(np.float16(hi))
    vals = FINITE_H[(FINITE_H >= lo16) & (FINITE_H <= hi16)]
    W = groups_from_values(vals, [lo16, hi16])
    codes, scales, zeros = orc.q4_quantize_pack(W, g=128, sym=False)
    u = unpack_nibbles(codes, 128)
    zp = unpack_nibbles(zeros, 1)[:, 0]
    sf = scales.astype(np.float32)[:, 0]
    x = W.astype(np.float32)
    # one group per row: the widened range of the row defines s and zp
    lo_w = np.minimum(0, x.min(1))
    hi_w = np.maximum(0, x.max(1))
    s32 = (hi_w - lo_w) / np.float32(15)
    s16 = s32.astype(np.float16).astype(np.float32)
    s16[s16 == 0] = 1.0
    assert np.array_equal(sf, s16)
    assert np.all((zp >= 0) & (zp <= 15))
    for r in range(W.shape[0]):
        assert zp[r] == int(np.clip(np.rint(np.float32(-lo_w[r]) / np.float32(sf[r])), 0, 15))
        assert np.array_equal(u[r], brute_codes(x[r], sf[r], zp[r])), r
    # the code is the nearest level in exact arithmetic (up to the fp32 quotient)
    xd = x.astype(np.float64)
    lev = (np.arange(16)[None, None, :] - zp[:, None, None]) * sf[:, None, None].astype(np.float64)
    dist = np.abs(xd[:, :, None] - lev)
    chosen = np.take_along_axis(dist, u[:, :, None], axis=2)[..., 0]
    slack = 2.0 ** -22 * np.maximum(np.abs(xd), sf[:, None])
    assert np.all(chosen <= dist.min(axis=2) + slack)
    # error bound, clipped ends included: half a step, plus the 15 steps' share
    # of the scale's fp16 rounding (at most 15 * 2^-11 of a step for a normal
    # fp16 scale, more for a subnormal one)
    w_hat = (u - zp[:, None]) * sf[:, None].astype(np.float64)
    err = np.abs(xd - w_hat)
    bound = 0.5 * sf + 15 * np.abs(s32.astype(np.float64) - sf) + 2.0 ** -22 * np.abs(x).max(1)
    assert np.all(err <= bound[:, None])
    normal = sf >= 2.0 ** -14
    assert np.all(err[normal] <= 0.51 * sf[normal, None])
    # x = 0 maps to zp
    assert np.all(u[x == 0] == np.broadcast_to(zp[:, None], u.shape)[x == 0])


@pytest.mark.parametrize("amax", [1.0, 0.37, 3.2, 2.0 ** -13, 5e-7, 65504.0, 0.06])
def test_sym_codes_exhaustive(orc, amax):
    a16 = np.float32(np.float16(amax))
    vals = FINITE_H[np.abs(FINITE_H) <= a16]
    W = groups_from_values(vals, [a16, -a16])
    codes, scales, zeros = orc.q4_quantize_pack(W, g=128, sym=True)
    assert zeros is None
    u = unpack_nibbles(codes, 128)
    sf = scales.astype(np.float32)[:, 0]
    x = W.astype(np.float32)
    s16 = np.float32(np.float16(np.abs(x).max(1) / np.float32(7)))
    s16 = np.where(s16 == 0, np.float32(1), s16)
    assert np.array_equal(sf, s16.astype(np.float32))
    for r in range(W.shape[0]):
        assert np.array_equal(u[r], brute_codes(x[r], sf[r], 8)), r
    # |x| = max|x| maps to +-7 unless the fp16 scale is subnormal and rounds far
    # from max/7 (then the clip at -8/+7 decides)
    if sf[0] >= 2.0 ** -14:
        assert u[0, 0] == 15 and u[0, 1] == 1
    assert np.all(u[x == 0] == 8)


def test_all_zero_and_constant_groups(orc):
    W = np.zeros((4, 256), np.float16)
    W[1, :128] = 0.5                       # constant positive group
    W[2, 128:] = -0.25                     # constant negative group
    W[3, :] = np.float16(2.0 ** -24)       # smallest subnormal everywhere
    for sym in (False, True):
        codes, scales, zeros = orc.q4_quantize_pack(W, g=128, sym=sym)
        u = unpack_nibbles(codes, 256)
        zp = np.full((4, 2), 8) if sym else unpack_nibbles(zeros, 2)
        w_hat = orc.q4_dequant(codes, scales, zeros, 256, 128)
        # an all-zero group has scale 1.0 and dequantizes to exactly 0
        assert scales[0, 0] == np.float16(1.0)
        assert np.all(w_hat[0] == 0)
        assert np.all(u[0] == zp[0, 0])
        # constant groups: within half a step (the end value sits on the top
        # level up to the scale's fp16 rounding); zeros stay exactly zero
        sf = np.repeat(scales.astype(np.float64), 128, axis=1)
        assert np.all(np.abs(w_hat - W.astype(np.float64)) <= 0.51 * sf)
        assert np.all(w_hat[1, 128:] == 0) and np.all(w_hat[2, :128] == 0)
        assert abs(w_hat[1, 0] - 0.5) <= 15 * 2.0 ** -11 * 0.5


def test_p1_worked_example(orc):
    ex = load("p1_uniform_int4_example.txt")
    lo, hi, w = num(ex["range_lo"]), num(ex["range_hi"]), num(ex["w"])
    rng = np.random.default_rng(1)
    row = rng.uniform(lo, hi, 128).astype(np.float32)
    row[0], row[1], row[2] = lo, hi, w
    W = row.astype(np.float16)[None, :]
    codes, scales, zeros = orc.q4_quantize_pack(W, g=128, sym=False)
    step = float(scales[0, 0])
    assert round(step, 3) == num(ex["step"])
    assert abs(step - (hi - lo) / (num(ex["levels"]) - 1)) < 2 ** -11
    w_hat = orc.q4_dequant(codes, scales, zeros, 128, 128)[0]
    assert w_hat[2] == num(ex["w_hat"])
    assert abs(float(W[0, 2]) - w_hat[2]) == pytest.approx(num(ex["error"]), abs=1e-3)


def test_p5_granularity_table(orc):
    """Core ideas §2.3: symmetric RTN error by granularity on a 256 x 512
    N(0, 1) weight. The page's numbers come from an fp64 scale; the oracle
    stores an fp16 scale, so each cell is held to +-0.001."""
    tab = load("p5_granularity_rel_l2.txt")
    W64 = np.random.default_rng(0).standard_normal((256, 512))
    W16 = W64.astype(np.float16)
    Wd = W16.astype(np.float64)

    def rel(w_hat):
        return np.linalg.norm(Wd - w_hat) / np.linalg.norm(Wd)

    errs = {}
    for g in (128, 32):
        codes, scales, zeros = orc.q4_quantize_pack(W16, g=g, sym=True)
        errs[g] = rel(orc.q4_dequant(codes, scales, zeros, 512, g))
    assert errs[128] == pytest.approx(num(tab["group_128"])[1], abs=1e-3)
    assert errs[32] == pytest.approx(num(tab["group_32"])[1], abs=1e-3)
    drop = 100 * (1 - errs[32] / errs[128])
    assert drop == pytest.approx(num(tab["g128_to_g32_error_drop_percent"]), abs=1.0)
    # per-channel INT8 (the INT8 weight quantizer with no smoothing)
    Wq, sw = orc.q8_quantize_weight(W16)
    e8 = rel(Wq.astype(np.float64) * sw[:, None].astype(np.float64))
    assert e8 == pytest.approx(num(tab["per_channel"])[0], abs=5e-4)


@pytest.mark.parametrize("g,sym,key", [(128, True, "sym_g128"), (32, True, "sym_g32"),
                                       (128, False, "asym_g128")])
def test_bits_per_weight(orc, g, sym, key):
    bits = load("bits_per_weight.txt")
    N, K = 64, 1024
    W = np.random.default_rng(3).standard_normal((N, K)).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=sym)
    total = codes.nbytes + scales.nbytes + (0 if zeros is None else zeros.nbytes)
    assert 8 * total / (N * K) == num(bits[key])
    if sym:
        per_group = (codes.nbytes + scales.nbytes) / (N * K // g)
        assert per_group == num(bits[f"bytes_per_group_g{g}"])


def test_pack_order_and_odd_group_count(orc):
    """Even k in the low nibble; zero-points of groups 2i and 2i+1 share a
    byte, low nibble first; an odd group count leaves a zero high nibble."""
    rng = np.random.default_rng(11)
    N, K, g = 5, 3 * 64, 64
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=False)
    assert codes.shape == (N, K // 2) and scales.shape == (N, 3) and zeros.shape == (N, 2)
    assert np.all(zeros[:, 1] >> 4 == 0)
    u = unpack_nibbles(codes, K)
    zp = unpack_nibbles(zeros, 3)
    w_hat = orc.q4_dequant(codes, scales, zeros, K, g)
    expect = (u - np.repeat(zp, g, axis=1)) * np.repeat(scales.astype(np.float64), g, axis=1)
    assert np.array_equal(w_hat, expect)
    # re-quantizing element by element from the stored scale/zp gives the same codes
    x = W.astype(np.float32)
    for n in range(N):
        for j in range(3):
            sl = slice(j * g, (j + 1) * g)
            assert np.array_equal(u[n, sl], brute_codes(x[n, sl], np.float32(scales[n, j]), zp[n, j]))


def test_rejects_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.q4_quantize_pack(np.zeros((2, 100), np.float16), g=128)
