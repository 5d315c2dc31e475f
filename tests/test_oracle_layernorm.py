"""Pins of the oracle's LayerNorm + SmoothQuant divide + per-token INT8
quantizer (Quantization operators guide §5.3, deployment fusion). CPU only.

  * x' agrees with torch's own layer_norm in fp64 (weight gamma / s, bias
    beta / s) after rounding to fp32, and the statistics with torch's biased
    var_mean: an independent library routine for the normalisation;
  * the statistics come from exact sums: with S1 and S2 computed with Python
    integers and rounded by Python's correctly rounded int -> float, the
    oracle's variance is the same double bit for bit, on rows built so that
    a plain running fp64 sum of the squares would round differently;
  * the 128-bit -> fp64 rounding the oracle relies on equals Python's on
    random values and on exact ties;
  * scaling a row by 4 (and eps by 16) leaves x', codes and scales unchanged
    bit for bit, and permuting the columns (with gamma, beta, s) permutes
    them: both hold exactly only if nothing depends on summation order;
  * closed forms: a constant row normalises to zero; a row of +-a to
    +-a / sqrt(a^2 + eps) with codes +-127; gamma = 0 leaves fl32(beta / s);
  * the codes are the per-token quantizer's: every code within half a step
    of x' / sx, the largest |x'| of a row at +-127;
  * a row holding a NaN or an infinity, or whose x' overflows fp32, is
    flagged (NaN scale, zero codes) and no other row changes;
  * the FP8 form: the same x' with scale max|x'| / 448, every code equal to
    torch's float8_e4m3fn cast of fl32(x' / scale), the row maximum at
    +-448, flagged rows as in the INT8 form.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch


def _params(K, seed=7):
    rng = np.random.default_rng(seed)
    gamma = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    beta = (0.05 * rng.standard_normal(K)).astype(np.float32)
    s = np.exp(0.5 * rng.standard_normal(K)).astype(np.float32)
    return gamma, beta, s


def _act(M, K, seed=11):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, rng.permutation(K)[: max(1, K // 100)]] *= 30
    return X.astype(np.float16)


def _adversarial(K, seed=5):
    """Rows with a few fp16 maxima and many values whose squares sit below
    half an fp64 ulp of the running sum: a plain sequential fp64 sum of
    the squares drops them, the exact sum does not."""
    rng = np.random.default_rng(seed)
    rows = []
    for big in (65504.0, 30000.0, 4096.0):
        r = np.full(K, 2.0 ** -11, np.float32) * rng.choice([-1.0, 1.0], K).astype(np.float32)
        r[rng.choice(K, 3, replace=False)] = [big, -big, big / 2]
        rows.append(r)
    return np.array(rows, np.float32).astype(np.float16)


def _ulp32(a):
    return np.spacing(np.abs(a).astype(np.float32)).astype(np.float64)


@pytest.mark.parametrize("M,K", [(32, 1024), (8, 8192), (5, 200)])
def test_matches_torch_layer_norm(orc, M, K):
    X = _act(M, K)
    gamma, beta, s = _params(K)
    eps = 1e-5
    Xq, sx, xs, st = orc.layernorm_quant_smooth(X, gamma, beta, s, eps, want_x=True)
    x64 = torch.from_numpy(X.astype(np.float64))
    w = torch.from_numpy(gamma.astype(np.float64) / s.astype(np.float64))
    b = torch.from_numpy(beta.astype(np.float64) / s.astype(np.float64))
    ref = torch.nn.functional.layer_norm(x64, (K,), weight=w, bias=b, eps=eps).numpy()
    ref32 = ref.astype(np.float32)
    diff = np.abs(xs.astype(np.float64) - ref32.astype(np.float64))
    assert (diff <= _ulp32(ref32)).all()
    assert (xs == ref32).mean() > 0.999
    var, mean = torch.var_mean(x64, dim=1, unbiased=False)
    np.testing.assert_allclose(st[:, 0], mean.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(st[:, 1], var.numpy(), rtol=1e-12)
    np.testing.assert_allclose(st[:, 2], 1.0 / np.sqrt(var.numpy() + eps), rtol=1e-12)
    # and the codes are those of the per-token quantizer on x'
    q = xs.astype(np.float64) / sx[:, None].astype(np.float64)
    assert (np.abs(q - Xq) <= 0.5 + 1e-6).all()
    assert (np.abs(Xq).max(axis=1) == 127).all()


def test_statistics_from_exact_sums(orc):
    K = 8192
    X = _adversarial(K)
    gamma, beta, _ = _params(K)
    _, _, _, st = orc.layernorm_quant_smooth(X, gamma, beta, None, 1e-5, want_x=True)
    naive_differs = 0
    for m in range(X.shape[0]):
        xv = [Fraction(float(v)) for v in X[m].astype(np.float64)]
        a = [int(v * 2 ** 24) for v in xv]
        assert all(Fraction(ai, 2 ** 24) == v for ai, v in zip(a, xv))
        s1 = sum(a)
        s2 = sum(ai * ai for ai in a)
        mean = (s1 * 2.0 ** -24) / K
        ex2 = (float(s2) * 2.0 ** -48) / K
        var = max(ex2 - mean * mean, 0.0)
        assert st[m, 0] == mean and st[m, 1] == var
        # a sequential fp64 sum of the squares rounds differently here
        acc = 0.0
        for v in X[m].astype(np.float64):
            acc += v * v
        naive_differs += (acc != float(s2) * 2.0 ** -48)
        exact_var = Fraction(s2, 2 ** 48 * K) - Fraction(s1, 2 ** 24 * K) ** 2
        assert abs(Fraction(var) - exact_var) <= 4 * 2.0 ** -53 * (ex2 + mean * mean)
    assert naive_differs >= 1


def test_u128_rounding(orc):
    rng = np.random.default_rng(3)
    vals = [int(rng.integers(0, 2 ** 62)) << int(rng.integers(0, 66)) | int(rng.integers(0, 2 ** 40))
            for _ in range(2000)]
    # exact ties half an ulp above a 53-bit significand (odd: rounds up to
    # even; even: rounds down), and one unit either side of the tie
    for sh in (10, 40, 70):
        for sig in ((1 << 52) + 1, (1 << 52) + 2, (1 << 53) - 1):
            tie = sig << (sh + 1) | (1 << sh)
            vals += [tie, tie + 1, tie - 1]
    vals += [0, 1, 2 ** 64 - 1, 2 ** 64, 2 ** 128 - 1]
    for v in vals:
        v &= (1 << 128) - 1
        assert orc.u128_to_double(v) == float(v), v


def test_power_of_two_scaling_is_exact(orc):
    M, K = 16, 2048
    X = np.clip(_act(M, K).astype(np.float32), -4000, 4000).astype(np.float16)
    gamma, beta, s = _params(K)
    base = orc.layernorm_quant_smooth(X, gamma, beta, s, 1e-5, want_x=True)
    X4 = (X.astype(np.float32) * 4).astype(np.float16)
    assert (X4.astype(np.float32) == X.astype(np.float32) * 4).all()
    sc = orc.layernorm_quant_smooth(X4, gamma, beta, s, 1e-5 * 16, want_x=True)
    np.testing.assert_array_equal(sc[0], base[0])
    np.testing.assert_array_equal(sc[1], base[1])
    np.testing.assert_array_equal(sc[2], base[2])


def test_column_permutation(orc):
    K = 8192
    X = np.concatenate([_adversarial(K), _act(4, K)])
    gamma, beta, s = _params(K)
    Xq, sx, xs, _ = orc.layernorm_quant_smooth(X, gamma, beta, s, 1e-5, want_x=True)
    p = np.random.default_rng(9).permutation(K)
    Xq2, sx2, xs2, _ = orc.layernorm_quant_smooth(np.ascontiguousarray(X[:, p]), gamma[p], beta[p], s[p],
                                                  1e-5, want_x=True)
    np.testing.assert_array_equal(xs2, xs[:, p])
    np.testing.assert_array_equal(Xq2, Xq[:, p])
    np.testing.assert_array_equal(sx2, sx)


def test_closed_forms(orc):
    K = 512
    ones, zeros = np.ones(K, np.float32), np.zeros(K, np.float32)
    # a constant row: variance 0, every x' = 0 -> codes 0 and the floored scale
    X = np.full((2, K), 3.25, np.float16)
    X[1] = -0.0078125
    Xq, sx, xs, st = orc.layernorm_quant_smooth(X, ones, zeros, None, 1e-5, want_x=True)
    assert (st[:, 1] == 0).all() and (xs == 0).all() and (Xq == 0).all()
    assert (sx == np.float32(np.float32(1e-8) / np.float32(127))).all()
    # a row of +-a: mean 0, variance a^2, x' = +-a / sqrt(a^2 + eps), codes +-127
    a = 1.5
    X = np.where(np.arange(K) % 2 == 0, a, -a).astype(np.float16)[None, :]
    Xq, sx, xs, st = orc.layernorm_quant_smooth(X, ones, zeros, None, 1e-5, want_x=True)
    v = a / np.sqrt(a * a + 1e-5)
    assert st[0, 0] == 0 and st[0, 1] == a * a
    np.testing.assert_array_equal(xs[0], np.where(np.arange(K) % 2 == 0, v, -v).astype(np.float32))
    np.testing.assert_array_equal(Xq[0], np.where(np.arange(K) % 2 == 0, 127, -127))
    # gamma = 0: x' is the folded bias beta / s whatever x is
    _, beta, s = _params(K)
    X = _act(3, K)
    _, _, xs, _ = orc.layernorm_quant_smooth(X, zeros, beta, s, 1e-5, want_x=True)
    ref = (beta.astype(np.float64) / s.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(xs, np.broadcast_to(ref, xs.shape))


def test_nonfinite_rows_flagged(orc):
    M, K = 6, 256
    X = _act(M, K)
    gamma, beta, s = _params(K)
    clean_q, clean_s = orc.layernorm_quant_smooth(X, gamma, beta, s)
    Xb = X.copy()
    Xb[1, 7] = np.float16(np.nan)
    Xb[3, 0] = np.float16(np.inf)
    Xb[4, 255] = np.float16(-np.inf)
    q, sc = orc.layernorm_quant_smooth(Xb, gamma, beta, s)
    for m in (1, 3, 4):
        assert np.isnan(sc[m]) and (q[m] == 0).all()
    for m in (0, 2, 5):
        assert sc[m] == clean_s[m] and (q[m] == clean_q[m]).all()
    # an x' past the fp32 range (beta / s overflows) flags its row too
    big = beta.copy()
    big[5] = 3e38
    s2 = s.copy()
    s2[5] = 1e-3
    q, sc = orc.layernorm_quant_smooth(X, gamma, big, s2)
    assert np.isnan(sc).all() and (q == 0).all()


def test_fp8_form(orc):
    M, K = 24, 2048
    X = _act(M, K)
    X[3, 9] = np.float16(np.nan)
    gamma, beta, s = _params(K)
    q8, sx8, xs, _ = orc.layernorm_quant_smooth(X, gamma, beta, s, 1e-5, want_x=True)
    q, sx = orc.layernorm_quant_smooth_fp8(X, gamma, beta, s, 1e-5)
    ok = np.isfinite(sx8)
    assert np.array_equal(np.isnan(sx), ~ok) and (q[~ok] == 0).all()
    a = np.abs(xs[ok]).max(axis=1)
    np.testing.assert_array_equal(sx[ok], (np.maximum(a, np.float32(1e-8)) / np.float32(448)).astype(np.float32))
    quot = (xs[ok] / sx[ok][:, None]).astype(np.float32)
    ref = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q[ok], ref)
    assert ((q[ok] & 0x7F) == 0x7E).any(axis=1).all()   # the row maximum at +-448
