"""Pins of the oracle's AWQ-style scaling on the W4A16 path (Quantization
operators guide §3.2: W'' = W * s, x'' = x / s per input channel; Schemes
notes, AWQ section: Y = X W = (X / s)(W * s)): the identity s = 1, exact
power-of-two scaling, the nearest binary16 of the exact rational product or
quotient (brute force with fractions), the pages' identity
(X / s)(W s)^T = X W^T within the binary16 rounding bound, and the pages'
claim that scaling the salient input channels lowers the INT4 output error."""
from fractions import Fraction

import numpy as np


def _nearest_half(q: Fraction):
    """binary16 value nearest to the rational q (ties to even), and the
    distance from q to the closest binary16 midpoint, both exact."""
    f = np.float16(float(q))
    cands = {f, np.nextafter(f, np.float16(np.inf)), np.nextafter(f, np.float16(-np.inf))}
    cands = [c for c in cands if np.isfinite(c)]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(c.view(np.uint16)) & 1))
    mids = []
    for a in cands:
        for b in cands:
            if a < b:
                mids.append((Fraction(float(a)) + Fraction(float(b))) / 2)
    dist = min(abs(m - q) for m in mids)
    return best, dist


def test_scale_one_is_identity(orc):
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float16)
    X = rng.standard_normal((4, 256)).astype(np.float16)
    one = np.ones(256, np.float32)
    assert np.array_equal(orc.awq_scale_weight(W, one), W.view(np.uint16))
    assert np.array_equal(orc.awq_scale_act(X, one), X.view(np.uint16))


def test_powers_of_two_are_exact(orc):
    rng = np.random.default_rng(2)
    K = 512
    e = rng.integers(-3, 4, K)
    s = np.ldexp(np.ones(K, np.float32), e).astype(np.float32)
    W = rng.standard_normal((16, K)).astype(np.float16)
    X = rng.standard_normal((16, K)).astype(np.float16)
    # keep every scaled value a normal binary16 (no bits lost, no overflow)
    W[np.abs(W) < np.float16(2.0 ** -10)] = np.float16(0.5)
    X[np.abs(X) < np.float16(2.0 ** -10)] = np.float16(-0.75)
    w2 = orc.awq_scale_weight(W, s).view(np.float16)
    x2 = orc.awq_scale_act(X, s).view(np.float16)
    assert np.array_equal(w2, np.ldexp(W, e).astype(np.float16))
    assert np.array_equal(x2, np.ldexp(X, -e).astype(np.float16))


def test_nearest_binary16_of_exact_value(orc):
    """Away from binary16 midpoints (where the binary32 step may decide), the
    scaled value is the binary16 nearest to the exact rational."""
    rng = np.random.default_rng(3)
    K = 400
    s = (np.exp(rng.uniform(-2, 2, K))).astype(np.float32)
    W = rng.standard_normal((3, K)).astype(np.float16)
    X = rng.standard_normal((3, K)).astype(np.float16)
    w2 = orc.awq_scale_weight(W, s).view(np.float16)
    x2 = orc.awq_scale_act(X, s).view(np.float16)
    checked = 0
    for n in range(3):
        for k in range(K):
            for val, is_w in ((W[n, k], True), (X[n, k], False)):
                q = Fraction(float(val)) * Fraction(float(s[k])) if is_w else \
                    Fraction(float(val)) / Fraction(float(s[k]))
                best, dist = _nearest_half(q)
                if q != 0 and dist <= abs(q) * Fraction(1, 2 ** 23):
                    continue
                got = w2[n, k] if is_w else x2[n, k]
                assert got.view(np.uint16) == best.view(np.uint16), (n, k, is_w)
                checked += 1
    assert checked > 0.99 * 2 * 3 * K


def test_page_identity(orc):
    """(X / s)(W s)^T equals X W^T up to the two binary16 roundings."""
    rng = np.random.default_rng(4)
    M, N, K = 6, 10, 1024
    s = (np.exp(rng.uniform(-1.5, 1.5, K))).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.5).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float16)
    W[np.abs(W) < np.float16(2.0 ** -8)] = np.float16(0.25)
    X[np.abs(X) < np.float16(2.0 ** -8)] = np.float16(0.25)
    w2 = orc.awq_scale_weight(W, s).view(np.float16).astype(np.float64)
    x2 = orc.awq_scale_act(X, s).view(np.float16).astype(np.float64)
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    lhs = x2 @ w2.T
    rhs = Xd @ Wd.T
    bound = np.abs(Xd) @ np.abs(Wd).T
    assert np.all(np.abs(lhs - rhs) <= bound * (2 * 2.0 ** -11 * (1 + 2.0 ** -10)) + 1e-12)
    # the scale on the wrong side breaks it
    bad = orc.awq_scale_act(X, 1.0 / s).view(np.float16).astype(np.float64) @ w2.T
    assert np.max(np.abs(bad - rhs) / bound) > 1e-2


def test_awq_lowers_int4_error_on_salient_channels(orc):
    """Schemes notes / Operators guide §3.2 (qualitative): with 1% of input
    channels carrying ~20x larger activations, s = act^alpha / mean (the pages'
    search form, alpha = 0.5) gives a smaller W4A16 output error than plain
    INT4 of W."""
    rng = np.random.default_rng(5)
    M, N, K = 64, 512, 1024
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, rng.permutation(K)[:K // 100]] *= 20
    X = X.astype(np.float16)
    exact = X.astype(np.float64) @ W.astype(np.float64).T

    def out(Xa, Wa):
        codes, scales, zeros = orc.q4_quantize_pack(Wa, g=128, sym=False)
        return orc.w4a16_ref(Xa, codes, scales, zeros)[0]

    plain = np.sqrt(np.mean((out(X, W) - exact) ** 2))
    act = np.abs(X.astype(np.float64)).mean(axis=0)
    s = act ** 0.5
    s = (s / s.mean()).astype(np.float32)
    scaled = out(orc.awq_scale_act(X, s), orc.awq_scale_weight(W, s))
    awq = np.sqrt(np.mean((scaled - exact) ** 2))
    assert awq < 0.85 * plain, (awq, plain)
