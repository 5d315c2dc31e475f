"""The division-free quotients the INT8 row quantizer relies on, checked on the
host with numpy (no GPU code involved).

For a binary16-valued (or binary32) numerator a and a binary32 divisor b, the
exact quotient a / b never lies on a midpoint between two binary32 neighbours
and otherwise stays at least 2^-49 (relative) away from one (a - m b is a
nonzero multiple of 2^(ea - 25) for a = A 2^ea,
A < 2^24, and a midpoint m of 25 significant bits), so a fp64 product with a
reciprocal of b accurate to ~2^-50 rounds to the same binary32
value as the IEEE division: fl32(fl64(a * r)) == fl32(a / b). The kernel's r is
the fp64 hardware reciprocal refined by two Newton steps; here the starting
point is deliberately worse (14 significant bits, perturbed) so that the
refinement, not the starting accuracy, carries the result."""
import numpy as np

FINITE_F16 = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_F16 = FINITE_F16[np.isfinite(FINITE_F16)].astype(np.float32)


def refined_reciprocal(b: np.ndarray, rng) -> np.ndarray:
    b64 = b.astype(np.float64)
    m, e = np.frexp(1.0 / b64)
    r = np.ldexp(np.round(m * 16384.0) / 16384.0, e)                 # 14 bits
    r *= 1.0 + (rng.integers(-500, 500, size=b.shape) * 1e-8)          # and perturbed
    for _ in range(2):                                                 # Newton: r + r (1 - b r)
        r = r + r * (1.0 - b64 * r)   # fp64 fma-free form is within the same error budget
    return r


def divisors(rng, n: int) -> np.ndarray:
    exp = rng.integers(127 - 30, 127 + 31, size=n).astype(np.uint32)
    man = rng.integers(0, 1 << 23, size=n).astype(np.uint32)
    man[0::4] = 0x7FFFFF - (man[0::4] & 63)   # just below powers of two
    man[1::4] = man[1::4] & 63                 # just above
    man[2::4] = man[2::4] & 0x7FF000           # short mantissas
    return ((exp << 23) | man).view(np.float32)


def test_fp16_numerator_every_value():
    rng = np.random.default_rng(11)
    s = divisors(rng, 2000)
    r = refined_reciprocal(s, rng)
    x = FINITE_F16
    for i in range(len(s)):
        ref = x / s[i]                                                  # IEEE binary32 division
        got = (x.astype(np.float64) * r[i]).astype(np.float32)
        bad = (ref != got) & ~((ref == 0) & (got == 0))
        assert not bad.any(), f"x={x[bad][0]!r} s={s[i]!r}"


def test_fp32_numerator_random():
    rng = np.random.default_rng(12)
    n = 2_000_000
    v = rng.integers(0x0D000000, 0x72000000, size=n, dtype=np.uint32).view(np.float32)
    c = divisors(rng, n)
    with np.errstate(over="ignore"):
        ref = v / c
        got = (v.astype(np.float64) * refined_reciprocal(c, rng)).astype(np.float32)
    ok = np.isfinite(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_scale_shaped_divisors():
    # v / (amax / 127) with |v| <= amax: the activation quantizer's second quotient
    rng = np.random.default_rng(13)
    amax = (np.abs(rng.standard_normal(20000)) * 30 + 1e-3).astype(np.float32)
    scale = amax / np.float32(127.0)
    r = refined_reciprocal(scale, rng)
    frac = rng.uniform(-1, 1, size=(64, amax.size)).astype(np.float32)
    v = (frac * amax).astype(np.float32)
    ref = v / scale
    got = (v.astype(np.float64) * r).astype(np.float32)
    assert np.array_equal(ref, got)
