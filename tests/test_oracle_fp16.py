"""Pins of the oracle's binary16 conversions against NumPy's float16 (an
independent implementation of IEEE 754 binary16 with round-to-nearest-even)."""
import numpy as np


def test_h2f_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.h2f(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _boundary_set():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float32)
    v = v[np.isfinite(v)]
    v = np.unique(v)
    mids = (v[:-1].astype(np.float64) + v[1:].astype(np.float64)) / 2
    mids = mids.astype(np.float32)           # fp16 midpoints are exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    extra = np.array([65504, 65519.996, 65520, 65536, 1e6, np.inf, -np.inf,
                      2 ** -24, 2 ** -25, 2 ** -25 * 1.0000001, 2 ** -26, 2 ** -14,
                      2 ** -14 * (1 - 2 ** -12), 0.0, -0.0], np.float32)
    return np.concatenate([v, mids, up, dn, extra, -extra])


@np.errstate(over="ignore")
def test_f2h_boundaries(orc):
    x = _boundary_set()
    ours = orc.f2h(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


@np.errstate(over="ignore")
def test_f2h_random(orc):
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = orc.f2h(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    # and a dense sweep over the fp16 range
    y = rng.uniform(-70000, 70000, 1_000_000).astype(np.float32)
    assert np.array_equal(orc.f2h(y), y.astype(np.float16).view(np.uint16))
