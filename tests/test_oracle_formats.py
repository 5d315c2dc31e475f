"""Pins of the oracle's small-float decoders against the limits printed on
the Core ideas page (§2.1) and, independently, PyTorch's float8 dtypes."""
import numpy as np
import torch

from golden_io import load, num

F = load("formats.txt")


def test_e2m1_value_set(orc):
    vals = sorted(orc.e2m1_decode(c) for c in range(16))
    want = sorted(num(F["e2m1_values"]))
    assert vals == want


def test_e4m3_limits(orc):
    vals = np.array([orc.e4m3_decode(c) for c in range(256)])
    nan_codes = [c for c in range(256) if np.isnan(vals[c])]
    assert nan_codes == num(F["e4m3_nan_codes"])
    fin = vals[np.isfinite(vals)]
    assert fin.max() == num(F["e4m3_max"]) and fin.min() == -num(F["e4m3_max"])
    pos = fin[fin > 0]
    normals = [orc.e4m3_decode(c) for c in range(8, 0x7f)]
    assert min(normals) == num(F["e4m3_min_normal"])
    assert not np.isinf(vals).any()
    # independent: torch's float8_e4m3fn
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(vals))
    assert np.array_equal(ref[~np.isnan(ref)], vals[~np.isnan(vals)])
    assert pos.min() == 2.0 ** -9


def test_e5m2_limits(orc):
    vals = np.array([orc.e5m2_decode(c) for c in range(256)])
    fin = vals[np.isfinite(vals)]
    assert fin.max() == num(F["e5m2_max"])
    assert orc.e5m2_decode(0b00000100) == num(F["e5m2_min_normal"])
    assert np.isinf(vals).sum() == 2 and np.isnan(vals).sum() == 6
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(vals))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], vals[ok])
