"""Pins of the oracle's rule for non-finite inputs (the failure-detection
reading: NaN and infinity propagate into the scale, which flags the group).
Every quantizer flags a group (INT4 group, INT8 / E4M3 row, MXFP4 block of
32, NF4 block of 64, NVFP4 block of 16) that holds a NaN or an infinity:
its scale is the format's NaN and its codes (and INT4 zero-point) are 0;
every other group is quantized exactly as in a copy of the input with the
poisoned cells set to 0, and the references carry NaN into exactly the
outputs that use a flagged group."""
import numpy as np
import pytest

import workloads
from parity import flagged_mask, poisoned

N, K = 24, 512


def nibbles(codes):
    u = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    return u


def expand(mask, group):
    return np.repeat(mask, group, axis=1)


@pytest.mark.parametrize("g,sym", [(128, False), (128, True), (32, False)])
def test_int4_groups(orc, g, sym):
    W, _ = workloads.small_case(11, 1, N, K)
    Wp, cells, clean = poisoned(W, g + sym)
    bad = flagged_mask(cells, W.shape, g)
    c, s, z = orc.q4_quantize_pack(Wp, g=g, sym=sym)
    c0, s0, z0 = orc.q4_quantize_pack(clean, g=g, sym=sym)
    assert np.all(s.view(np.uint16)[bad] == 0x7E00)
    assert np.array_equal(s.view(np.uint16)[~bad], s0.view(np.uint16)[~bad])
    u, u0 = nibbles(c), nibbles(c0)
    assert np.all(u[expand(bad, g)] == 0)
    assert np.array_equal(u[~expand(bad, g)], u0[~expand(bad, g)])
    if not sym:
        zn = nibbles(z)[:, : K // g]
        assert np.all(zn[bad] == 0) and np.array_equal(zn[~bad], nibbles(z0)[:, : K // g][~bad])
    # the reference: NaN in exactly the columns that use a flagged group
    X = np.ones((2, K), np.float16)
    Y, _ = orc.w4a16_ref(X, c, s, z, g=g)
    assert np.array_equal(np.isnan(Y).all(axis=0), bad.any(axis=1)) and not np.isnan(Y[:, ~bad.any(axis=1)]).any()


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_rows(orc, fmt):
    quant_w = orc.q8_quantize_weight if fmt == "int8" else orc.fp8_quantize_weight
    quant_a = orc.q8_quantize_act if fmt == "int8" else orc.fp8_quantize_act
    W, X = workloads.small_case(12, N, N, K)
    for quant, A in ((quant_w, W), (quant_a, X)):
        Ap, cells, clean = poisoned(A, 3)
        bad = flagged_mask(cells, A.shape, K)[:, 0]
        q, sc = quant(Ap)
        q0, sc0 = quant(clean)
        assert np.all(sc.view(np.uint32)[bad] == 0x7FC00000) and np.all(q[bad] == 0)
        assert np.array_equal(sc[~bad], sc0[~bad]) and np.array_equal(q[~bad], q0[~bad])
    # a zero smoothing factor makes x / s non-finite in every row
    s = np.ones(K, np.float32)
    s[7] = 0
    q, sc = quant_a(X, s)
    assert np.all(np.isnan(sc)) and not q.any()


def test_mxfp4_blocks(orc):
    W, _ = workloads.small_case(13, 1, N, K)
    Wp, cells, clean = poisoned(W, 4)
    bad = flagged_mask(cells, W.shape, 32)
    c, sc = orc.mxfp4_quantize_weight(Wp)
    c0, sc0 = orc.mxfp4_quantize_weight(clean)
    assert np.all(sc[bad] == 0xFF) and np.array_equal(sc[~bad], sc0[~bad])
    u, u0 = nibbles(c), nibbles(c0)
    assert np.all(u[expand(bad, 32)] == 0) and np.array_equal(u[~expand(bad, 32)], u0[~expand(bad, 32)])


@pytest.mark.parametrize("fmt,group,nan", [("nf4", 64, 0x7FC00000), ("nvfp4", 16, 0x7F)])
def test_lookup_formats(orc, fmt, group, nan):
    quant = orc.nf4_quantize if fmt == "nf4" else orc.nvfp4_quantize
    ref = orc.nf4_ref if fmt == "nf4" else orc.nvfp4_ref
    W, _ = workloads.small_case(14, 1, N, K)
    Wp, cells, clean = poisoned(W, 5)
    bad = flagged_mask(cells, W.shape, group)
    c, sc = quant(Wp)
    c0, sc0 = quant(clean)
    sb = sc.view(np.uint32) if fmt == "nf4" else sc
    assert np.all(sb[bad] == nan)
    assert np.array_equal(sc[~bad], sc0[~bad])
    u, u0 = nibbles(c), nibbles(c0)
    assert np.all(u[expand(bad, group)] == 0) and np.array_equal(u[~expand(bad, group)], u0[~expand(bad, group)])
    Y, _ = ref(np.ones((1, K), np.float16), c, sc)
    assert np.array_equal(np.isnan(Y[0]), bad.any(axis=1))
