"""GPU parity of the flagged-group rule for non-finite inputs: every
quantizer gives a group that holds a NaN or an infinity the format's NaN
scale and zero codes, bit for bit with the oracle (NaN bit patterns
included), and the layers carry NaN into exactly the outputs that use a
flagged group while every other output stays within tolerance."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, flagged_mask, gpu, host, poisoned

pytestmark = pytest.mark.gpu


def same_bits(a, b, what):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.dtype.itemsize == b.dtype.itemsize
    ua = a.view(np.uint8).reshape(a.shape[0], -1)
    ub = b.view(np.uint8).reshape(b.shape[0], -1)
    bad = np.nonzero(ua != ub)
    assert bad[0].size == 0, f"{what}: {bad[0].size} bytes differ, first at {bad[0][0]}, {bad[1][0]}"


@pytest.mark.parametrize("g,sym", [(128, False), (128, True), (32, False), (64, True), (64, False)])
def test_int4_quantizer(orc, g, sym):
    W, _ = workloads.small_case(21, 1, 40, 1024)
    Wp, _, _ = poisoned(W, g + sym, count=9)
    c, s, z = q4.q4_quantize_pack(gpu(Wp), g=g, sym=sym)
    c0, s0, z0 = orc.q4_quantize_pack(Wp, g=g, sym=sym)
    same_bits(host(s), s0, "scales")
    same_bits(host(c), c0, "codes")
    if not sym:
        same_bits(host(z), z0, "zeros")


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("K", [1024, 8192, 8320])
@pytest.mark.parametrize("smooth", [False, True])
def test_row_quantizers(orc, fmt, K, smooth):
    W, X = workloads.small_case(22, 37, 33, K)
    s = (np.abs(np.random.default_rng(K).standard_normal(K)) + 0.5).astype(np.float32) if smooth else None
    pairs = [(q4.q8_quantize_weight, orc.q8_quantize_weight), (q4.q8_quantize_act, orc.q8_quantize_act)]
    if fmt == "fp8":
        pairs = [(q4.fp8_quantize_weight, orc.fp8_quantize_weight), (q4.fp8_quantize_act, orc.fp8_quantize_act)]
    for (dev_q, orc_q), A in zip(pairs, (W, X)):
        Ap, cells, _ = poisoned(A, K + smooth, count=5)
        q, sc = dev_q(gpu(Ap), None if s is None else gpu(s))
        q0, sc0 = orc_q(Ap, s)
        same_bits(host(sc)[:, None], sc0[:, None], "scales")
        same_bits(host(q), q0, "codes")
        assert np.isnan(sc0).sum() == len({r for r, _ in cells})


def test_zero_smoothing_factor_flags_every_row(orc):
    _, X = workloads.small_case(23, 9, 1, 2048)
    s = np.ones(2048, np.float32)
    s[100] = 0
    for dev_q, orc_q in ((q4.q8_quantize_act, orc.q8_quantize_act), (q4.fp8_quantize_act, orc.fp8_quantize_act)):
        q, sc = dev_q(gpu(X), gpu(s))
        q0, sc0 = orc_q(X, s)
        same_bits(host(sc)[:, None], sc0[:, None], "scales")
        assert np.isnan(host(sc)).all() and not host(q).any()


@pytest.mark.parametrize("fmt", ["mxfp4", "nf4", "nvfp4"])
def test_block_quantizers(orc, fmt):
    W, _ = workloads.small_case(24, 1, 48, 2048)
    Wp, _, _ = poisoned(W, 7, count=11)
    if fmt == "mxfp4":
        c, sc = q4.mxfp4_quantize_weight(gpu(Wp))
        c0, sc0 = orc.mxfp4_quantize_weight(Wp)
    elif fmt == "nf4":
        c, sc = q4.nf4_quantize(gpu(Wp))
        c0, sc0 = orc.nf4_quantize(Wp)
    else:
        c, sc = q4.nvfp4_quantize(gpu(Wp))
        c0, sc0 = orc.nvfp4_quantize(Wp)
    same_bits(host(sc), sc0, "scales")
    same_bits(host(c), c0, "codes")


def nan_columns_exactly(Y, Yref, B, bad_cols, what):
    assert np.isnan(Y[:, bad_cols]).all(), f"{what}: a flagged column is not NaN"
    good = ~bad_cols
    check_gemm(Y[:, good], Yref[:, good], B[:, good], what)


@pytest.mark.parametrize("M", [1, 5, 40, 300])
def test_w4a16_layer_carries_nan(orc, M):
    W, X = workloads.small_case(25, M, 300, 1024)
    Wp, cells, _ = poisoned(W, M, count=4)
    c, s, z = orc.q4_quantize_pack(Wp, g=128)
    Y = host(q4.w4a16_linear(gpu(X), gpu(c), gpu(s), gpu(z), g=128))
    Yref, B = orc.w4a16_ref(X, c, s, z, g=128)
    bad_cols = flagged_mask(cells, W.shape, 1024)[:, 0]
    nan_columns_exactly(Y, Yref, B, bad_cols, f"w4a16 M={M}")


@pytest.mark.parametrize("fmt", ["nf4", "nvfp4"])
@pytest.mark.parametrize("M", [1, 100])
def test_lookup_layers_carry_nan(orc, fmt, M):
    W, X = workloads.small_case(26, M, 200, 1024)
    Wp, cells, _ = poisoned(W, M + 1, count=3)
    quant, lin, ref = ((orc.nf4_quantize, q4.nf4_linear, orc.nf4_ref) if fmt == "nf4"
                       else (orc.nvfp4_quantize, q4.nvfp4_linear, orc.nvfp4_ref))
    c, s = quant(Wp)
    Y = host(lin(gpu(X), gpu(c), gpu(s)))
    Yref, B = ref(X, c, s)
    bad_cols = flagged_mask(cells, W.shape, 1024)[:, 0]
    nan_columns_exactly(Y, Yref, B, bad_cols, f"{fmt} M={M}")


@pytest.mark.parametrize("M", [1, 3, 300])
def test_w8a8_layer_carries_nan(orc, M):
    """A poisoned activation row: its per-token scale is NaN and its row of Y
    is NaN (the decode sizes quantize X inside the GEMV, larger M in a pass of
    its own); the other rows match the oracle."""
    W, X = workloads.small_case(27, M, 256, 1024)
    Xp = X.copy()
    Xp[M // 2, 17] = np.float16(np.nan)
    Wq, sw = orc.q8_quantize_weight(W)
    Y = host(q4.w8a8_linear(gpu(Xp), gpu(Wq), gpu(sw)))
    Xq, sx = orc.q8_quantize_act(Xp)
    acc, aacc, _ = orc.int8_gemm(Xq, Wq)
    Yref, B, _ = orc.w8a8_epilogue(acc, aacc, sx, sw)
    assert np.isnan(Y[M // 2]).all()
    good = np.ones(M, bool)
    good[M // 2] = False
    if good.any():
        check_gemm(Y[good], Yref[good], B[good], f"w8a8 M={M}")
