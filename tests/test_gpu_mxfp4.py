"""GPU parity of the MXFP4 weight path (W4A8: E2M1 weights with an E8M0
scale per block of 32, per-token E4M3 activations) against the oracle:
codes and block scales bit for bit (every finite fp16 value of magnitude
<= 6 through the encoder at scale 1, scaled rows, zero blocks, the smoothing
multiply), the W4A8 GEMM on the scaled matrix cores within tolerance of the
exact product, and the W8A8 workload's layer through mxfp4_linear on
sampled rows."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, sample_rows

pytestmark = pytest.mark.gpu


def compare_quant(orc, W, s=None):
    codes, sc = q4.mxfp4_quantize_weight(gpu(W), None if s is None else gpu(s))
    codes_ref, sc_ref = orc.mxfp4_quantize_weight(W, s)
    assert np.array_equal(host(sc), sc_ref)
    bad = np.nonzero(host(codes) != codes_ref)
    assert bad[0].size == 0, f"{bad[0].size} code bytes differ, first at {bad[0][0]}, {bad[1][0]}"
    return codes_ref, sc_ref


def test_every_small_fp16_value(orc):
    """Blocks of 32 led by 6.0 (so each block's scale is 2^0 and each code is
    the encoding of the value itself), filled with every finite fp16 value of
    magnitude <= 6; the same rows times 2^-10 and x 40 change the scales."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = h[np.isfinite(h) & (np.abs(h.astype(np.float32)) <= 6)]
    nblk = (f.size + 30) // 31
    vals = np.zeros(nblk * 31, np.float16)
    vals[: f.size] = f
    blocks = np.concatenate([np.full((nblk, 1), 6.0, np.float16), vals.reshape(nblk, 31)], axis=1)
    K = 1024
    row = np.zeros(((blocks.size + K - 1) // K) * K, np.float16)
    row[: blocks.size] = blocks.reshape(-1)
    W = row.reshape(-1, K)
    codes, sc = compare_quant(orc, W)
    assert np.all(sc.reshape(-1)[: nblk] == 127)
    compare_quant(orc, (W.astype(np.float32) * 2.0 ** -10).astype(np.float16))
    compare_quant(orc, np.clip(W.astype(np.float32) * 40, -65504, 65504).astype(np.float16))


@pytest.mark.parametrize("N,K", [(1, 32), (7, 64), (100, 1024), (33, 8224), (64, 4096)])
@pytest.mark.parametrize("smooth", [False, True])
def test_quantizer_shapes(orc, N, K, smooth):
    rng = np.random.default_rng(N * 3 + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0, :32] = 0                                       # an all-zero block
    if N > 2:
        W[1, 32:64] = -0.75                             # amax exactly 6 * 2^-3
        W[2, :] *= 1000
    W = W.astype(np.float16)
    s = rng.uniform(0.2, 5.0, K).astype(np.float32) if smooth else None
    compare_quant(orc, W, s)


def run_gemm(orc, M, N, K, seed, rows=None):
    W, X = workloads.small_case(seed, M, N, K)
    Xq, sx = orc.fp8_quantize_act(X)
    codes, sc = orc.mxfp4_quantize_weight(W)
    Y = host(q4.mxfp4_gemm(gpu(Xq), gpu(sx), gpu(codes), gpu(sc)))
    acc, aacc = orc.mxfp4_gemm(Xq, codes, sc, rows=rows)
    Yref, B = orc.mxfp4_reference(acc, aacc, sx, rows=rows)
    return check_gemm(Y if rows is None else Y[rows], Yref, B, f"mxfp4 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (5, 7, 256), (64, 64, 128), (130, 257, 384),
                                   (300, 200, 8192), (513, 300, 256), (257, 511, 768),
                                   (256, 256, 1024)])
def test_gemm_shapes(orc, M, N, K):
    run_gemm(orc, M, N, K, M * 137 + N * 11 + K)


# More than 256 output tiles with a remainder: the whole rounds run as full
# 256 x 256 tiles and the remaining tiles as two 128-row halves each (the
# prefill shape's 344 tiles; 264 tiles with the per-step scale route, K % 512
# != 0; M = 1900, where the last row tile is partial and its upper half lies
# wholly past M). Sampled rows include every tile edge.
@pytest.mark.parametrize("M,N,K", [(2048, 11008, 4096), (2048, 8448, 384), (1900, 8448, 512)])
def test_gemm_tail_tiles(orc, M, N, K):
    run_gemm(orc, M, N, K, M + N + K, rows=sample_rows(M))


# Shapes that take the decode GEMVs (K a multiple of 1024): 16 weight rows per
# block for M <= 16 (X staged in LDS up to 32 KB, else in registers), 32 rows
# for 16 < M <= 32; each steps-per-wavefront variant (K = 1024 .. 8192),
# ragged N, rows past M; K = 3072 falls back to the GEMM.
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (5, 77, 2048), (17, 1000, 4096), (32, 64, 8192),
                                   (1, 11008, 4096), (3, 4096, 4096), (31, 33, 3072),
                                   (16, 100, 4096), (9, 50, 8192), (20, 70, 2048)])
def test_gemv_shapes(orc, M, N, K):
    run_gemm(orc, M, N, K, M * 31 + N + K)


@pytest.mark.parametrize("M,K", [(64, 256), (3, 1024), (24, 1024)])   # GEMM, 16- and 32-row GEMVs
def test_gemm_block_scales_and_nibbles(orc, M, K):
    """Each 32-block of every weight row gets its own scale and only one
    nonzero code, at a position that moves with the block: a wrong scale
    lane, block or nibble order changes the sum."""
    N = 64
    rng = np.random.default_rng(40)
    Xq = rng.integers(0x30, 0x48, (M, K)).astype(np.uint8)      # E4M3 values around 0.5 .. 4
    sx = np.full(M, 1.0, np.float32)
    codes = np.zeros((N, K // 2), np.uint8)
    sc = rng.integers(120, 134, (N, K // 32)).astype(np.uint8)
    for n in range(N):
        for b in range(K // 32):
            k = b * 32 + (n + 5 * b) % 32
            codes[n, k // 2] |= np.uint8((2 + (n + b) % 6) << (4 * (k & 1)))
    Y = host(q4.mxfp4_gemm(gpu(Xq), gpu(sx), gpu(codes), gpu(sc)))
    acc, aacc = orc.mxfp4_gemm(Xq, codes, sc)
    Yref, B = orc.mxfp4_reference(acc, aacc, sx)
    check_gemm(Y, Yref, B, "mxfp4 block scales")


def test_mxfp4_linear_workload(orc):
    """The W8A8 workload's layer (M = 2048, K = N = 8192, SmoothQuant s at
    alpha = 0.5) with MXFP4 weights and E4M3 activations."""
    w = workloads.w8a8()
    s_ref = orc.smooth_scales(w["Xcal"], w["W"], 0.5)
    s = gpu(s_ref)
    codes_ref, sc_ref = orc.mxfp4_quantize_weight(w["W"], s_ref)
    codes, sc = q4.mxfp4_quantize_weight(gpu(w["W"]), s)
    assert np.array_equal(host(codes), codes_ref) and np.array_equal(host(sc), sc_ref)
    M, K = w["X"].shape
    ws = q4.w8a8_workspace(M, K, "cuda")
    Y = host(q4.mxfp4_linear(gpu(w["X"]), codes, sc, s, workspace=ws))
    Xq_ref, sx_ref = orc.fp8_quantize_act(w["X"], s_ref)
    assert np.array_equal(host(ws)[: M * K].reshape(M, K), Xq_ref)
    rows = sample_rows(M)
    acc, aacc = orc.mxfp4_gemm(Xq_ref, codes_ref, sc_ref, rows=rows)
    Yref, B = orc.mxfp4_reference(acc, aacc, sx_ref, rows=rows)
    check_gemm(Y[rows], Yref, B, "mxfp4 workload")


def test_errors():
    Xq = torch.zeros((4, 192), dtype=torch.uint8, device="cuda")
    one = torch.ones(4, dtype=torch.float32, device="cuda")
    codes = torch.zeros((4, 96), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((4, 6), dtype=torch.uint8, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.mxfp4_gemm(Xq, one, codes, sc)
    assert e.value.status == q4.Q4_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        q4.mxfp4_gemm(Xq[:, :128].contiguous(), one, codes, sc)
