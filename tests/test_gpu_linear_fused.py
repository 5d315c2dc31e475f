"""The decode-sized W8A8, E4M3 and MXFP4 layers whose per-token quantizer runs
inside the GEMV (one launch; M * K <= 16384): the codes and scales the call
leaves in the workspace are bit for bit the oracle's per-token quantizer
(Quantization operators guide §5.2: X / s, then per-token INT8 or E4M3),
the INT8 path's int32 sums are bit for bit the oracle's exact sums, and the
fp16 outputs are bit for bit those of the two-launch form (the standalone
quantizer, then the GEMM) and within tolerance of the exact product."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, out_buffer

pytestmark = pytest.mark.gpu

# (M, N, K): every K the fused kernel takes (1024 .. 8192), one row up to the
# M * K = 16384 limit, a ragged N; (5, 300, 4096) is past the limit (two launches)
SHAPES = [(1, 300, 1024), (1, 11008, 4096), (4, 1000, 4096), (2, 77, 8192), (16, 100, 1024),
          (3, 33, 2048), (1, 129, 8192), (5, 300, 4096)]


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, : max(1, K // 100)] *= 30
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    Xcal = rng.standard_normal((64, K)).astype(np.float16)
    return X, W, Xcal


def _workspace_rows(ws, M, K):
    h = host(ws)
    off = (M * K + 255) // 256 * 256
    return h[: M * K].reshape(M, K), h[off: off + 4 * M].view(np.uint32)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("smooth", [True, False])
def test_w8a8_linear_decode(orc, M, N, K, smooth):
    X, W, Xcal = _inputs(M, N, K, M * 31 + N + K + int(smooth))
    s_ref = orc.smooth_scales(Xcal, W, 0.5) if smooth else None
    s = None if s_ref is None else gpu(s_ref)
    Wq_ref, sw_ref = orc.q8_quantize_weight(W, s_ref)
    Wq, sw = gpu(Wq_ref), gpu(sw_ref)
    ws = q4.w8a8_workspace(M, K, "cuda")
    acc = out_buffer((M, N), torch.int32)
    Y = host(q4.w8a8_linear(gpu(X), Wq, sw, s, workspace=ws, acc_out=acc))
    Xq_ref, sx_ref = orc.q8_quantize_act(X, s_ref)
    codes, scales = _workspace_rows(ws, M, K)
    assert np.array_equal(codes.view(np.int8), Xq_ref), "per-token codes differ from the oracle"
    assert np.array_equal(scales, sx_ref.view(np.uint32)), "per-token scales differ from the oracle"
    acc_ref, aacc, ovf = orc.int8_gemm(Xq_ref, Wq_ref)
    assert ovf == 0
    assert np.array_equal(host(acc).astype(np.int64), acc_ref), "int32 sums differ"
    Yref, B, y16 = orc.w8a8_epilogue(acc_ref, aacc, sx_ref, sw_ref)
    assert np.array_equal(Y.view(np.uint16), y16), "fp16 outputs differ from the oracle's epilogue"
    check_gemm(Y, Yref, B, f"w8a8 decode M={M} N={N} K={K}")
    # the two-launch form gives the same bits
    Xq2, sx2 = q4.q8_quantize_act(gpu(X), s)
    Y2 = host(q4.w8a8_gemm(Xq2, sx2, Wq, sw))
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("smooth", [True, False])
def test_fp8_linear_decode(orc, M, N, K, smooth):
    X, W, Xcal = _inputs(M, N, K, M * 37 + N + K + int(smooth))
    s_ref = orc.smooth_scales(Xcal, W, 0.5) if smooth else None
    s = None if s_ref is None else gpu(s_ref)
    Wq_ref, sw_ref = orc.fp8_quantize_weight(W, s_ref)
    Wq, sw = gpu(Wq_ref), gpu(sw_ref)
    ws = q4.w8a8_workspace(M, K, "cuda")
    Y = host(q4.fp8_linear(gpu(X), Wq, sw, s, workspace=ws))
    Xq_ref, sx_ref = orc.fp8_quantize_act(X, s_ref)
    codes, scales = _workspace_rows(ws, M, K)
    assert np.array_equal(codes, Xq_ref), "per-token E4M3 codes differ from the oracle"
    assert np.array_equal(scales, sx_ref.view(np.uint32)), "per-token scales differ from the oracle"
    acc, aacc = orc.fp8_gemm(Xq_ref, Wq_ref)
    Yref, B = orc.fp8_reference(acc, aacc, sx_ref, sw_ref)
    check_gemm(Y, Yref, B, f"fp8 decode M={M} N={N} K={K}")
    Xq2, sx2 = q4.fp8_quantize_act(gpu(X), s)
    Y2 = host(q4.fp8_gemm(Xq2, sx2, Wq, sw))
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))


def test_noalloc_decode_uses_the_fused_kernel(orc):
    M, N, K = 1, 500, 4096
    X, W, Xcal = _inputs(M, N, K, 99)
    s_ref = orc.smooth_scales(Xcal, W, 0.5)
    Wq_ref, sw_ref = orc.q8_quantize_weight(W, s_ref)
    Wq, sw, s = gpu(Wq_ref), gpu(sw_ref), gpu(s_ref)
    acc = out_buffer((M, N), torch.int32)
    Y = host(q4.w8a8_linear_noalloc(gpu(X), Wq, sw, s, acc_out=acc))
    Xq_ref, sx_ref = orc.q8_quantize_act(X, s_ref)
    acc_ref, aacc, _ = orc.int8_gemm(Xq_ref, Wq_ref)
    assert np.array_equal(host(acc).astype(np.int64), acc_ref)
    _, _, y16 = orc.w8a8_epilogue(acc_ref, aacc, sx_ref, sw_ref)
    assert np.array_equal(Y.view(np.uint16), y16)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("smooth", [True, False])
def test_mxfp4_linear_decode(orc, M, N, K, smooth):
    """MXFP4 weights with the per-token E4M3 quantizer fused into the decode GEMV."""
    X, W, Xcal = _inputs(M, N, K, M * 41 + N + K + int(smooth))
    s_ref = orc.smooth_scales(Xcal, W, 0.5) if smooth else None
    s = None if s_ref is None else gpu(s_ref)
    codes_ref, sc_ref = orc.mxfp4_quantize_weight(W, s_ref)
    codes, sc = gpu(codes_ref), gpu(sc_ref)
    ws = q4.w8a8_workspace(M, K, "cuda")
    Y = host(q4.mxfp4_linear(gpu(X), codes, sc, s, workspace=ws))
    Xq_ref, sx_ref = orc.fp8_quantize_act(X, s_ref)
    xcodes, xscales = _workspace_rows(ws, M, K)
    assert np.array_equal(xcodes, Xq_ref), "per-token E4M3 codes differ from the oracle"
    assert np.array_equal(xscales, sx_ref.view(np.uint32)), "per-token scales differ from the oracle"
    acc, aacc = orc.mxfp4_gemm(Xq_ref, codes_ref, sc_ref)
    Yref, B = orc.mxfp4_reference(acc, aacc, sx_ref)
    check_gemm(Y, Yref, B, f"mxfp4 decode M={M} N={N} K={K}")
    Xq2, sx2 = q4.fp8_quantize_act(gpu(X), s)
    Y2 = host(q4.mxfp4_gemm(Xq2, sx2, codes, sc))
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))
