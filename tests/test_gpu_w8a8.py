"""GPU parity of the W8A8 path against the oracle: INT8 weight and per-token
activation codes and scales bit for bit, the SmoothQuant factor bit for bit
at alpha = 0.5, int32 accumulators bit for bit, fp16 outputs bit for bit with
the oracle's fp32 epilogue expression and within tolerance of the exact
product; full-size W8A8 workload (GEMM checked on sampled rows)."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, out_buffer, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 8), (7, 64), (100, 1000), (33, 8200), (5, 16384), (64, 4096)])
@pytest.mark.parametrize("smooth", [False, True])
def test_q8_weight(orc, N, K, smooth):
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = rng.uniform(0.2, 5.0, K).astype(np.float32) if smooth else None
    Wq_ref, sw_ref = orc.q8_quantize_weight(W, s)
    Wq, sw = q4.q8_quantize_weight(gpu(W), None if s is None else gpu(s))
    assert np.array_equal(host(Wq), Wq_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 8), (3, 64), (100, 1000), (33, 8200), (2, 16384), (64, 4096)])
@pytest.mark.parametrize("smooth", [False, True])
def test_q8_act(orc, M, K, smooth):
    rng = np.random.default_rng(M * 3 + K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, : max(1, K // 100)] *= 30
    if M > 2:
        X[1] = 0
    X = X.astype(np.float16)
    s = rng.uniform(0.2, 8.0, K).astype(np.float32) if smooth else None
    Xq_ref, sx_ref = orc.q8_quantize_act(X, s)
    Xq, sx = q4.q8_quantize_act(gpu(X), None if s is None else gpu(s))
    assert np.array_equal(host(Xq), Xq_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))


@pytest.mark.parametrize("alpha", [0.5, 0.25, 1.0, 0.0])
def test_smoothquant_scales_small(orc, alpha):
    rng = np.random.default_rng(7)
    X = rng.standard_normal((300, 520)).astype(np.float32)
    X[:, 3] *= 30
    X[:, 10] = 0
    W = (rng.standard_normal((77, 520)) * 0.02).astype(np.float32)
    W[:, 11] = 0
    X, W = X.astype(np.float16), W.astype(np.float16)
    s_ref = orc.smooth_scales(X, W, alpha)
    s = host(q4.smoothquant_scales(gpu(X), gpu(W), alpha))
    if alpha == 0.5:
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    else:
        assert np.allclose(s, s_ref, rtol=8 * 2.0 ** -23, atol=0)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (5, 7, 48), (64, 64, 128), (130, 257, 272),
                                   (128, 128, 1024), (300, 200, 8192), (513, 300, 256),
                                   (257, 511, 768), (300, 520, 384), (70, 260, 640)])
def test_gemm_shapes(orc, M, N, K):
    W, X = workloads.small_case(M * 131 + N * 7 + K, M, N, K)
    Xq, sx = orc.q8_quantize_act(X)
    Wq, sw = orc.q8_quantize_weight(W)
    acc = out_buffer((M, N), torch.int32)
    Y = host(q4.w8a8_gemm(gpu(Xq), gpu(sx), gpu(Wq), gpu(sw), acc_out=acc))
    acc_ref, aacc, ovf = orc.int8_gemm(Xq, Wq)
    assert ovf == 0
    assert np.array_equal(host(acc).astype(np.int64), acc_ref)
    Yref, B, y16 = orc.w8a8_epilogue(acc_ref, aacc, sx, sw)
    assert np.array_equal(Y.view(np.uint16), y16)
    check_gemm(Y, Yref, B, f"w8a8 M={M} N={N} K={K}")


# M <= 16 with K a multiple of 1024 up to 8192: the decode GEMV (16 weight
# rows per block, K split over 8 wavefronts); K = 3072 takes the GEMMs
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (5, 77, 2048), (16, 1000, 4096),
                                   (3, 64, 8192), (1, 11008, 4096), (7, 33, 3072),
                                   (16, 17, 1024)])
@pytest.mark.parametrize("xs0", ["0", "1"])
def test_gemv_shapes(orc, M, N, K, xs0, monkeypatch):
    """Both forms of the decode GEMV's X operand: staged per wavefront in LDS
    (M * K / 1024 <= 32) and loaded directly per lane (Q4_GEMV_XS0=1)."""
    monkeypatch.setenv("Q4_GEMV_XS0", xs0)
    test_gemm_shapes(orc, M, N, K)


def test_closed_form_accumulator():
    K = 8192
    Xq = torch.full((3, K), 127, dtype=torch.int8, device="cuda")
    Wq = torch.full((5, K), -127, dtype=torch.int8, device="cuda")
    one = torch.ones(3, dtype=torch.float32, device="cuda")
    acc = out_buffer((3, 5), torch.int32)
    q4.w8a8_gemm(Xq, one, Wq, torch.ones(5, dtype=torch.float32, device="cuda"), acc_out=acc)
    assert torch.all(acc == -16129 * K)


def test_w8a8_workload(orc):
    w = workloads.w8a8()
    s_ref = orc.smooth_scales(w["Xcal"], w["W"], 0.5)
    s = q4.smoothquant_scales(gpu(w["Xcal"]), gpu(w["W"]), 0.5)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    Wq_ref, sw_ref = orc.q8_quantize_weight(w["W"], s_ref)
    Wq, sw = q4.q8_quantize_weight(gpu(w["W"]), s)
    assert np.array_equal(host(Wq), Wq_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    M, K = w["X"].shape
    N = w["W"].shape[0]
    ws = q4.w8a8_workspace(M, K, "cuda")
    acc = out_buffer((M, N), torch.int32)
    Y = host(q4.w8a8_linear(gpu(w["X"]), Wq, sw, s, workspace=ws, acc_out=acc))
    # the workspace holds the per-token codes and scales: bit for bit
    Xq_ref, sx_ref = orc.q8_quantize_act(w["X"], s_ref)
    wsh = host(ws)
    assert np.array_equal(wsh[: M * K].view(np.int8).reshape(M, K), Xq_ref)
    off = (M * K + 255) // 256 * 256
    assert np.array_equal(wsh[off: off + 4 * M].view(np.uint32), sx_ref.view(np.uint32))
    rows = sample_rows(M)
    acc_ref, aacc, ovf = orc.int8_gemm(Xq_ref, Wq_ref, rows=rows)
    assert ovf == 0
    assert np.array_equal(host(acc)[rows].astype(np.int64), acc_ref)
    Yref, B, y16 = orc.w8a8_epilogue(acc_ref, aacc, sx_ref, sw_ref, rows=rows)
    assert np.array_equal(Y[rows].view(np.uint16), y16)
    check_gemm(Y[rows], Yref, B, "w8a8 workload")


def test_errors():
    Xq = torch.zeros((4, 100), dtype=torch.int8, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.w8a8_gemm(Xq, torch.ones(4, device="cuda"), torch.zeros((4, 100), dtype=torch.int8, device="cuda"),
                     torch.ones(4, device="cuda"))
    assert e.value.status == q4.Q4_ERR_INVALID_ARG
    X = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.w8a8_linear(X, torch.zeros((4, 128), dtype=torch.int8, device="cuda"),
                       torch.ones(4, device="cuda"),
                       workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == q4.Q4_ERR_INVALID_ARG


def test_linear_checks_gemm_preconditions_before_launching():
    """A misaligned Wq is an error of the GEMM step; w8a8_linear must report
    it before its activation quantizer runs, so the workspace stays as it
    was."""
    M, N, K = 4, 8, 128
    X = torch.ones((M, K), dtype=torch.float16, device="cuda")
    Wbuf = torch.zeros(N * K + 16, dtype=torch.int8, device="cuda")
    Wq_mis = Wbuf[1: 1 + N * K].view(N, K)
    ws = torch.full((q4.w8a8_workspace_bytes(M, K),), 0x5A, dtype=torch.uint8, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.w8a8_linear(X, Wq_mis, torch.ones(N, device="cuda"), workspace=ws)
    assert e.value.status == q4.Q4_ERR_MISALIGNED
    torch.cuda.synchronize()
    assert bool((ws == 0x5A).all()), "the activation quantizer ran before the GEMM's checks"
