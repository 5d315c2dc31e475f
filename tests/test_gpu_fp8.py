"""GPU parity of the FP8 E4M3 variant of the W8A8 path against the oracle:
E4M3 weight and per-token activation codes and scales bit for bit (every
finite fp16 value through the encoder, ragged and wide rows, the smoothing
divide and multiply), the E4M3 GEMM within tolerance of the exact product
(fp32 sums in the matrix cores' order are not bit-reproducible), and the
full-size W8A8 workload through fp8_linear on sampled rows."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, sample_rows

pytestmark = pytest.mark.gpu


def test_every_fp16_value_encodes_like_the_oracle(orc):
    """One row holds every finite fp16 value of magnitude <= 448 and 448
    itself, so the row scale is 448 / 448 = 1 and each code is the encoding
    of the value; the other rows are the same values times 1/64 and x300
    (scaled rows: the quotients differ from the inputs)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = h[np.isfinite(h) & (np.abs(h.astype(np.float32)) <= 448)]
    K = (f.size + 7) // 8 * 8 + 8
    row = np.zeros(K, np.float16)
    row[: f.size] = f
    row[-1] = 448.0
    X = np.stack([row, (row.astype(np.float32) / 64).astype(np.float16),
                  np.clip(row.astype(np.float32) * 300, -65504, 65504).astype(np.float16)])
    for fn, ref in ((q4.fp8_quantize_act, orc.fp8_quantize_act),
                    (q4.fp8_quantize_weight, orc.fp8_quantize_weight)):
        q, sc = fn(gpu(X))
        q_ref, sc_ref = ref(X)
        assert np.array_equal(host(sc).view(np.uint32), sc_ref.view(np.uint32))
        bad = np.nonzero(host(q) != q_ref)
        assert bad[0].size == 0, (f"{bad[0].size} codes differ, first: row {bad[0][0]} "
                                  f"x={float(X[bad[0][0], bad[1][0]])} got {host(q)[bad][0]:#x} "
                                  f"want {q_ref[bad][0]:#x}")
    assert sc_ref[0] == 1.0


@pytest.mark.parametrize("rows,K", [(1, 8), (7, 64), (100, 1000), (33, 8200), (5, 16384), (64, 4096)])
@pytest.mark.parametrize("smooth", [False, True])
def test_row_quantizers(orc, rows, K, smooth):
    rng = np.random.default_rng(rows * 5 + K)
    X = rng.standard_normal((rows, K)).astype(np.float32)
    X[:, : max(1, K // 100)] *= 30
    if rows > 2:
        X[1] = 0
    X = X.astype(np.float16)
    W = (rng.standard_normal((rows, K)) * 0.02).astype(np.float16)
    s = rng.uniform(0.2, 8.0, K).astype(np.float32) if smooth else None
    sg = None if s is None else gpu(s)
    Xq, sx = q4.fp8_quantize_act(gpu(X), sg)
    Xq_ref, sx_ref = orc.fp8_quantize_act(X, s)
    assert np.array_equal(host(Xq), Xq_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))
    Wq, sw = q4.fp8_quantize_weight(gpu(W), sg)
    Wq_ref, sw_ref = orc.fp8_quantize_weight(W, s)
    assert np.array_equal(host(Wq), Wq_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))


def run_gemm(orc, M, N, K, seed, rows=None):
    W, X = workloads.small_case(seed, M, N, K)
    Xq, sx = orc.fp8_quantize_act(X)
    Wq, sw = orc.fp8_quantize_weight(W)
    Y = host(q4.fp8_gemm(gpu(Xq), gpu(sx), gpu(Wq), gpu(sw)))
    acc, aacc = orc.fp8_gemm(Xq, Wq, rows=rows)
    Yref, B = orc.fp8_reference(acc, aacc, sx, sw, rows=rows)
    return check_gemm(Y if rows is None else Y[rows], Yref, B, f"fp8 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (5, 7, 256), (64, 64, 128), (130, 257, 384),
                                   (300, 200, 8192), (513, 300, 256), (257, 511, 768),
                                   (256, 256, 1024)])
def test_gemm_shapes(orc, M, N, K):
    run_gemm(orc, M, N, K, M * 131 + N * 7 + K)


# Shapes that take the decode GEMV (M <= 16, K a multiple of 1024): each
# steps-per-wavefront variant (K = 1024 .. 8192), ragged N, rows past M;
# K = 3072 falls back to the GEMM.
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (5, 77, 2048), (16, 1000, 4096), (3, 64, 8192),
                                   (1, 11008, 4096), (7, 33, 3072)])
@pytest.mark.parametrize("xs0", ["0", "1"])
def test_gemv_shapes(orc, M, N, K, xs0, monkeypatch):
    """Both forms of the decode GEMV's X operand: staged per wavefront in LDS
    (M * K / 1024 <= 32) and loaded directly per lane (Q4_GEMV_XS0=1)."""
    monkeypatch.setenv("Q4_GEMV_XS0", xs0)
    run_gemm(orc, M, N, K, M * 29 + N + K)


def test_gemm_closed_form():
    K = 8192
    Xq = torch.full((3, K), 0x7E, dtype=torch.uint8, device="cuda")     # 448
    Wq = torch.full((5, K), 0xB0, dtype=torch.uint8, device="cuda")     # -0.5
    sx = torch.full((3,), 2.0 ** -12, dtype=torch.float32, device="cuda")
    sw = torch.ones(5, dtype=torch.float32, device="cuda")
    Y = q4.fp8_gemm(Xq, sx, Wq, sw)
    assert torch.all(Y == -448.0 * 0.5 * K * 2.0 ** -12)   # every partial sum exact in fp32


def test_fp8_linear_workload(orc):
    """The W8A8 workload (M = 2048, K = N = 8192, SmoothQuant s at alpha = 0.5)
    through the E4M3 path; codes bit for bit, the GEMM on sampled rows."""
    w = workloads.w8a8()
    s_ref = orc.smooth_scales(w["Xcal"], w["W"], 0.5)
    s = gpu(s_ref)
    Wq_ref, sw_ref = orc.fp8_quantize_weight(w["W"], s_ref)
    Wq, sw = q4.fp8_quantize_weight(gpu(w["W"]), s)
    assert np.array_equal(host(Wq), Wq_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    M, K = w["X"].shape
    ws = q4.w8a8_workspace(M, K, "cuda")
    Y = host(q4.fp8_linear(gpu(w["X"]), Wq, sw, s, workspace=ws))
    Xq_ref, sx_ref = orc.fp8_quantize_act(w["X"], s_ref)
    wsh = host(ws)
    assert np.array_equal(wsh[: M * K].reshape(M, K), Xq_ref)
    off = (M * K + 255) // 256 * 256
    assert np.array_equal(wsh[off: off + 4 * M].view(np.uint32), sx_ref.view(np.uint32))
    rows = sample_rows(M)
    acc, aacc = orc.fp8_gemm(Xq_ref, Wq_ref, rows=rows)
    Yref, B = orc.fp8_reference(acc, aacc, sx_ref, sw_ref, rows=rows)
    check_gemm(Y[rows], Yref, B, "fp8 workload")


def test_errors_and_empty():
    Xq = torch.zeros((4, 200), dtype=torch.uint8, device="cuda")
    one = torch.ones(4, dtype=torch.float32, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.fp8_gemm(Xq, one, Xq, one)
    assert e.value.status == q4.Q4_ERR_UNSUPPORTED
    big = torch.zeros((2, 8320), dtype=torch.uint8, device="cuda")
    two = torch.ones(2, dtype=torch.float32, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.fp8_gemm(big, two, big, two)
    assert e.value.status == q4.Q4_ERR_INVALID_ARG
    Y = q4.fp8_gemm(Xq[:0, :128], one[:0], Xq[:, :128].contiguous(), one)
    assert Y.shape == (0, 4)
