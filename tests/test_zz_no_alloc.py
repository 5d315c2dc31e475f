"""The no-allocation W8A8 entry point through the C ABI: w8a8_linear_noalloc
against w8a8_linear with a caller workspace (the same kernels, so the fp16
outputs and the int32 accumulators agree bit for bit), on two calls in a row
whose second is smaller (the scratch array keeps the first call's contents),
then against the oracle; a request beyond the scratch array is refused
before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, out_buffer

pytestmark = pytest.mark.gpu


def _call_noalloc(X, Wq, sw, s, Y, acc):
    M, K = X.shape
    N = Wq.shape[0]
    st = q4.lib().w8a8_linear_noalloc(X.data_ptr(), M, N, K, Wq.data_ptr(), sw.data_ptr(),
                                      None if s is None else s.data_ptr(), Y.data_ptr(),
                                      None if acc is None else acc.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    return st


def _case(seed, M, N, K, smooth):
    W, X = workloads.small_case(seed, M, N, K)
    Xg, Wg = gpu(X), gpu(W)
    s = q4.smoothquant_scales(Xg, Wg) if smooth else None
    Wq, sw = q4.q8_quantize_weight(Wg, s)
    return Xg, Wq, sw, s


@pytest.mark.parametrize("smooth", [True, False])
def test_noalloc_matches_workspace_entry_point(orc, smooth):
    # first a large call (the W8A8 workload's M x K, the scratch array's
    # design size), then a smaller one with a ragged shape
    for seed, (M, N, K) in enumerate([(2048, 1024, 8192), (37, 300, 1040)]):
        Xg, Wq, sw, s = _case(seed + 10 * int(smooth), M, N, K, smooth)
        Y = out_buffer((M, N), torch.float16)
        acc = out_buffer((M, N), torch.int32)
        assert _call_noalloc(Xg, Wq, sw, s, Y, acc) == q4.Q4_OK, q4.lib().q4_last_error()
        ws = q4.w8a8_workspace(M, K, "cuda")
        acc_ws = out_buffer((M, N), torch.int32)
        Y_ws = q4.w8a8_linear(Xg, Wq, sw, s, workspace=ws, acc_out=acc_ws)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ws), f"int32 accumulators differ at M={M} N={N} K={K}"
        assert torch.equal(Y.view(torch.int16), Y_ws.view(torch.int16)), f"outputs differ at M={M}"
        # and against the oracle on a few rows
        rows = [0, M // 2, M - 1]
        Xh = host(Xg)
        s_h = None if s is None else host(s)
        Xq_ref, sx_ref = orc.q8_quantize_act(Xh, s_h)
        acc_ref, aacc, ovf = orc.int8_gemm(Xq_ref, host(Wq), rows=rows)
        assert ovf == 0
        assert np.array_equal(host(acc)[rows].astype(np.int64), acc_ref)
        Yref, B, y16 = orc.w8a8_epilogue(acc_ref, aacc, sx_ref, host(sw), rows=rows)
        assert np.array_equal(host(Y)[rows].view(np.uint16), y16)
        check_gemm(host(Y)[rows], Yref, B, f"noalloc M={M} N={N} K={K}")


def test_noalloc_refuses_too_large():
    limit = q4.w8a8_noalloc_max_bytes()
    assert limit == 16 * 1024 * 1024 + 64 * 1024
    K = 8192
    M = limit // K + 1          # M * K alone passes the limit
    assert q4.w8a8_workspace_bytes(M, K) > limit
    X = torch.empty((1, K), dtype=torch.float16, device="cuda")   # never read
    Wq = torch.zeros((16, K), dtype=torch.int8, device="cuda")
    sw = torch.ones(16, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, 16), dtype=torch.float16, device="cuda")
    st = q4.lib().w8a8_linear_noalloc(X.data_ptr(), M, 16, K, Wq.data_ptr(), sw.data_ptr(), None,
                                      Y.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert st == q4.Q4_ERR_UNSUPPORTED
    assert b"scratch" in q4.lib().q4_last_error()


def test_noalloc_binding_and_empty(orc):
    Xg, Wq, sw, s = _case(3, 5, 40, 256, True)
    Y = q4.w8a8_linear_noalloc(Xg, Wq, sw, s)
    Y_ws = q4.w8a8_linear(Xg, Wq, sw, s)
    assert torch.equal(Y.view(torch.int16), Y_ws.view(torch.int16))
    Ye = q4.w8a8_linear_noalloc(Xg[:0], Wq, sw, s)
    assert Ye.shape == (0, 40)
