"""GPU parity of the AWQ-style scaling on the W4A16 path against the oracle:
the scaled weights and activations bit for bit (every finite fp16 value
against several factors, random data, in place), and w4a16_linear_awq within
tolerance of the exact product over x'' = f2h(x / s) and the dequantized
INT4 weight of w'' = f2h(w * s): the fused decode GEMV (one token: every
launch variant, the decode workload's layers) and the scaled-copy path for
more tokens (batched and prefill kernels), one-hot inputs that pin the
fused path's column indexing bit for bit."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host

pytestmark = pytest.mark.gpu


def factors(K, seed):
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(-1.5, 1.5, K)).astype(np.float32)


@pytest.mark.parametrize("s", [0.3, 1.7, 3.0, 1.0 / 3.0, 1e-3, 700.0])
def test_scaling_every_fp16_value(orc, s):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    K = 1024
    A = np.zeros(((h.size + K - 1) // K) * K, np.float16)
    A[: h.size] = h
    A = A.reshape(-1, K)
    sv = np.full(K, s, np.float32)
    sv[1::3] = np.float32(s * 1.37)
    for fn, ref in ((q4.awq_scale_weight, orc.awq_scale_weight), (q4.awq_scale_act, orc.awq_scale_act)):
        got = host(fn(gpu(A), gpu(sv))).view(np.uint16)
        want = ref(A, sv)
        bad = np.nonzero(got != want)
        assert bad[0].size == 0, f"{fn.__name__} s={s}: {bad[0].size} values differ"


@pytest.mark.parametrize("rows,K", [(1, 8), (3, 136), (64, 4096), (257, 1000)])
def test_scaling_random_and_in_place(orc, rows, K):
    rng = np.random.default_rng(rows + K)
    A = (rng.standard_normal((rows, K)) * 3).astype(np.float16)
    s = factors(K, rows)
    want_w, want_x = orc.awq_scale_weight(A, s), orc.awq_scale_act(A, s)
    assert np.array_equal(host(q4.awq_scale_weight(gpu(A), gpu(s))).view(np.uint16), want_w)
    t = gpu(A)
    q4.awq_scale_act(t, gpu(s), out=t)
    assert np.array_equal(host(t).view(np.uint16), want_x)


def run_awq(orc, W, X, s, sym, what, g=128):
    Ws = orc.awq_scale_weight(W, s)
    codes, scales, zeros = orc.q4_quantize_pack(Ws, g=g, sym=sym)
    Y = host(q4.w4a16_linear_awq(gpu(X), gpu(codes), gpu(scales.view(np.float16)),
                                 None if zeros is None else gpu(zeros), gpu(s), g=g))
    Xs = orc.awq_scale_act(X, s)
    Yref, B = orc.w4a16_ref(Xs, codes, scales, zeros, g=g)
    check_gemm(Y, Yref, B, what)


# g = 64 and 32: the scaled copy in the workspace, then the small-group kernel
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (20, 130, 512), (300, 100, 512)])
@pytest.mark.parametrize("g", [32, 64])
def test_linear_awq_small_groups(orc, M, N, K, g):
    W, X = workloads.small_case(M * 3 + N + K + g, M, N, K)
    run_awq(orc, W, X, factors(K, M + N + g), False, f"awq g={g} M={M} N={N} K={K}", g=g)


# one token: the fused decode GEMV in each launch variant (16 / 8 / 4
# wavefronts per block), ragged N; more tokens: the scaled copy, then the
# GEMV (M <= 7 at K = 4096), batched (8 < M <= 64) or prefill kernels
@pytest.mark.parametrize("M,N,K", [(1, 1000, 4096), (1, 4096, 4096), (1, 11008, 4096),
                                   (1, 300, 1024), (1, 77, 8192), (3, 300, 4096),
                                   (16, 300, 4096), (33, 130, 2048), (64, 200, 4096),
                                   (300, 260, 1024)])
@pytest.mark.parametrize("sym", [False, True])
def test_linear_awq(orc, M, N, K, sym):
    W, X = workloads.small_case(M * 5 + N + K + int(sym), M, N, K)
    run_awq(orc, W, X, factors(K, M + N), sym, f"awq M={M} N={N} K={K} sym={sym}")


def test_linear_awq_one_hot_pins_columns(orc):
    """X = x e_k: Y[0, n] = f2h(fl32(x''_k * w_hat[n, k])) exactly (the one
    nonzero product, rounded to fp32 by the fp32 accumulation and then to
    fp16), for k across every wavefront's k-range."""
    N, K = 64, 4096
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = factors(K, 12)
    Ws = orc.awq_scale_weight(W, s)
    codes, scales, zeros = orc.q4_quantize_pack(Ws, g=128, sym=False)
    w_hat = orc.q4_dequant(codes, scales, zeros, K, 128)
    args = (gpu(codes), gpu(scales.view(np.float16)), gpu(zeros), gpu(s))
    for k in [0, 1, 7, 8, 127, 128, 511, 512, 1000, 2047, 2048, 3071, 4095]:
        X = np.zeros((1, K), np.float16)
        X[0, k] = np.float16(rng.uniform(0.5, 2.0))
        xs = orc.awq_scale_act(X, s).view(np.float16)[0, k]
        Y = host(q4.w4a16_linear_awq(gpu(X), *args))
        want = (np.float32(xs) * w_hat[:, k].astype(np.float32)).astype(np.float16)
        assert np.array_equal(Y[0].view(np.uint16), want.view(np.uint16)), k


def test_decode_workload_layers(orc):
    """The decode workload's layers with AWQ factors from the pages' search
    form: s = mean|x|^0.5 over a seeded calibration draw, normalised."""
    for N in (11008, 4096):
        w = workloads.decode(N)
        K = w["W"].shape[1]
        cal = workloads.normal_fp16(77, (64, K), 1.0, (w["outliers"], 10.0))
        act = np.abs(cal.astype(np.float64)).mean(axis=0) ** 0.5
        s = (act / act.mean()).astype(np.float32)
        Ws = q4.awq_scale_weight(gpu(w["W"]), gpu(s))
        packed = q4.q4_quantize_pack(Ws, g=128, sym=w["sym"])
        codes, scales, zeros = (None if t is None else host(t) for t in packed)
        assert np.array_equal(codes, orc.q4_quantize_pack(host(Ws), g=128, sym=w["sym"])[0])
        Y = host(q4.w4a16_linear_awq(gpu(w["X"]), *packed, gpu(s)))
        Yref, B = orc.w4a16_ref(orc.awq_scale_act(w["X"], s), codes, scales, zeros)
        check_gemm(Y, Yref, B, f"awq decode N={N}")


def test_errors():
    X = torch.zeros((2, 256), dtype=torch.float16, device="cuda")
    codes = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((8, 2), dtype=torch.float16, device="cuda")
    s = torch.ones(256, dtype=torch.float32, device="cuda")
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.w4a16_linear_awq(X, codes, scales, None, s, workspace=small)
    assert e.value.status == q4.Q4_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        q4.w4a16_linear_awq(X, codes, scales, None, s[:128])
