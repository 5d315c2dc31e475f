"""GPU parity of the NVFP4 path against the oracle: codes and E4M3 block
scales bit for bit (every fp16 value in range at a unit, a non-power-of-two
and a subnormal scale, zero, saturating and random blocks), and the layer
within tolerance of the exact product over the dequantized weight: decode
passes of X, the large-M GEMM at each tile width, ragged shapes, one-hot
inputs that read the dequantized weight back exactly (it is exact in fp16),
the decode workload's layers and the prefill shape on sampled rows."""
import numpy as np
import pytest

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, sample_rows

pytestmark = pytest.mark.gpu


def compare_quant(orc, W):
    codes, sc = q4.nvfp4_quantize(gpu(W))
    codes_ref, sc_ref = orc.nvfp4_quantize(W)
    bad = np.nonzero(host(sc) != sc_ref)
    assert bad[0].size == 0, f"{bad[0].size} scale bytes differ, first at {bad[0][0]}, {bad[1][0]}"
    bad = np.nonzero(host(codes) != codes_ref)
    assert bad[0].size == 0, f"{bad[0].size} code bytes differ, first at {bad[0][0]}, {bad[1][0]}"
    return codes_ref, sc_ref


# lead 6 gives the scale 1.0, 8.25 the scale 1.375, 6 * 2^-8 the subnormal 2^-8
@pytest.mark.parametrize("lead", [6.0, 8.25, 6 * 2.0 ** -8])
def test_every_fp16_value_in_range(orc, lead):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = h[np.isfinite(h) & (np.abs(h.astype(np.float32)) <= lead)]
    nblk = (f.size + 14) // 15
    vals = np.zeros(nblk * 15, np.float16)
    vals[: f.size] = f
    blocks = np.concatenate([np.full((nblk, 1), lead, np.float16), vals.reshape(nblk, 15)], axis=1)
    K = 1024
    row = np.zeros(((blocks.size + K - 1) // K) * K, np.float16)
    row[: blocks.size] = blocks.reshape(-1)
    compare_quant(orc, row.reshape(-1, K))


@pytest.mark.parametrize("N,K", [(1, 16), (7, 48), (100, 1024), (33, 8256), (64, 4096)])
def test_quantizer_shapes(orc, N, K):
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0, :16] = 0
    if N > 3:
        W[1, :16] = -0.3
        W[2] *= 100
        W[3, 16:32] *= 3e5           # amax / 6 past 448: the saturated scale
    compare_quant(orc, W.astype(np.float16))


def run_linear(orc, M, N, K, seed):
    W, X = workloads.small_case(seed, M, N, K)
    codes, sc = orc.nvfp4_quantize(W)
    Y = host(q4.nvfp4_linear(gpu(X), gpu(codes), gpu(sc)))
    Yref, B = orc.nvfp4_ref(X, codes, sc)
    return check_gemm(Y, Yref, B, f"nvfp4 M={M} N={N} K={K}")


# up to 16 rows per decode pass, more rows in several passes
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (1, 300, 1024), (3, 77, 256), (16, 300, 640),
                                   (17, 129, 384), (40, 64, 4096), (1, 11008, 4096), (2, 4096, 11008),
                                   (5, 1000, 8192), (16, 11008, 4096), (9, 257, 1024), (1, 64, 32768)])
def test_linear_shapes(orc, M, N, K):
    run_linear(orc, M, N, K, M * 73 + N + K)


@pytest.mark.parametrize("N", [11008, 4096])
def test_decode_workload(orc, N):
    w = workloads.decode(N)
    codes, sc = q4.nvfp4_quantize(gpu(w["W"]))
    codes_ref, sc_ref = orc.nvfp4_quantize(w["W"])
    assert np.array_equal(host(codes), codes_ref) and np.array_equal(host(sc), sc_ref)
    Y = host(q4.nvfp4_linear(gpu(w["X"]), codes, sc))
    Yref, B = orc.nvfp4_ref(w["X"], codes_ref, sc_ref)
    check_gemm(Y, Yref, B, f"nvfp4 decode N={N}")


def one_hot(orc, M, N, K, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.3).astype(np.float16)
    codes, sc = orc.nvfp4_quantize(W)
    kk = (np.arange(M) * 7 + 3) % K
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), kk] = 1.0
    Y = host(q4.nvfp4_linear(gpu(X), gpu(codes), gpu(sc)))
    expect = orc.nvfp4_dequant(codes, sc)[:, kk].T.astype(np.float16)   # exact in fp16
    # equal as numbers: bit for bit except the sign of zero (a -0 weight comes
    # out +0, since the fp32 sum adds the +0 products of the other k)
    assert np.array_equal(Y.astype(np.float32), expect.astype(np.float32))
    assert (expect == 0).any() and (expect != 0).mean() > 0.9


def test_decode_one_hot(orc):
    """X[m, k(m)] = 1 for 16 rows: Y[m, n] is w_hat[n, k(m)] bit for bit -- the
    E2M1 lookup, the sign, the E4M3 scale of each block of 16 and the k order."""
    one_hot(orc, 16, 300, 1024, 1)


# M > 48: the large-M GEMM with e2m1 * e4m3 (exact) dequantized into LDS, at
# each tile width, ragged in M and N.
@pytest.mark.parametrize("nu", [4, 8, 11])
@pytest.mark.parametrize("M,N,K", [(49, 100, 256), (300, 1000, 768), (513, 383, 1280), (256, 352, 128)])
def test_large_m_shapes(orc, monkeypatch, nu, M, N, K):
    monkeypatch.setenv("Q4_GEMM_NU", str(nu))
    run_linear(orc, M, N, K, M * 5 + N + K + nu)


@pytest.mark.parametrize("nu", [4, 11])
def test_large_m_one_hot(orc, monkeypatch, nu):
    monkeypatch.setenv("Q4_GEMM_NU", str(nu))
    one_hot(orc, 300, 385, 512, nu)


def test_prefill_shape_sampled(orc):
    w = workloads.prefill()
    codes, sc = q4.nvfp4_quantize(gpu(w["W"]))
    Y = host(q4.nvfp4_linear(gpu(w["X"]), codes, sc))
    rows = sample_rows(w["X"].shape[0])
    Yref, B = orc.nvfp4_ref(w["X"], host(codes), host(sc), rows=rows)
    check_gemm(Y[rows], Yref, B, "nvfp4 prefill shape")
