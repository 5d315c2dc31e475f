"""GPU parity of the NF4 path against the oracle: codes and block scales bit
for bit (every fp16 value of magnitude <= 1 at scale 1 and at a non-power-of-
two scale, zero and constant blocks, random weights), and the NF4 decode
GEMV within tolerance of the exact product over the dequantized weight, over
ragged shapes, row chunks of X and the decode workload's layers."""
import numpy as np
import pytest

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, sample_rows

pytestmark = pytest.mark.gpu


def compare_quant(orc, W):
    codes, sc = q4.nf4_quantize(gpu(W))
    codes_ref, sc_ref = orc.nf4_quantize(W)
    assert np.array_equal(host(sc).view(np.uint32), sc_ref.view(np.uint32))
    bad = np.nonzero(host(codes) != codes_ref)
    assert bad[0].size == 0, f"{bad[0].size} code bytes differ, first at {bad[0][0]}, {bad[1][0]}"
    return codes_ref, sc_ref


@pytest.mark.parametrize("lead", [1.0, 0.75])
def test_every_small_fp16_value(orc, lead):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = h[np.isfinite(h) & (np.abs(h.astype(np.float32)) <= lead)]
    nblk = (f.size + 62) // 63
    vals = np.zeros(nblk * 63, np.float16)
    vals[: f.size] = f
    blocks = np.concatenate([np.full((nblk, 1), lead, np.float16), vals.reshape(nblk, 63)], axis=1)
    K = 1024
    row = np.zeros(((blocks.size + K - 1) // K) * K, np.float16)
    row[: blocks.size] = blocks.reshape(-1)
    compare_quant(orc, row.reshape(-1, K))


@pytest.mark.parametrize("N,K", [(1, 64), (7, 128), (100, 1024), (33, 8256), (64, 4096)])
def test_quantizer_shapes(orc, N, K):
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0, :64] = 0
    if N > 2:
        W[1, :64] = -0.3
        W[2] *= 100
    compare_quant(orc, W.astype(np.float16))


def run_linear(orc, M, N, K, seed):
    W, X = workloads.small_case(seed, M, N, K)
    codes, sc = orc.nf4_quantize(W)
    Y = host(q4.nf4_linear(gpu(X), gpu(codes), gpu(sc)))
    Yref, B = orc.nf4_ref(X, codes, sc)
    return check_gemm(Y, Yref, B, f"nf4 M={M} N={N} K={K}")


# up to 8 rows per pass the two 64-block halves ride in paired MFMA rows, 9 to
# 16 in two MFMA chains; large K passes fewer rows at a time, and past 9 rows
# of X in the LDS only paired passes of 8 (K = 32768)
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (1, 300, 1024), (3, 77, 256), (16, 300, 640),
                                   (17, 129, 384), (40, 64, 4096), (1, 11008, 4096), (2, 4096, 11008),
                                   (5, 1000, 8192), (16, 11008, 4096), (64, 1000, 4096),
                                   (8, 500, 2048), (9, 257, 1024), (12, 130, 28672), (1, 64, 32768),
                                   (12, 40, 32768)])
def test_linear_shapes(orc, M, N, K):
    run_linear(orc, M, N, K, M * 71 + N + K)


@pytest.mark.parametrize("N", [11008, 4096])
def test_decode_workload(orc, N):
    w = workloads.decode(N)
    codes, sc = q4.nf4_quantize(gpu(w["W"]))
    codes_ref, sc_ref = orc.nf4_quantize(w["W"])
    assert np.array_equal(host(codes), codes_ref)
    Y = host(q4.nf4_linear(gpu(w["X"]), codes, sc))
    Yref, B = orc.nf4_ref(w["X"], codes_ref, sc_ref)
    check_gemm(Y, Yref, B, f"nf4 decode N={N}")


# M > 48: the large-M GEMM with the NF4 weight dequantized (level * block
# scale, rounded once to fp16) into LDS, at each tile width, ragged in M and N.
@pytest.mark.parametrize("nu", [4, 8, 11])
@pytest.mark.parametrize("M,N,K", [(49, 100, 256), (300, 1000, 768), (513, 383, 1280), (256, 352, 128)])
def test_large_m_shapes(orc, monkeypatch, nu, M, N, K):
    monkeypatch.setenv("Q4_GEMM_NU", str(nu))
    run_linear(orc, M, N, K, M * 5 + N + K + nu)


@pytest.mark.parametrize("nu", [4, 11])
def test_large_m_one_hot(orc, monkeypatch, nu):
    """X[m, k(m)] = 1: Y[m, n] is the dequantized weight w_hat[n, k(m)] as the
    GEMM forms it (the fp32 product of the level and the block scale, rounded
    to fp16), bit for bit: pins the level lookup, the block-scale indexing and
    the k order."""
    monkeypatch.setenv("Q4_GEMM_NU", str(nu))
    M, N, K = 300, 385, 512
    rng = np.random.default_rng(nu)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, sc = orc.nf4_quantize(W)
    kk = (np.arange(M) * 7 + 3) % K
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), kk] = 1.0
    Y = host(q4.nf4_linear(gpu(X), gpu(codes), gpu(sc)))
    lv = orc.nf4_levels().astype(np.float32)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(N, K)
    w32 = lv[nib] * np.repeat(sc, 64, axis=1)          # fp32 products (exact level x fp32 scale)
    expect = w32[:, kk].T.astype(np.float16)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))


def test_prefill_shape_sampled(orc):
    w = workloads.prefill()
    codes, sc = q4.nf4_quantize(gpu(w["W"]))
    Y = host(q4.nf4_linear(gpu(w["X"]), codes, sc))
    rows = sample_rows(w["X"].shape[0])
    Yref, B = orc.nf4_ref(w["X"], host(codes), host(sc), rows=rows)
    check_gemm(Y[rows], Yref, B, "nf4 prefill shape")
