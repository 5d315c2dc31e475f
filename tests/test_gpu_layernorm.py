"""GPU parity of the fused LayerNorm + SmoothQuant divide + per-token INT8
quantizer against the oracle: codes and scales bit for bit on the full
W8A8-shaped workload (2048 x 8192), on every chunk layout of the kernel
(K a multiple of 512, and K that leaves partial chunks), on rows whose
squares a running fp64 sum would round differently, constant rows,
fp16-extreme rows, more rows than wavefronts (rows revisited by the grid
stride), and flagged rows (NaN / infinity in X, x' past the fp32 range);
the FP8 E4M3 form on the same cases."""
import numpy as np
import pytest

import quantized_gemm_q4_amd as q4
import workloads
from parity import gpu, host

pytestmark = pytest.mark.gpu


def _params(K, seed):
    rng = np.random.default_rng(seed)
    return ((1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32),
            (0.05 * rng.standard_normal(K)).astype(np.float32),
            np.exp(0.5 * rng.standard_normal(K)).astype(np.float32))


def _x(M, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, rng.permutation(K)[: max(1, K // 100)]] *= 30
    return X.astype(np.float16)


def _check(orc, X, gamma, beta, s, eps=1e-5, fp8=False):
    ref = orc.layernorm_quant_smooth_fp8 if fp8 else orc.layernorm_quant_smooth
    fn = q4.layernorm_quant_smooth_fp8 if fp8 else q4.layernorm_quant_smooth
    ref_q, ref_s = ref(X, gamma, beta, s, eps)
    Xq, sx = fn(gpu(X), gpu(gamma), gpu(beta), None if s is None else gpu(s), eps)
    got_q, got_s = host(Xq), host(sx)
    bad = np.nonzero((got_q != ref_q).any(axis=1) | (got_s.view(np.uint32) != ref_s.view(np.uint32)))[0]
    assert bad.size == 0, f"rows {bad[:8]} differ (of {X.shape[0]})"
    return ref_q, ref_s


@pytest.mark.parametrize("M,K", [(1, 4096), (7, 512), (33, 1024), (9, 8192), (20, 5120), (3, 1536),
                                 (5, 200), (4, 2056), (3, 4104), (2, 8), (70, 8184)])
@pytest.mark.parametrize("smooth", [False, True])
def test_shapes(orc, M, K, smooth):
    gamma, beta, s = _params(K, M + K)
    _check(orc, _x(M, K, 3 * M + K), gamma, beta, s if smooth else None)


def test_workload_full(orc):
    """The W8A8 workload's activation (2048 x 8192, 82 channels x30) as the
    hidden state in front of the norm: every row bit for bit."""
    X = workloads.w8a8()["X"]
    p = workloads.layernorm_params(X.shape[1])
    q, sx = _check(orc, X, p["gamma"], p["beta"], p["s"])
    assert (np.abs(q).max(axis=1) == 127).all() and np.isfinite(sx).all()


def test_grid_stride_rows(orc):
    """More rows than the grid's wavefronts (256 blocks x 8): waves take
    several rows, with the next row's loads issued after the codes."""
    K = 8192
    gamma, beta, s = _params(K, 1)
    _check(orc, _x(4100, K, 2), gamma, beta, s)
    gamma, beta, s = _params(1024, 3)
    _check(orc, _x(5003, 1024, 4), gamma, beta, s)


def test_exact_sums_and_special_rows(orc):
    K = 8192
    rng = np.random.default_rng(5)
    rows = []
    for big in (65504.0, 30000.0, 4096.0):   # squares a running fp64 sum would drop
        r = np.full(K, 2.0 ** -11, np.float32) * rng.choice([-1.0, 1.0], K).astype(np.float32)
        r[rng.choice(K, 3, replace=False)] = [big, -big, big / 2]
        rows.append(r)
    rows.append(np.full(K, 3.25, np.float32))                       # constant: variance 0
    rows.append(np.full(K, -65504.0, np.float32))                   # constant at the fp16 limit
    rows.append(np.where(np.arange(K) % 2 == 0, 65504.0, -65504.0))  # +-max: the largest sums
    rows.append(np.full(K, 2.0 ** -24, np.float32))                 # subnormal
    rows.append(np.zeros(K, np.float32))
    X = np.array(rows, np.float32).astype(np.float16)
    gamma, beta, s = _params(K, 7)
    _check(orc, X, gamma, beta, s)
    _check(orc, X, np.ones(K, np.float32), np.zeros(K, np.float32), None)


def test_flagged_rows(orc):
    M, K = 12, 4096
    X = _x(M, K, 8)
    X[1, 5] = np.float16(np.nan)
    X[4, 0] = np.float16(np.inf)
    X[7, 4095] = np.float16(-np.inf)
    X[9, 100] = np.float16(np.inf)
    X[9, 101] = np.float16(-np.inf)
    gamma, beta, s = _params(K, 9)
    q, sx = _check(orc, X, gamma, beta, s)
    assert np.isnan(sx[[1, 4, 7, 9]]).all() and np.isfinite(sx[[0, 2, 3, 5, 6, 8, 10, 11]]).all()
    # an x' past the fp32 range flags every row; a zero smoothing factor too
    big, s2 = beta.copy(), s.copy()
    big[17], s2[17] = 3e38, 1e-3
    q, sx = _check(orc, X, gamma, big, s2)
    assert np.isnan(sx).all()
    s3 = s.copy()
    s3[3] = 0.0
    _check(orc, X, gamma, beta, s3)


@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.25])
def test_eps(orc, eps):
    gamma, beta, s = _params(1024, 11)
    X = _x(6, 1024, 12)
    X[2] = np.float16(0.5)   # var = 0: x' = b only through eps
    _check(orc, X, gamma, beta, s, eps)


@pytest.mark.parametrize("M,K", [(1, 4096), (33, 1024), (9, 8192), (5, 200), (3, 4104)])
def test_fp8_shapes(orc, M, K):
    gamma, beta, s = _params(K, M + K + 1)
    X = _x(M, K, 3 * M + K + 1)
    if M > 2:
        X[1, 0] = np.float16(np.inf)
    _check(orc, X, gamma, beta, s, fp8=True)


def test_fp8_workload_full(orc):
    X = workloads.w8a8()["X"]
    p = workloads.layernorm_params(X.shape[1])
    q, sx = _check(orc, X, p["gamma"], p["beta"], p["s"], fp8=True)
    assert ((q & 0x7F) == 0x7E).any(axis=1).all() and np.isfinite(sx).all()
