"""GPU parity of w4a16_linear against the oracle's exact fp64 product over
the dequantized weight: small shapes that span several tiles with ragged M
and N (both the skinny M <= 64 kernel and the tiled prefill kernel), one-hot
inputs that pin nibble order and scale/zero indexing bit for bit, and the
full-size decode, batched-decode and prefill workloads in the launch
configuration the benchmark times (prefill on sampled rows)."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host, sample_rows

pytestmark = pytest.mark.gpu


def quantize_gpu(W, g, sym):
    return q4.q4_quantize_pack(gpu(W), g=g, sym=sym)


def run_case(orc, W, X, g, sym, rows=None, what=""):
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=sym)
    Y = host(q4.w4a16_linear(gpu(X), gpu(codes), gpu(scales.view(np.float16)),
                             None if zeros is None else gpu(zeros), g=g))
    Yref, B = orc.w4a16_ref(X, codes, scales, zeros, g=g, rows=rows)
    Ysel = Y if rows is None else Y[rows]
    return check_gemm(Ysel, Yref, B, what)


def test_tiny_workload(orc):
    w = workloads.tiny()
    run_case(orc, w["W"], w["X"], w["g"], w["sym"], what="tiny")


SHAPES = [(1, 16, 128), (1, 1000, 1024), (2, 33, 256), (3, 77, 256), (16, 300, 640),
          (17, 129, 384), (33, 64, 256), (64, 130, 512), (65, 129, 384), (128, 128, 128),
          (200, 260, 1024), (300, 1000, 768), (256, 130, 256), (257, 1, 128)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("sym", [False, True])
def test_shapes(orc, M, N, K, sym):
    W, X = workloads.small_case(M * 7919 + N * 31 + K, M, N, K)
    run_case(orc, W, X, 128, sym, what=f"M={M} N={N} K={K} sym={sym}")


@pytest.mark.parametrize("M,K,N", [(64, 256, 100), (7, 384, 33), (256, 256, 130)])
def test_one_hot_pins_layout(orc, M, K, N):
    """X = rows of the identity: Y[m, n] = fp16(w_hat[n, m]) exactly."""
    rng = np.random.default_rng(M + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=128, sym=False)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), np.arange(M)] = 1.0
    Y = host(q4.w4a16_linear(gpu(X), gpu(codes), gpu(scales.view(np.float16)), gpu(zeros)))
    w_hat = orc.q4_dequant(codes, scales, zeros, K, 128)
    expect = w_hat[:, :M].T.astype(np.float16)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))


# The large-M kernel (M >= 256) at each of its tile widths (32 * nu output
# columns per tile), ragged in M and N, with one 32-wide k step per group
# quarter: K = 128 is a single group, g = 256 spans two steps' worth of groups.
LARGE_SHAPES = [(256, 352, 128, 128), (300, 1000, 768, 128), (513, 700, 1280, 128),
                (260, 383, 1024, 256)]


@pytest.mark.parametrize("nu", [4, 8, 11])
@pytest.mark.parametrize("M,N,K,g", LARGE_SHAPES)
@pytest.mark.parametrize("sym", [False, True])
def test_large_m_tile_widths(orc, monkeypatch, nu, M, N, K, g, sym):
    monkeypatch.setenv("Q4_GEMM_NU", str(nu))
    W, X = workloads.small_case(M * 3 + N * 5 + K + g + nu, M, N, K)
    run_case(orc, W, X, g, sym, what=f"large-M nu={nu} M={M} N={N} K={K} g={g} sym={sym}")


@pytest.mark.parametrize("nu", [4, 8, 11])
@pytest.mark.parametrize("sym", [False, True])
def test_large_m_one_hot(orc, monkeypatch, nu, sym):
    """X[m, k(m)] = 1 for a spread of k: Y[m, n] = fp16(w_hat[n, k(m)])
    exactly, which pins the dequantized value of every weight used, its
    scale and zero-point indexing and the X/W k order, bit for bit."""
    monkeypatch.setenv("Q4_GEMM_NU", str(nu))
    M, N, K, g = 300, 385, 512, 256
    rng = np.random.default_rng(nu * 2 + int(sym))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=sym)
    kk = (np.arange(M) * 7 + 3) % K
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), kk] = 1.0
    Y = host(q4.w4a16_linear(gpu(X), gpu(codes), gpu(scales.view(np.float16)),
                             None if zeros is None else gpu(zeros), g=g))
    w_hat = orc.q4_dequant(codes, scales, zeros, K, g)
    expect = w_hat[:, kk].T.astype(np.float16)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))


def test_prefill_shape_asym_sampled(orc):
    """The prefill shape with asymmetric codes at M = 512 (the tile-width
    choice differs from M = 2048), checked on sampled rows."""
    w = workloads.prefill()
    X = w["X"][:512]
    q = quantize_gpu(w["W"], 128, False)
    codes, scales, zeros = (host(t) for t in q)
    Y = host(q4.w4a16_linear(gpu(X), *q))
    rows = sample_rows(X.shape[0])
    Yref, B = orc.w4a16_ref(X, codes, scales, zeros, rows=rows)
    check_gemm(Y[rows], Yref, B, "prefill shape asym M=512")


def test_codes_at_zero_point_give_zero(orc):
    M, N, K = 300, 50, 512
    X = workloads.normal_fp16(5, (M, K))
    codes = np.full((N, K // 2), 0x33, np.uint8)
    zeros = np.full((N, 2), 0x33, np.uint8)
    scales = np.full((N, 4), 0.7, np.float16)
    for m in (1, 20, 70, M):
        Y = host(q4.w4a16_linear(gpu(X[:m]), gpu(codes), gpu(scales), gpu(zeros)))
        assert np.all(Y == 0)


@pytest.mark.parametrize("N", [11008, 4096])
def test_decode_workload(orc, N):
    w = workloads.decode(N)
    q = quantize_gpu(w["W"], w["g"], w["sym"])
    codes, scales, zeros = (None if t is None else host(t) for t in q)
    Y = host(q4.w4a16_linear(gpu(w["X"]), *q))
    Yref, B = orc.w4a16_ref(w["X"], codes, scales, zeros)
    check_gemm(Y, Yref, B, f"decode N={N}")


@pytest.mark.parametrize("M", [16, 64])
def test_batched_decode_workload(orc, M):
    w = workloads.quant(M)
    q = quantize_gpu(w["W"], w["g"], w["sym"])
    codes, scales, zeros = (None if t is None else host(t) for t in q)
    Y = host(q4.w4a16_linear(gpu(w["X"]), *q))
    Yref, B = orc.w4a16_ref(w["X"], codes, scales, zeros)
    check_gemm(Y, Yref, B, f"batched decode M={M}")


def test_prefill_workload_sampled(orc):
    w = workloads.prefill()
    q = quantize_gpu(w["W"], w["g"], w["sym"])
    codes, scales, zeros = (None if t is None else host(t) for t in q)
    Y = host(q4.w4a16_linear(gpu(w["X"]), *q))
    rows = sample_rows(w["X"].shape[0])
    Yref, B = orc.w4a16_ref(w["X"], codes, scales, zeros, rows=rows)
    check_gemm(Y[rows], Yref, B, "prefill")
    assert np.isfinite(Y.astype(np.float32)).all()


def test_errors_and_empty():
    X = torch.zeros((4, 240), dtype=torch.float16, device="cuda")
    codes = torch.zeros((8, 120), dtype=torch.uint8, device="cuda")
    with pytest.raises(q4.Q4Error) as e:   # 80 is not a multiple of 32
        q4.w4a16_linear(X, codes, torch.zeros((8, 3), dtype=torch.float16, device="cuda"), None, g=80)
    assert e.value.status == q4.Q4_ERR_UNSUPPORTED
    X = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    codes = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    Y = q4.w4a16_linear(X[:0], codes, torch.zeros((8, 2), dtype=torch.float16, device="cuda"), None)
    assert Y.shape == (0, 8)
    with pytest.raises(q4.Q4Error) as e:
        q4.w4a16_linear(X.view(-1)[1:257].view(1, 256), codes,
                        torch.zeros((8, 2), dtype=torch.float16, device="cuda"), None)
    assert e.value.status == q4.Q4_ERR_MISALIGNED


# Shapes that route to each launch variant of the decode GEMV kernel
# (wavefronts per block x k-blocks per wavefront): (11008, 4096) -> 4 x 8,
# (4096, 4096) -> 8 x 4, (1000, 4096) -> 16 x 2 with a ragged last tile,
# (4096, 8192) -> 8 x 8; M up to 7 (X must fit in 64 KiB of LDS).
# With several X rows each wavefront stages the rows of its own k-range
# (M * k-blocks per wavefront <= 32); Q4_GEMV_PW=0 forces the block-staged
# form that larger M * k-blocks take.
@pytest.mark.parametrize("M,N,K", [(1, 11008, 4096), (3, 11008, 4096), (1, 4096, 4096),
                                   (7, 4096, 4096), (2, 1000, 4096), (1, 4096, 8192),
                                   (5, 4096, 8192), (8, 11008, 4096), (4, 4096, 16384)])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("pw", ["1", "0"])
def test_gemv_variants(orc, monkeypatch, M, N, K, sym, pw):
    monkeypatch.setenv("Q4_GEMV_PW", pw)
    W, X = workloads.small_case(M * 13 + N + K * 3 + int(sym), M, N, K)
    run_case(orc, W, X, 128, sym, what=f"gemv M={M} N={N} K={K} sym={sym} pw={pw}")


# Shapes that route to each variant of the batched-decode kernels (8 <= M <=
# 64): X resident in LDS (M <= 16, K = 1024, 2048, 4096), code runs resident
# in registers with X through the LDS ring (M = 20, 33, 64 at K = 1024, 2048,
# 4096: one or two k-split groups), the X ring with row tiles of 16 (M <= 16,
# K = 6144), 32 (M = 20) and 64 (M = 33, 64) at K = 3072 and 6144, the
# skinny fallback (M <= 16, K = 3072); ragged M and N (the last block's
# columns run past N).
@pytest.mark.parametrize("M", [8, 16, 20, 33, 64])
@pytest.mark.parametrize("K", [1024, 2048, 3072, 4096, 6144])
@pytest.mark.parametrize("sym", [False, True])
def test_batched_variants(orc, M, K, sym):
    N = 300
    W, X = workloads.small_case(M * 7 + K + int(sym), M, N, K)
    run_case(orc, W, X, 128, sym, what=f"batched M={M} N={N} K={K} sym={sym}")


# The X-in-registers batched decode (8 <= M <= 16, K = 2048 or 4096, N <=
# 4096): g = 32 / 64 / 128, symmetric and asymmetric, ragged N (the last
# column tile runs past N) and M below 16 (rows of the X fragments past M
# are zero); the second decode layer's shape (N = 4096).
@pytest.mark.parametrize("M,N", [(8, 1000), (11, 1000), (16, 1000), (16, 4096)])
@pytest.mark.parametrize("K", [2048, 4096])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("sym", [False, True])
def test_batched_xreg(orc, M, N, K, g, sym):
    W, X = workloads.small_case(M * 17 + N + K + g * 3 + int(sym), M, N, K)
    run_case(orc, W, X, g, sym, what=f"xreg g={g} M={M} N={N} K={K} sym={sym}")


@pytest.mark.parametrize("K", [2048, 4096])
@pytest.mark.parametrize("g", [32, 64, 128])
def test_batched_xreg_one_hot(orc, K, g):
    """One-hot X rows whose k lie in different wavefronts' k-ranges, k-blocks
    and lane groups: Y[m, n] = fp16(w_hat[n, k(m)]) exactly (pins the X
    fragment order, the lane transpose of the code runs and the scale and
    zero-point indexing)."""
    M, N = 16, 100
    rng = np.random.default_rng(K + g)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=False)
    kk = (np.arange(M) * 1031 + 7) % K
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), kk] = 1.0
    Y = host(q4.w4a16_linear(gpu(X), gpu(codes), gpu(scales.view(np.float16)), gpu(zeros), g=g))
    w_hat = orc.q4_dequant(codes, scales, zeros, K, g)
    expect = w_hat[:, kk].T.astype(np.float16)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))


# N large enough that 48-column blocks would not fit one round of the CUs:
# the X-resident kernel (M <= 16) and the whole-slice kernel (16 < M <= 64,
# one or two k-split groups) then use 64-column blocks (4 column tiles).
@pytest.mark.parametrize("M,K", [(8, 1024), (16, 1024), (20, 1024), (64, 1024), (40, 4096)])
@pytest.mark.parametrize("sym", [False, True])
def test_batched_wide_n(orc, M, K, sym):
    N = 12800
    W, X = workloads.small_case(M * 11 + int(sym), M, N, K)
    run_case(orc, W, X, 128, sym, what=f"batched wide M={M} N={N} K={K} sym={sym}")


# A packed weight past 4 GiB (codes of 2^32 + 2^20 bytes, K = 65536): byte
# offsets beyond 32 bits. The GEMV and batched kernels decline such operands
# and the 64-bit kernels run; sampled columns (the last rows lie past the
# 2^32-byte mark) against the oracle. Codes, scales and zero-points are drawn
# on the GPU from a seeded generator and copied back for the sampled rows.
@pytest.mark.parametrize("M", [1, 20, 300])
def test_weight_past_32bit_offsets(orc, M):
    K = 65536
    N = (2 ** 32 + 2 ** 20) // (K // 2)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7 + M)
    codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=gen)
    scales = (torch.rand((N, K // 128), device="cuda", generator=gen) * 0.01 + 0.002).half()
    zeros = torch.randint(0, 256, (N, K // 256), dtype=torch.uint8, device="cuda", generator=gen)
    X = workloads.normal_fp16(101 + M, (M, K), 1.0)
    Y = host(q4.w4a16_linear(gpu(X), codes, scales, zeros))
    rng = np.random.default_rng(M)
    sel = np.unique(np.concatenate([[0, 1, N // 2, N - 33, N - 2, N - 1], rng.integers(0, N, 20)]))
    idx = torch.from_numpy(sel).to("cuda")
    c, s, z = (host(t.index_select(0, idx)) for t in (codes, scales, zeros))
    Yref, B = orc.w4a16_ref(X, c, s.view(np.uint16), z)
    check_gemm(Y[:, sel], Yref, B, f"M={M} N={N} K={K} past 32-bit offsets")
    del codes, scales, zeros
    torch.cuda.empty_cache()


# Group sizes other than 128: g = 32 and 64 (what the quantizer also writes;
# the Core ideas granularity table uses g = 32) on every route -- the
# small-group kernel (any M; K a multiple of g but not of 128 included) and
# the large-M GEMM (M >= 256, K a multiple of 128) -- and g = 256, 384 (a
# multiple of 128 that is not a power of two never takes the large-M GEMM).
SMALL_G_SHAPES = [(1, 300, 512), (1, 1000, 96 * 4), (5, 77, 320), (16, 129, 1024),
                  (17, 64, 192), (33, 130, 640), (64, 100, 256), (65, 129, 384),
                  (300, 260, 512), (300, 100, 448)]


@pytest.mark.parametrize("M,N,K", SMALL_G_SHAPES)
@pytest.mark.parametrize("g", [32, 64])
@pytest.mark.parametrize("sym", [False, True])
def test_small_group_sizes(orc, M, N, K, g, sym):
    if K % g:
        pytest.skip("K must be a multiple of g")
    W, X = workloads.small_case(M * 5 + N * 3 + K + g + int(sym), M, N, K)
    run_case(orc, W, X, g, sym, what=f"g={g} M={M} N={N} K={K} sym={sym}")


# g = 32 and 64 on the decode GEMV (M <= 16, X within its LDS) and on the
# X-resident batched kernel (M <= 16 otherwise: K = 4096 with M >= 8, K = 2048
# with M = 16; 3 or 4 column tiles per block): the code runs transposed
# across the four lane groups so that each MFMA step sums one group; 2, 4 and
# 8 k-blocks per wavefront, one X row and several, ragged N, and the decode
# workload's shapes.
GEMV_SMALL_G = [(1, 300, 1024), (1, 300, 2048), (3, 130, 2048), (7, 1000, 1024), (16, 300, 4096),
                (1, 11008, 4096), (16, 4096, 4096), (8, 300, 4096), (16, 300, 2048), (10, 12800, 4096)]


@pytest.mark.parametrize("M,N,K", GEMV_SMALL_G)
@pytest.mark.parametrize("g", [32, 64])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("pw", ["1", "0"])
def test_small_group_gemv(orc, monkeypatch, M, N, K, g, sym, pw):
    monkeypatch.setenv("Q4_GEMV_PW", pw)
    W, X = workloads.small_case(M * 13 + N + K + g + int(sym), M, N, K)
    run_case(orc, W, X, g, sym, what=f"gemv g={g} M={M} N={N} K={K} sym={sym}")


# g = 32 and 64 on the batched kernel for 16 < M <= 64 (K = 1024, 2048 or
# 4096; X streamed through an LDS ring): the same lane transpose, each group's
# partial sum scaled when its last MFMA step ends; two and four 16-row tiles,
# one and two k-split groups, 3 and 4 column tiles per block, ragged N.
CRES_SMALL_G = [(17, 300, 1024), (32, 130, 2048), (33, 1000, 4096), (64, 300, 1024),
                (20, 4096, 2048), (48, 12800, 1024), (40, 12800, 4096), (64, 11008, 4096)]


@pytest.mark.parametrize("M,N,K", CRES_SMALL_G)
@pytest.mark.parametrize("g", [32, 64])
@pytest.mark.parametrize("sym", [False, True])
def test_small_group_batched(orc, M, N, K, g, sym):
    W, X = workloads.small_case(M * 11 + N + K + g + int(sym), M, N, K)
    run_case(orc, W, X, g, sym, what=f"batched g={g} M={M} N={N} K={K} sym={sym}")


@pytest.mark.parametrize("M", [1, 17, 65, 300])
@pytest.mark.parametrize("g", [256, 384])
@pytest.mark.parametrize("sym", [False, True])
def test_large_group_sizes(orc, M, g, sym):
    N, K = 200, 3 * 768
    W, X = workloads.small_case(M * 7 + g + int(sym), M, N, K)
    run_case(orc, W, X, g, sym, what=f"g={g} M={M} N={N} K={K} sym={sym}")


@pytest.mark.parametrize("M,K", [(40, 192), (300, 512), (300, 96), (1, 1024), (8, 1024), (16, 4096),
                                 (33, 2048), (64, 4096)])
@pytest.mark.parametrize("g", [32, 64])
def test_small_group_one_hot(orc, M, K, g):
    """One-hot X through the small-group kernel, the decode GEMV (M <= 16),
    the batched kernel (16 < M <= 64) and the large-M GEMM at g = 32 / 64:
    Y[m, n] = fp16(w_hat[n, k(m)]) exactly (pins each group's scale and
    zero-point indexing and the lane transpose)."""
    if K % g:
        pytest.skip("K must be a multiple of g")
    N = 70
    rng = np.random.default_rng(M + K + g)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=False)
    kk = (np.arange(M) * 5 + 1) % K
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), kk] = 1.0
    Y = host(q4.w4a16_linear(gpu(X), gpu(codes), gpu(scales.view(np.float16)), gpu(zeros), g=g))
    w_hat = orc.q4_dequant(codes, scales, zeros, K, g)
    expect = w_hat[:, kk].T.astype(np.float16)
    assert np.array_equal(Y.view(np.uint16), expect.view(np.uint16))


def test_quantize_out_must_match(orc):
    """q4_quantize_pack(out=...) checks the caller's buffers before any launch."""
    W = torch.zeros((8, 256), dtype=torch.float16, device="cuda")
    good = (torch.empty((8, 128), dtype=torch.uint8, device="cuda"),
            torch.empty((8, 8), dtype=torch.float16, device="cuda"),
            torch.empty((8, 4), dtype=torch.uint8, device="cuda"))
    q4.q4_quantize_pack(W, g=32, out=good)
    with pytest.raises(ValueError):   # sized for g = 128, used with g = 32
        q4.q4_quantize_pack(W, g=32, out=(good[0], torch.empty((8, 2), dtype=torch.float16, device="cuda"),
                                          torch.empty((8, 1), dtype=torch.uint8, device="cuda")))
    with pytest.raises(ValueError):
        q4.q4_quantize_pack(W, g=32, out=(good[0], good[1], None))
    with pytest.raises(TypeError):
        q4.q4_quantize_pack(W, g=32, out=(good[0], good[1].float(), good[2]))
    with pytest.raises(ValueError):
        q4.q4_quantize_pack(W, g=32, out=(good[0].cpu(), good[1], good[2]))


def test_debug_mode_synchronises_and_logs():
    """Q4_DEBUG=1: every call waits for its stream and logs itself to stderr
    (run in a child process: the mode is read when the library loads)."""
    import os
    import subprocess
    import sys
    code = (
        "import torch, quantized_gemm_q4_amd as q4\n"
        "W = torch.randn(64, 256, device='cuda').half()\n"
        "c, s, z = q4.q4_quantize_pack(W)\n"
        "Y = q4.w4a16_linear(torch.randn(3, 256, device='cuda').half(), c, s, z)\n"
        "print('rows', Y.shape[0])\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, Q4_DEBUG="1", PYTHONPATH=root)
    proc = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                          text=True, timeout=120)
    assert proc.returncode == 0, proc.stderr[-2000:]
    assert "rows 3" in proc.stdout
    assert "[q4] q4_quantize_pack: ok" in proc.stderr
    assert "[q4] w4a16_linear: ok" in proc.stderr
