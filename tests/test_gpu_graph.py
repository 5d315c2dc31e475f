"""HIP-graph capture of the layers as a serving loop would use them: each
call is captured once with static input and output buffers (and, for W8A8,
a static workspace), then replayed several times with new X contents copied
in and eager work and synchronisations between the replays. Every replay
must equal the eager call on the same input bit for bit (the same kernels
on the same data), and the first eager result is checked against the
oracle, so a kernel that depended on state left by a previous launch (a
counter, a cleared buffer) would show up here."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host

pytestmark = pytest.mark.gpu


def capture(call):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                      # first call outside the graph (one-time set-up)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def check_replays(call, eager, X, outs, seed, reps=4):
    g = capture(call)
    rng = np.random.default_rng(seed)
    for r in range(reps):
        Xr = gpu(rng.standard_normal(tuple(X.shape)).astype(np.float16))
        X.copy_(Xr)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(o) for o in outs]
        _ = torch.empty(1 << 20, device=X.device).uniform_()   # unrelated eager work between replays
        want = [host(o) for o in eager(Xr)]
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"replay {r} differs from the eager call"


def test_w4a16_decode_step(orc):
    """The decode step (N = 11008 and 4096 on one X, one launch)."""
    ws = [workloads.decode(N) for N in (11008, 4096)]
    layers = []
    for w in ws:
        c, s, z = orc.q4_quantize_pack(w["W"], g=128, sym=False)
        layers.append((gpu(c), gpu(s), gpu(z)))
    X = gpu(ws[0]["X"])
    outs = [torch.empty((1, N), dtype=torch.float16, device=X.device) for N in (11008, 4096)]
    call = lambda: q4.w4a16_linear_multi(X, layers, out=outs)
    eager = lambda Xr: q4.w4a16_linear_multi(Xr, layers)
    y0 = host(eager(X)[0])
    c, s, z = (host(t) for t in layers[0])
    Yref, B = orc.w4a16_ref(ws[0]["X"], c, s, z)
    check_gemm(y0, Yref, B, "graph: decode step, N = 11008")
    check_replays(call, eager, X, outs, 1)


@pytest.mark.parametrize("M", [16, 300])
def test_w4a16_batched_and_prefill(orc, M):
    W, X0 = workloads.small_case(31, M, 2048, 4096)
    c, s, z = (gpu(t) for t in orc.q4_quantize_pack(W, g=128))
    X = gpu(X0)
    Y = torch.empty((M, 2048), dtype=torch.float16, device=X.device)
    check_replays(lambda: q4.w4a16_linear(X, c, s, z, out=Y), lambda Xr: [q4.w4a16_linear(Xr, c, s, z)], X, [Y], M)


@pytest.mark.parametrize("fmt", ["w8a8", "fp8", "mxfp4"])
def test_w8_decode_layers(orc, fmt):
    """The one-launch decode layers that quantize X inside the GEMV (the
    workspace receives the codes and scales on every call)."""
    M, N, K = 1, 4096, 4096
    W, X0 = workloads.small_case(32, M, N, K)
    X = gpu(X0)
    Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    wsp = q4.w8a8_workspace(M, K, X.device)
    if fmt == "w8a8":
        Wq, sw = (gpu(t) for t in orc.q8_quantize_weight(W))
        call = lambda: q4.w8a8_linear(X, Wq, sw, workspace=wsp, out=Y)
        eager = lambda Xr: [q4.w8a8_linear(Xr, Wq, sw)]
    elif fmt == "fp8":
        Wq, sw = (gpu(t) for t in orc.fp8_quantize_weight(W))
        call = lambda: q4.fp8_linear(X, Wq, sw, workspace=wsp, out=Y)
        eager = lambda Xr: [q4.fp8_linear(Xr, Wq, sw)]
    else:
        cq, sq = (gpu(t) for t in orc.mxfp4_quantize_weight(W))
        call = lambda: q4.mxfp4_linear(X, cq, sq, workspace=wsp, out=Y)
        eager = lambda Xr: [q4.mxfp4_linear(Xr, cq, sq)]
    check_replays(call, eager, X, [Y], 7)


@pytest.mark.parametrize("fmt", ["nf4", "nvfp4"])
@pytest.mark.parametrize("M", [1, 100])
def test_lookup_layers(orc, fmt, M):
    W, X0 = workloads.small_case(33, M, 2048, 4096)
    quant, lin = (orc.nf4_quantize, q4.nf4_linear) if fmt == "nf4" else (orc.nvfp4_quantize, q4.nvfp4_linear)
    c, s = (gpu(t) for t in quant(W))
    X = gpu(X0)
    Y = torch.empty((M, 2048), dtype=torch.float16, device=X.device)
    check_replays(lambda: lin(X, c, s, out=Y), lambda Xr: [lin(Xr, c, s)], X, [Y], M + 3)


@pytest.mark.parametrize("fp8", [False, True])
def test_layernorm_quant(orc, fp8):
    """The LayerNorm with the divide and the per-token quantizer fused in
    (INT8 and E4M3 forms), as a serving loop would capture it."""
    M, K = 64, 4096
    p = workloads.layernorm_params(K)
    gam, bet, s = gpu(p["gamma"]), gpu(p["beta"]), gpu(p["s"])
    X0 = np.random.default_rng(31).standard_normal((M, K)).astype(np.float16)
    X = gpu(X0)
    fn = q4.layernorm_quant_smooth_fp8 if fp8 else q4.layernorm_quant_smooth
    ref = orc.layernorm_quant_smooth_fp8 if fp8 else orc.layernorm_quant_smooth
    q = torch.empty((M, K), dtype=torch.uint8 if fp8 else torch.int8, device=X.device)
    sx = torch.empty(M, dtype=torch.float32, device=X.device)
    fn(X, gam, bet, s, 1e-5, out=(q, sx))
    rq, rs = ref(X0, p["gamma"], p["beta"], p["s"], 1e-5)
    assert np.array_equal(host(q), rq) and np.array_equal(host(sx).view(np.uint32), rs.view(np.uint32))
    call = lambda: fn(X, gam, bet, s, 1e-5, out=(q, sx))
    eager = lambda Xr: fn(Xr, gam, bet, s, 1e-5)
    check_replays(call, eager, X, [q, sx], seed=37)
