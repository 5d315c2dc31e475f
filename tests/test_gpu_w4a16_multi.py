"""GPU parity of w4a16_linear_multi (several W4A16 layers reading one X)
against the oracle's exact fp64 product per layer: the decode workload's two
layers in one launch, ragged and empty layers, every GEMV launch variant the
one-launch form picks, and the shapes that fall back to one launch per layer
(M > 16, g = 256, mixed symmetric / asymmetric layers)."""
import numpy as np
import pytest
import torch

import quantized_gemm_q4_amd as q4
import workloads
from parity import check_gemm, gpu, host

pytestmark = pytest.mark.gpu


def packed(orc, W, g, sym):
    codes, scales, zeros = orc.q4_quantize_pack(W, g=g, sym=sym)
    return (codes, scales, zeros), (gpu(codes), gpu(scales.view(np.float16)),
                                    None if zeros is None else gpu(zeros))


def run_multi(orc, X, Ws, g, syms, what):
    host_packs, dev_packs = zip(*(packed(orc, W, g, s) for W, s in zip(Ws, syms)))
    Ys = q4.w4a16_linear_multi(gpu(X), list(dev_packs), g=g)
    assert len(Ys) == len(Ws)
    for i, (Y, (codes, scales, zeros)) in enumerate(zip(Ys, host_packs)):
        assert Y.shape == (X.shape[0], Ws[i].shape[0])
        if Ws[i].shape[0] == 0:
            continue
        Yref, B = orc.w4a16_ref(X, codes, scales, zeros, g=g)
        check_gemm(host(Y), Yref, B, f"{what} layer {i}")


def test_decode_workload_one_launch(orc):
    """The decode workload's two layers (N = 11008 and 4096) share X."""
    w11, w4 = workloads.decode(11008), workloads.decode(4096)
    assert np.array_equal(w11["X"], w4["X"])
    run_multi(orc, w11["X"], [w11["W"], w4["W"]], 128, [False, False], "decode multi")


# (M, [N_i], K): the total block count picks 16, 8 or 4 wavefronts per block
# and 2, 4 or 8 k-blocks per wavefront; ragged N; a layer with N = 0.
SHAPES = [(1, [300, 17, 1000], 1024), (1, [11008, 4096, 4096], 4096), (3, [64, 0, 129], 2048),
          (7, [1000, 2000], 4096), (16, [500, 700], 4096), (2, [33] * 8, 8192), (1, [5], 256)]


@pytest.mark.parametrize("M,Ns,K", SHAPES)
@pytest.mark.parametrize("sym", [False, True])
def test_shapes(orc, M, Ns, K, sym):
    seed = M * 101 + K + sum(Ns) + int(sym)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 50, M, 1, K)
    run_multi(orc, X, Ws, 128, [sym] * len(Ns), f"multi M={M} Ns={Ns} K={K} sym={sym}")


@pytest.mark.parametrize("M,Ns,K,g,syms", [
    (20, [100, 200], 1024, 128, [False, False]),      # M > 16
    (64, [130, 7], 512, 128, [True, True]),
    (1, [256, 300], 512, 256, [False, False]),        # g = 256
    (1, [256, 300], 512, 64, [False, False]),         # g = 64 and 32: small-group kernel
    (5, [100, 77], 384, 32, [True, True]),
    (2, [300, 17], 1024, 128, [False, True]),         # mixed symmetric / asymmetric
])
def test_fallback_one_launch_per_layer(orc, M, Ns, K, g, syms):
    seed = M * 7 + K + g + sum(Ns)
    Ws = [workloads.small_case(seed + i, 1, N, K)[0] for i, N in enumerate(Ns)]
    _, X = workloads.small_case(seed + 50, M, 1, K)
    run_multi(orc, X, Ws, g, syms, f"multi fallback M={M} Ns={Ns} K={K} g={g}")


def test_out_argument_and_empty(orc):
    W, X = workloads.small_case(5, 2, 40, 512)
    _, dev = packed(orc, W, 128, False)
    Y = torch.full((2, 40), 7.0, dtype=torch.float16, device="cuda")
    (Yo,) = q4.w4a16_linear_multi(gpu(X), [dev], out=[Y])
    assert Yo.data_ptr() == Y.data_ptr()
    ref = q4.w4a16_linear(gpu(X), *dev)
    assert torch.equal(Y, ref)    # one layer, same launch configuration
    assert q4.w4a16_linear_multi(gpu(X), []) == []
    (Ye,) = q4.w4a16_linear_multi(gpu(X)[:0], [dev])
    assert Ye.shape == (0, 40)
    with pytest.raises(ValueError):
        q4.w4a16_linear_multi(gpu(X), [dev], out=[torch.empty((2, 41), dtype=torch.float16, device="cuda")])
