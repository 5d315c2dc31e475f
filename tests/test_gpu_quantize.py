"""GPU parity of the INT4 quantize + pack kernel: codes, scales and
zero-points bit for bit against the oracle, on small ragged shapes, on groups
covering every fp16 value of several ranges, on degenerate groups and on the
full-size weights of the quantize and prefill workloads."""
import numpy as np
import pytest

import quantized_gemm_q4_amd as q4
import workloads
from parity import gpu, host
from test_oracle_q4 import ASYM_RANGES, FINITE_H, groups_from_values

pytestmark = pytest.mark.gpu


def run_both(orc, W, g, sym):
    c_ref, s_ref, z_ref = orc.q4_quantize_pack(W, g=g, sym=sym)
    c, s, z = q4.q4_quantize_pack(gpu(W), g=g, sym=sym)
    assert np.array_equal(host(c), c_ref), "codes differ"
    assert np.array_equal(host(s).view(np.uint16), s_ref.view(np.uint16)), "scales differ"
    if sym:
        assert z is None
    else:
        assert np.array_equal(host(z), z_ref), "zeros differ"


def test_tiny_workload(orc):
    w = workloads.tiny()
    run_both(orc, w["W"], w["g"], w["sym"])


@pytest.mark.parametrize("N,K,g", [(1, 32, 32), (7, 96, 32), (33, 640, 64), (5, 192, 64),
                                   (100, 384, 128), (3, 640, 128), (257, 1152, 128),
                                   (2, 4096 + 128, 128), (9, 2048 * 3, 64)])
@pytest.mark.parametrize("sym", [False, True])
def test_ragged_shapes(orc, N, K, g, sym):
    rng = np.random.default_rng(N * 1000 + K + g)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    run_both(orc, W, g, sym)


@pytest.mark.parametrize("lo,hi", ASYM_RANGES)
def test_every_fp16_value_asym(orc, lo, hi):
    lo16, hi16 = np.float32(np.float16(lo)), np.float32(np.float16(hi))
    vals = FINITE_H[(FINITE_H >= lo16) & (FINITE_H <= hi16)]
    run_both(orc, groups_from_values(vals, [lo16, hi16]), 128, False)


@pytest.mark.parametrize("amax", [1.0, 0.37, 3.2, 2.0 ** -13, 5e-7, 65504.0, 0.06])
def test_every_fp16_value_sym(orc, amax):
    a16 = np.float32(np.float16(amax))
    vals = FINITE_H[np.abs(FINITE_H) <= a16]
    run_both(orc, groups_from_values(vals, [a16, -a16]), 128, True)


def test_degenerate_groups(orc):
    W = np.zeros((6, 512), np.float16)
    W[1, :128] = 0.5
    W[2, 128:256] = -0.25
    W[3, :] = np.float16(2.0 ** -24)
    W[4, ::2] = np.float16(-65504.0)
    W[4, 1::2] = np.float16(65504.0)
    W[5, 256:384] = np.float16(3e-5)
    for sym in (False, True):
        for g in (32, 64, 128):
            run_both(orc, W, g, sym)


def test_quant_workload_full(orc):
    w = workloads.quant()
    run_both(orc, w["W"], w["g"], w["sym"])


def test_prefill_weight_full(orc):
    w = workloads.prefill()
    run_both(orc, w["W"], w["g"], w["sym"])


def test_zero_rows_noop():
    import torch
    W = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    c, s, z = q4.q4_quantize_pack(W)
    assert c.shape == (0, 128) and s.shape == (0, 2)
