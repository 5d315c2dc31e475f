"""The C-ABI library loads, exports every symbol include/q4.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: every
call here fails validation or is a zero-size no-op, so nothing is launched).
"""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_gemm_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"Q4_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q4.LIB_PATH):
        from quantized_gemm_q4_amd import build
        build.build()
    return q4.lib()


def test_header_declares_the_binding(lib):
    names = declared_functions()
    assert names == sorted(q4.SIGNATURES), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", q4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported
    # nothing else of ours leaks out (internal launchers are hidden)
    ours = {s for s in exported if s.startswith(("q4", "w4a16", "w8a8", "q8", "fp8", "mxfp4", "nf4", "nvfp4", "awq", "smoothquant", "layernorm", "_ZN3q4k"))}
    assert ours == set(declared_functions())


def test_layout_version_and_workspace(lib):
    assert lib.q4_layout_version() == 1
    assert lib.w8a8_workspace_bytes(2048, 8192) == 2048 * 8192 + 2048 * 4
    assert lib.w8a8_workspace_bytes(3, 16) == 256 + 12
    assert lib.w8a8_workspace_bytes(0, 16) == 0
    assert lib.w4a16_awq_workspace_bytes(1, 4096) == 8192
    assert lib.w4a16_awq_workspace_bytes(3, 24) == 256
    assert lib.w4a16_awq_workspace_bytes(0, 128) == 0
    # the no-allocation scratch array holds the W8A8 workload's codes and scales
    assert lib.w8a8_noalloc_max_bytes() == 16 * 1024 * 1024 + 64 * 1024
    assert lib.w8a8_workspace_bytes(2048, 8192) <= lib.w8a8_noalloc_max_bytes()
    assert lib.w8a8_workspace_bytes(2100, 8192) > lib.w8a8_noalloc_max_bytes()


FAKE = 0x10000          # never dereferenced: validation fails first
MISAL = 0x10001


def layers(*descs):
    """A q4_w4a16_layer array from (codes, scales, zeros, Y, N) tuples."""
    table = (q4.W4A16Layer * len(descs))()
    for i, d in enumerate(descs):
        table[i] = q4.W4A16Layer(*d)
    return table


@pytest.mark.parametrize("call,status", [
    # bad group size / shape
    (lambda L: L.q4_quantize_pack(FAKE, 4, 512, 100, 0, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.q4_quantize_pack(FAKE, 4, 500, 128, 0, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.q4_quantize_pack(FAKE, -1, 512, 128, 0, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.q4_quantize_pack(FAKE, 4, 512, 128, 0, FAKE, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.q4_quantize_pack(None, 4, 512, 128, 1, FAKE, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.q4_quantize_pack(MISAL, 4, 512, 128, 1, FAKE, FAKE, None, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.q4_quantize_pack(FAKE, 0, 512, 128, 0, None, None, None, None), q4.Q4_OK),
    # group sizes must be multiples of 32 (32, 64, 128, 256, 384, ... are served)
    (lambda L: L.w4a16_linear(FAKE, 1, 16, 480, 80, FAKE, FAKE, FAKE, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.w4a16_linear(FAKE, 1, 16, 512, 0, FAKE, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear(FAKE, 65535 * 128 + 1, 16, 512, 128, FAKE, FAKE, FAKE, FAKE, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.w4a16_linear(FAKE, 1, 16, 500, 128, FAKE, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear(MISAL, 1, 16, 512, 128, FAKE, FAKE, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w4a16_linear(FAKE, 1, 16, 512, 128, MISAL, FAKE, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w4a16_linear(FAKE, 1, 16, 512, 128, None, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear(FAKE, 0, 16, 512, 128, None, None, None, None, None), q4.Q4_OK),
    (lambda L: L.w4a16_linear(FAKE, 3, 0, 512, 128, None, None, None, None, None), q4.Q4_OK),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 512, 128, layers((FAKE, FAKE, FAKE, FAKE, 16)), 9, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 512, 128, None, 1, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 480, 80, layers((FAKE, FAKE, FAKE, FAKE, 16)), 1, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 500, 128, layers((FAKE, FAKE, FAKE, FAKE, 16)), 1, None),
     q4.Q4_ERR_INVALID_ARG),
    # the second layer is checked before anything runs
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 512, 128, layers((FAKE, FAKE, FAKE, FAKE, 16),
                                                                (MISAL, FAKE, FAKE, FAKE, 16)), 2, None),
     q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 512, 128, layers((FAKE, FAKE, FAKE, FAKE, 16),
                                                                (None, FAKE, FAKE, FAKE, 16)), 2, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 512, 128, layers((FAKE, FAKE, FAKE, FAKE, -1)), 1, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_multi(FAKE, 1, 512, 128, None, 0, None), q4.Q4_OK),
    (lambda L: L.w4a16_linear_multi(FAKE, 0, 512, 128, layers((None, None, None, None, 16)), 1, None),
     q4.Q4_OK),
    (lambda L: L.w4a16_linear_multi(FAKE, 2, 512, 128, layers((None, None, None, None, 0)), 1, None),
     q4.Q4_OK),
    (lambda L: L.q8_quantize_weight(FAKE, None, 4, 100, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.q8_quantize_weight(FAKE, MISAL, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.q8_quantize_act(FAKE, None, 4, 128, MISAL, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.q8_quantize_act(FAKE, None, 4, 128, None, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.layernorm_quant_smooth(FAKE, FAKE, FAKE, None, 1e-5, 4, 100, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.layernorm_quant_smooth(FAKE, FAKE, FAKE, None, 0.0, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.layernorm_quant_smooth(FAKE, FAKE, FAKE, None, float("nan"), 4, 128, FAKE, FAKE, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.layernorm_quant_smooth(FAKE, FAKE, FAKE, None, 1e-5, 4, 8200, FAKE, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.layernorm_quant_smooth(FAKE, None, FAKE, None, 1e-5, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.layernorm_quant_smooth(FAKE, FAKE, MISAL, None, 1e-5, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.layernorm_quant_smooth(FAKE, FAKE, FAKE, MISAL, 1e-5, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.layernorm_quant_smooth(None, None, None, None, 1e-5, 0, 128, None, None, None), q4.Q4_OK),
    (lambda L: L.layernorm_quant_smooth_fp8(FAKE, FAKE, FAKE, None, 1e-5, 4, 8200, FAKE, FAKE, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.layernorm_quant_smooth_fp8(FAKE, FAKE, FAKE, None, -1.0, 4, 128, FAKE, FAKE, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.layernorm_quant_smooth_fp8(FAKE, FAKE, FAKE, None, 1e-5, 4, 128, MISAL, FAKE, None),
     q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w8a8_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w8a8_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 140000, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w8a8_gemm(MISAL, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, None, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w8a8_linear(FAKE, 4, 4, 128, FAKE, FAKE, None, FAKE, FAKE, 100, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w8a8_linear(FAKE, 4, 4, 128, FAKE, FAKE, None, FAKE, FAKE + 16, 4096, None, None), q4.Q4_ERR_MISALIGNED),
    # the GEMM's own preconditions are checked before the activation quantizer
    # would launch: a misaligned Wq, a too large M, a null w_scale
    (lambda L: L.w8a8_linear(FAKE, 4, 4, 128, MISAL, FAKE, None, FAKE, FAKE, 4096, None, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w8a8_linear(FAKE, 65535 * 128 + 1, 4, 128, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.w8a8_linear(FAKE, 4, 4, 128, FAKE, None, None, FAKE, FAKE, 4096, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w8a8_linear(MISAL, 4, 4, 128, FAKE, FAKE, None, FAKE, FAKE, 4096, None, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w8a8_linear(FAKE, 4, 4, 128, FAKE, FAKE, MISAL, FAKE, FAKE, 4096, None, None), q4.Q4_ERR_MISALIGNED),
    # the no-allocation entry point refuses before it touches the device
    (lambda L: L.w8a8_linear_noalloc(FAKE, 4, 4, 100, FAKE, FAKE, None, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w8a8_linear_noalloc(FAKE, 2100, 4, 8192, FAKE, FAKE, None, FAKE, None, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.w8a8_linear_noalloc(FAKE, 4, 4, 128, MISAL, FAKE, None, FAKE, None, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w8a8_linear_noalloc(FAKE, 4, 4, 128, FAKE, None, None, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w8a8_linear_noalloc(FAKE, 0, 4, 128, None, None, None, None, None, None), q4.Q4_OK),
    (lambda L: L.fp8_quantize_weight(FAKE, None, 4, 100, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.fp8_quantize_weight(FAKE, MISAL, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.fp8_quantize_act(FAKE, None, 4, 128, MISAL, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.fp8_quantize_act(FAKE, None, 4, 128, None, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.fp8_quantize_act(FAKE, None, 0, 128, None, None, None), q4.Q4_OK),
    (lambda L: L.fp8_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 200, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.fp8_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 8320, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.fp8_gemm(MISAL, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.fp8_gemm(FAKE, FAKE, None, FAKE, 4, 4, 128, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.fp8_gemm(FAKE, FAKE, FAKE, FAKE, 0, 4, 128, FAKE, None), q4.Q4_OK),
    (lambda L: L.fp8_gemm(FAKE, FAKE, FAKE, FAKE, 1 << 18, 4, 8192, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 4, 1 << 18, 8192, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.fp8_linear(FAKE, 4, 4, 128, FAKE, FAKE, None, FAKE, FAKE, 100, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.fp8_linear(FAKE, 4, 4, 128, FAKE, FAKE, None, FAKE, FAKE + 16, 4096, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.fp8_linear(FAKE, 4, 4, 96, FAKE, FAKE, None, FAKE, FAKE, 4096, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.fp8_linear(FAKE, 4, 4, 128, MISAL, FAKE, None, FAKE, FAKE, 4096, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.fp8_linear(FAKE, 1 << 18, 4, 8192, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.mxfp4_linear(FAKE, 4, 4, 128, MISAL, FAKE, None, FAKE, FAKE, 4096, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.mxfp4_linear(FAKE, 4, 1 << 18, 8192, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.mxfp4_linear(FAKE, 4, 4, 128, FAKE, None, None, FAKE, FAKE, 4096, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.mxfp4_quantize_weight(FAKE, None, 4, 48, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.mxfp4_quantize_weight(MISAL, None, 4, 64, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.mxfp4_quantize_weight(FAKE, None, 4, 64, FAKE + 2, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.mxfp4_quantize_weight(FAKE, None, 4, 64, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.mxfp4_quantize_weight(FAKE, None, 0, 64, None, None, None), q4.Q4_OK),
    (lambda L: L.mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 192, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.mxfp4_gemm(FAKE, FAKE, FAKE, FAKE, 4, 4, 8320, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.mxfp4_gemm(FAKE, FAKE, MISAL, FAKE, 4, 4, 128, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.mxfp4_gemm(FAKE, FAKE, FAKE, None, 4, 4, 128, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.mxfp4_linear(FAKE, 4, 4, 128, FAKE, FAKE, None, FAKE, FAKE, 100, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.mxfp4_linear(FAKE, 4, 0, 128, None, None, None, None, None, 0, None), q4.Q4_OK),
    (lambda L: L.nf4_quantize(FAKE, 4, 96, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nf4_quantize(MISAL, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.nf4_quantize(FAKE, 0, 128, None, None, None), q4.Q4_OK),
    (lambda L: L.nf4_linear(FAKE, 1, 16, 192, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nf4_linear(FAKE, 1, 16, 1 << 31, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nf4_linear(FAKE, 1, 1 << 20, 1 << 14, FAKE, FAKE, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.nf4_linear(FAKE, 1, 16, 256, FAKE, FAKE + 4, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.nf4_linear(FAKE, 1, 16, 256, None, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nf4_linear(FAKE, 0, 16, 256, None, None, None, None), q4.Q4_OK),
    (lambda L: L.nvfp4_quantize(FAKE, 4, 40, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nvfp4_quantize(MISAL, 4, 128, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.nvfp4_quantize(FAKE, 4, 128, FAKE + 2, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.nvfp4_quantize(FAKE, 0, 128, None, None, None), q4.Q4_OK),
    (lambda L: L.nvfp4_quantize(FAKE, 4, 128, FAKE, None, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nvfp4_linear(FAKE, 1, 16, 192, FAKE, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nvfp4_linear(FAKE, 1, 1 << 20, 1 << 14, FAKE, FAKE, FAKE, None), q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.nvfp4_linear(FAKE, 1, 16, 256, FAKE, FAKE + 1, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.nvfp4_linear(FAKE, 1, 16, 256, FAKE + 8, FAKE, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.nvfp4_linear(FAKE, 1, 16, 256, None, FAKE, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.nvfp4_linear(FAKE, 0, 16, 256, None, None, None, None), q4.Q4_OK),
    (lambda L: L.awq_scale_weight(FAKE, FAKE, 4, 12, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.awq_scale_weight(FAKE, None, 4, 16, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.awq_scale_weight(MISAL, FAKE, 4, 16, FAKE, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.awq_scale_act(FAKE, FAKE + 4, 4, 16, FAKE + 256, None), q4.Q4_ERR_MISALIGNED),
    (lambda L: L.awq_scale_act(FAKE, FAKE, 4, 16, FAKE + 64, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.awq_scale_act(FAKE, FAKE, 0, 16, FAKE, None), q4.Q4_OK),
    (lambda L: L.w4a16_linear_awq(FAKE, 1, 16, 256, 128, FAKE, FAKE, None, None, FAKE, FAKE, 512, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_awq(FAKE, 1, 16, 256, 128, FAKE, FAKE, None, FAKE, FAKE, FAKE, 256, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_awq(FAKE, 1, 16, 256, 128, FAKE, FAKE, None, FAKE, FAKE, None, 512, None),
     q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.w4a16_linear_awq(FAKE, 1, 16, 480, 80, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1024, None),
     q4.Q4_ERR_UNSUPPORTED),
    (lambda L: L.w4a16_linear_awq(FAKE, 1, 16, 256, 128, FAKE, FAKE, None, MISAL, FAKE, FAKE, 512, None),
     q4.Q4_ERR_MISALIGNED),
    (lambda L: L.w4a16_linear_awq(FAKE, 0, 16, 256, 128, None, None, None, None, None, None, 0, None),
     q4.Q4_OK),
    (lambda L: L.smoothquant_scales(FAKE, 4, FAKE, 4, 128, 1.5, FAKE, None), q4.Q4_ERR_INVALID_ARG),
    (lambda L: L.smoothquant_scales(FAKE, 0, FAKE, 4, 128, 0.5, FAKE, None), q4.Q4_ERR_INVALID_ARG),
])
def test_host_validation(lib, call, status):
    assert call(lib) == status
    msg = lib.q4_last_error().decode()
    assert (msg == "") == (status == q4.Q4_OK)


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        q4.w4a16_linear(torch.zeros(1, 128, dtype=torch.float16),
                        torch.zeros(4, 64, dtype=torch.uint8),
                        torch.zeros(4, 1, dtype=torch.float16), None)
    with pytest.raises(ValueError):
        q4.w4a16_linear_multi(torch.zeros(1, 128, dtype=torch.float16),
                              [(torch.zeros(4, 64, dtype=torch.uint8),
                                torch.zeros(4, 1, dtype=torch.float16), None)])


def test_nf4_levels_match_the_oracle(lib, orc):
    """The library's level table (constants in the HIP source) equals the
    oracle's, computed from the guide's formula with the normal quantile."""
    import numpy as np
    assert np.array_equal(q4.nf4_levels().view(np.uint16), orc.nf4_levels().view(np.uint16))
