"""MI355X (gfx950) group-quantized linear layers: W4A16 and SmoothQuant W8A8.

Thin Python binding of the C ABI in ``include/q4.h`` (library
``libq4amd.so`` in this directory). This module only marshals arguments:
PyTorch supplies device memory and the current HIP stream; every step of
the computation runs in the library's HIP kernels. If the library is not
built, every call raises -- there is no fallback path.

Functions (same names as the C ABI):
  q4_quantize_pack(W, g=128, sym=False) -> (codes, scales, zeros | None)
  w4a16_linear(X, codes, scales, zeros, g=128) -> Y
  w4a16_linear_multi(X, [(codes, scales, zeros), ...], g=128) -> [Y, ...]
  q8_quantize_weight(W, smooth_s=None) -> (Wq, w_scale)
  q8_quantize_act(X, smooth_s=None) -> (Xq, x_scale)
  layernorm_quant_smooth(X, gamma, beta, smooth_s=None, eps=1e-5) -> (Xq, x_scale)
  layernorm_quant_smooth_fp8(X, gamma, beta, smooth_s=None, eps=1e-5) -> (Xq E4M3, x_scale)
  w8a8_gemm(Xq, x_scale, Wq, w_scale, acc_out=None) -> Y
  w8a8_linear(X, Wq, w_scale, smooth_s=None, workspace=None, acc_out=None) -> Y
  w8a8_linear_noalloc(X, Wq, w_scale, smooth_s=None, acc_out=None) -> Y  (no workspace)
  smoothquant_scales(Xcal, W, alpha=0.5) -> s
  fp8_quantize_weight(W, smooth_s=None) -> (Wq, w_scale)      E4M3 codes as uint8
  fp8_quantize_act(X, smooth_s=None) -> (Xq, x_scale)
  fp8_gemm(Xq, x_scale, Wq, w_scale) -> Y
  fp8_linear(X, Wq, w_scale, smooth_s=None, workspace=None) -> Y
  mxfp4_quantize_weight(W, smooth_s=None) -> (codes, scales)  E2M1 + E8M0 per 32
  mxfp4_gemm(Xq, x_scale, codes, scales) -> Y                 W4A8
  mxfp4_linear(X, codes, scales, smooth_s=None, workspace=None) -> Y
  nf4_levels() -> 16 fp16 levels (host)
  nf4_quantize(W) -> (codes, scales)                         absmax per 64
  nf4_linear(X, codes, scales) -> Y
  nvfp4_quantize(W) -> (codes, scales)                       E4M3 scale per 16
  nvfp4_linear(X, codes, scales) -> Y
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4amd.so")

Q4_OK, Q4_ERR_INVALID_ARG, Q4_ERR_UNSUPPORTED, Q4_ERR_MISALIGNED, Q4_ERR_HIP = range(5)
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "MISALIGNED", 4: "HIP"}

# name -> (restype, argtypes), exactly the declarations of include/q4.h
_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32


class W4A16Layer(ctypes.Structure):
    """q4_w4a16_layer: one layer of w4a16_linear_multi."""
    _fields_ = [("codes", _vp), ("scales", _vp), ("zeros", _vp), ("Y", _vp), ("N", _i64)]


MAX_MULTI_LAYERS = 8
SIGNATURES = {
    "q4_layout_version": (ctypes.c_int, []),
    "q4_last_error": (ctypes.c_char_p, []),
    "q4_quantize_pack": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "w4a16_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp]),
    "w4a16_linear_multi": (ctypes.c_int, [_vp, _i64, _i64, _i32, ctypes.POINTER(W4A16Layer), _i32, _vp]),
    "awq_scale_weight": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "awq_scale_act": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "w4a16_awq_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "w4a16_linear_awq": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]),
    "q8_quantize_weight": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "q8_quantize_act": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "layernorm_quant_smooth": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_double, _i64, _i64, _vp, _vp, _vp]),
    "layernorm_quant_smooth_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_double, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "w8a8_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                                   ctypes.c_size_t, _vp, _vp]),
    "w8a8_noalloc_max_bytes": (ctypes.c_size_t, []),
    "w8a8_linear_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "smoothquant_scales": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, ctypes.c_float, _vp, _vp]),
    "fp8_quantize_weight": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "fp8_quantize_act": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "fp8_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "fp8_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "mxfp4_quantize_weight": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "mxfp4_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "mxfp4_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "nf4_levels": (None, [_vp]),
    "nf4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "nf4_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "nvfp4_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
}

_lib = None


class Q4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libq4amd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m quantized_gemm_q4_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _empty(shape, dtype, device):
    """Every buffer this binding allocates for the caller (outputs,
    workspaces) comes from here."""
    return torch.empty(shape, dtype=dtype, device=device)


def _check(status: int):
    if status != Q4_OK:
        raise Q4Error(status, lib().q4_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype, name: str, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def layout_version() -> int:
    return int(lib().q4_layout_version())


def q4_quantize_pack(W: torch.Tensor, g: int = 128, sym: bool = False, out=None):
    """Group-wise RTN INT4 of W fp16 [N, K]: (codes u8 [N, K/2],
    scales fp16 [N, K/g], zeros u8 [N, ceil(K/g/2)] or None when sym)."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    G = K // g if g > 0 else 0
    if out is None:
        codes = _empty((N, K // 2), dtype=torch.uint8, device=W.device)
        scales = _empty((N, G), dtype=torch.float16, device=W.device)
        zeros = None if sym else _empty((N, (G + 1) // 2), dtype=torch.uint8, device=W.device)
    else:
        codes, scales, zeros = out
        # the kernel writes whole rows of each: every buffer must be exactly the
        # packed shape, on W's device, contiguous
        _need(codes, torch.uint8, "codes", 2)
        _need(scales, torch.float16, "scales", 2)
        want = {"codes": (codes, (N, K // 2)), "scales": (scales, (N, G))}
        if zeros is not None:
            _need(zeros, torch.uint8, "zeros", 2)
            want["zeros"] = (zeros, (N, (G + 1) // 2))
        elif not sym:
            raise ValueError("zeros must be given when sym is False")
        for name, (t, shape) in want.items():
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} {tuple(t.shape)} does not match {shape} for W {tuple(W.shape)}, g={g}")
            if t.device != W.device:
                raise ValueError(f"{name} is on {t.device}, W on {W.device}")
    _check(lib().q4_quantize_pack(_ptr(W), N, K, g, int(bool(sym)), _ptr(codes), _ptr(scales),
                                  _ptr(zeros), _stream(W)))
    return codes, scales, zeros


def w4a16_linear(X: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor | None, g: int = 128, out: torch.Tensor | None = None):
    """Y fp16 [M, N] = X fp16 [M, K] x W_hat^T, W_hat dequantized in the GEMM."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    N = _check_packed(codes, scales, zeros, K, g)
    Y = _output(out, M, N, X.device)
    _check(lib().w4a16_linear(_ptr(X), M, N, K, g, _ptr(codes), _ptr(scales), _ptr(zeros),
                              _ptr(Y), _stream(X)))
    return Y


def _check_packed(codes, scales, zeros, K: int, g: int, what: str = "") -> int:
    """Shapes of one packed weight [N, K] as q4_quantize_pack writes it; returns N."""
    _need(codes, torch.uint8, what + "codes", 2)
    _need(scales, torch.float16, what + "scales", 2)
    if zeros is not None:
        _need(zeros, torch.uint8, what + "zeros", 2)
    N = codes.shape[0]
    if codes.shape[1] * 2 != K:
        raise ValueError(f"{what}codes {tuple(codes.shape)} does not match K={K}")
    if g <= 0 or scales.shape != (N, K // g):
        raise ValueError(f"{what}scales {tuple(scales.shape)} does not match [N, K/g]=[{N}, {K // max(g, 1)}]")
    if zeros is not None and zeros.shape != (N, (K // g + 1) // 2):
        raise ValueError(f"{what}zeros {tuple(zeros.shape)} does not match [N, ceil(K/g/2)]")
    return N


def _output(out, M: int, N: int, device):
    if out is None:
        return _empty((M, N), dtype=torch.float16, device=device)
    _need(out, torch.float16, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out {tuple(out.shape)} does not match [M, N]=[{M}, {N}]")
    if out.device != torch.device(device):
        raise ValueError(f"out is on {out.device}, the input on {device}")
    return out


def w4a16_linear_multi(X: torch.Tensor, layers, g: int = 128, out=None):
    """Y_i fp16 [M, N_i] = X x W_hat_i^T for every packed weight
    (codes, scales, zeros) in `layers`, all reading the same X; one launch
    when the shapes allow it (M <= 16, g = 128, all layers sym or all asym)."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    layers = list(layers)
    if len(layers) > MAX_MULTI_LAYERS:
        raise ValueError(f"at most {MAX_MULTI_LAYERS} layers per call, got {len(layers)}")
    if out is not None and len(out) != len(layers):
        raise ValueError("out must hold one tensor per layer")
    table = (W4A16Layer * max(len(layers), 1))()
    Ys = []
    for i, (codes, scales, zeros) in enumerate(layers):
        N = _check_packed(codes, scales, zeros, K, g, f"layer {i}: ")
        Y = _output(None if out is None else out[i], M, N, X.device)
        table[i] = W4A16Layer(_ptr(codes), _ptr(scales), _ptr(zeros), _ptr(Y), N)
        Ys.append(Y)
    _check(lib().w4a16_linear_multi(_ptr(X), M, K, g, table, len(layers), _stream(X)))
    return Ys


# --- AWQ-style per-input-channel scaling (W4A16) -------------------------------

def _need_awq(awq_s, K: int):
    _need(awq_s, torch.float32, "awq_s", 1)
    if awq_s.numel() != K:
        raise ValueError(f"awq_s has {awq_s.numel()} entries, K={K}")


def awq_scale_weight(W: torch.Tensor, awq_s: torch.Tensor, out: torch.Tensor | None = None):
    """W'' fp16 [N, K] = f2h(W * awq_s[k]); quantize it with q4_quantize_pack.
    out may be W itself."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    _need_awq(awq_s, K)
    Ws = _output(out, N, K, W.device)
    _check(lib().awq_scale_weight(_ptr(W), _ptr(awq_s), N, K, _ptr(Ws), _stream(W)))
    return Ws


def awq_scale_act(X: torch.Tensor, awq_s: torch.Tensor, out: torch.Tensor | None = None):
    """X'' fp16 [M, K] = f2h(X / awq_s[k]). out may be X itself."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    _need_awq(awq_s, K)
    Xs = _output(out, M, K, X.device)
    _check(lib().awq_scale_act(_ptr(X), _ptr(awq_s), M, K, _ptr(Xs), _stream(X)))
    return Xs


def w4a16_awq_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w4a16_awq_workspace_bytes(M, K))


def w4a16_linear_awq(X: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                     zeros: torch.Tensor | None, awq_s: torch.Tensor, g: int = 128,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Y fp16 [M, N] = (X / awq_s) x W_hat^T for the packed AWQ-scaled weight;
    the division is fused into the decode GEMV when M == 1."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    N = _check_packed(codes, scales, zeros, K, g)
    _need_awq(awq_s, K)
    if workspace is None:
        workspace = _empty((max(w4a16_awq_workspace_bytes(M, K), 1),), dtype=torch.uint8,
                                device=X.device)
    _need(workspace, torch.uint8, "workspace", 1)
    Y = _output(out, M, N, X.device)
    _check(lib().w4a16_linear_awq(_ptr(X), M, N, K, g, _ptr(codes), _ptr(scales), _ptr(zeros),
                                  _ptr(awq_s), _ptr(Y), _ptr(workspace), workspace.numel(),
                                  _stream(X)))
    return Y


def _need_smooth(smooth_s, K: int):
    if smooth_s is not None:
        _need(smooth_s, torch.float32, "smooth_s", 1)
        if smooth_s.numel() != K:
            raise ValueError(f"smooth_s has {smooth_s.numel()} entries, K={K}")


def _row_outputs(out, rows: int, K: int, code_dtype, device):
    if out is None:
        return (_empty((rows, K), dtype=code_dtype, device=device),
                _empty((rows,), dtype=torch.float32, device=device))
    q, sc = out
    _need(q, code_dtype, "codes", 2)
    _need(sc, torch.float32, "scale", 1)
    if tuple(q.shape) != (rows, K) or sc.numel() != rows:
        raise ValueError("out tensors do not match the input's shape")
    if q.device != torch.device(device) or sc.device != torch.device(device):
        raise ValueError("out tensors must be on the input's device")
    return q, sc


def q8_quantize_weight(W: torch.Tensor, smooth_s: torch.Tensor | None = None):
    """Per-output-channel INT8 of W diag(s): (Wq int8 [N, K], w_scale fp32 [N])."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    _need_smooth(smooth_s, K)
    Wq = _empty((N, K), dtype=torch.int8, device=W.device)
    sw = _empty((N,), dtype=torch.float32, device=W.device)
    _check(lib().q8_quantize_weight(_ptr(W), _ptr(smooth_s), N, K, _ptr(Wq), _ptr(sw), _stream(W)))
    return Wq, sw


def q8_quantize_act(X: torch.Tensor, smooth_s: torch.Tensor | None = None, out=None):
    """Per-token dynamic INT8 of X / s: (Xq int8 [M, K], x_scale fp32 [M])."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    _need_smooth(smooth_s, K)
    Xq, sx = _row_outputs(out, M, K, torch.int8, X.device)
    _check(lib().q8_quantize_act(_ptr(X), _ptr(smooth_s), M, K, _ptr(Xq), _ptr(sx), _stream(X)))
    return Xq, sx


def _layernorm_quant(name: str, code_dtype, X, gamma, beta, smooth_s, eps, out):
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    for pname, t in (("gamma", gamma), ("beta", beta)):
        _need(t, torch.float32, pname, 1)
        if t.numel() != K:
            raise ValueError(f"{pname} has {t.numel()} entries, K={K}")
    _need_smooth(smooth_s, K)
    Xq, sx = _row_outputs(out, M, K, code_dtype, X.device)
    _check(getattr(lib(), name)(_ptr(X), _ptr(gamma), _ptr(beta), _ptr(smooth_s), float(eps), M, K,
                                _ptr(Xq), _ptr(sx), _stream(X)))
    return Xq, sx


def layernorm_quant_smooth(X: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
                           smooth_s: torch.Tensor | None = None, eps: float = 1e-5, out=None):
    """LayerNorm of each row of X with the divide by smooth_s folded into
    gamma and beta, then per-token INT8: (Xq int8 [M, K], x_scale fp32 [M])."""
    return _layernorm_quant("layernorm_quant_smooth", torch.int8, X, gamma, beta, smooth_s, eps, out)


def layernorm_quant_smooth_fp8(X: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
                               smooth_s: torch.Tensor | None = None, eps: float = 1e-5, out=None):
    """The same LayerNorm with per-token FP8 E4M3 codes:
    (Xq E4M3 bytes uint8 [M, K], x_scale fp32 [M])."""
    return _layernorm_quant("layernorm_quant_smooth_fp8", torch.uint8, X, gamma, beta, smooth_s, eps, out)


def w8a8_gemm(Xq: torch.Tensor, x_scale: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
              acc_out: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Y fp16 [M, N] = fp16((Xq Wq^T) * x_scale[m] * w_scale[n]); optional
    int32 accumulator written to acc_out [M, N]."""
    _need(Xq, torch.int8, "Xq", 2)
    _need(Wq, torch.int8, "Wq", 2)
    _need(x_scale, torch.float32, "x_scale", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = Xq.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or x_scale.numel() != M or w_scale.numel() != N:
        raise ValueError("w8a8_gemm: shape mismatch")
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out", 2)
        if acc_out.shape != (M, N):
            raise ValueError("acc_out must be [M, N]")
    Y = _output(out, M, N, Xq.device)
    _check(lib().w8a8_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y),
                           _ptr(acc_out), _stream(Xq)))
    return Y


def w8a8_workspace_bytes(M: int, K: int) -> int:
    return int(lib().w8a8_workspace_bytes(M, K))


def w8a8_workspace(M: int, K: int, device) -> torch.Tensor:
    """A workspace tensor for w8a8_linear (torch's allocations are 256-byte aligned)."""
    return _empty((max(1, w8a8_workspace_bytes(M, K)),), dtype=torch.uint8, device=device)


def w8a8_linear(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
                smooth_s: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                acc_out: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """SmoothQuant W8A8 linear layer: per-token INT8 of X / s, INT8 GEMM,
    fp16 epilogue. smooth_s=None means X is already smoothed."""
    _need(X, torch.float16, "X", 2)
    _need(Wq, torch.int8, "Wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = X.shape
    N = Wq.shape[0]
    _need_smooth(smooth_s, K)
    if Wq.shape[1] != K or w_scale.numel() != N:
        raise ValueError("w8a8_linear: Wq must be [N, K] and w_scale [N]")
    if workspace is None:
        workspace = w8a8_workspace(M, K, X.device)
    _need(workspace, torch.uint8, "workspace", 1)
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out", 2)
        if acc_out.shape != (M, N):
            raise ValueError("acc_out must be [M, N]")
    Y = _output(out, M, N, X.device)
    _check(lib().w8a8_linear(_ptr(X), M, N, K, _ptr(Wq), _ptr(w_scale), _ptr(smooth_s), _ptr(Y),
                             _ptr(workspace), workspace.numel(), _ptr(acc_out), _stream(X)))
    return Y


def w8a8_noalloc_max_bytes() -> int:
    return int(lib().w8a8_noalloc_max_bytes())


def w8a8_linear_noalloc(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
                        smooth_s: torch.Tensor | None = None, acc_out: torch.Tensor | None = None,
                        out: torch.Tensor | None = None):
    """w8a8_linear with the per-token codes and scales in the library's own
    scratch array (no workspace; the C call allocates nothing). Calls that
    overlap on one GPU race on that array."""
    _need(X, torch.float16, "X", 2)
    _need(Wq, torch.int8, "Wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = X.shape
    N = Wq.shape[0]
    _need_smooth(smooth_s, K)
    if Wq.shape[1] != K or w_scale.numel() != N:
        raise ValueError("w8a8_linear_noalloc: Wq must be [N, K] and w_scale [N]")
    if acc_out is not None:
        _need(acc_out, torch.int32, "acc_out", 2)
        if acc_out.shape != (M, N):
            raise ValueError("acc_out must be [M, N]")
    Y = _output(out, M, N, X.device)
    _check(lib().w8a8_linear_noalloc(_ptr(X), M, N, K, _ptr(Wq), _ptr(w_scale), _ptr(smooth_s),
                                     _ptr(Y), _ptr(acc_out), _stream(X)))
    return Y


def smoothquant_scales(Xcal: torch.Tensor, W: torch.Tensor, alpha: float = 0.5):
    """SmoothQuant factor s[K] = max|Xcal_j|^alpha / max|W_j|^(1-alpha)."""
    _need(Xcal, torch.float16, "Xcal", 2)
    _need(W, torch.float16, "W", 2)
    R, K = Xcal.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("smoothquant_scales: Xcal and W must share K")
    s = _empty((K,), dtype=torch.float32, device=W.device)
    _check(lib().smoothquant_scales(_ptr(Xcal), R, _ptr(W), N, K, ctypes.c_float(alpha), _ptr(s),
                                    _stream(W)))
    return s


# --- FP8 E4M3 variant of the W8A8 path ------------------------------------------

def fp8_quantize_weight(W: torch.Tensor, smooth_s: torch.Tensor | None = None, out=None):
    """Per-output-channel E4M3 of W diag(s): (Wq uint8 codes [N, K], w_scale fp32 [N])."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    _need_smooth(smooth_s, K)
    Wq, sw = _row_outputs(out, N, K, torch.uint8, W.device)
    _check(lib().fp8_quantize_weight(_ptr(W), _ptr(smooth_s), N, K, _ptr(Wq), _ptr(sw), _stream(W)))
    return Wq, sw


def fp8_quantize_act(X: torch.Tensor, smooth_s: torch.Tensor | None = None, out=None):
    """Per-token dynamic E4M3 of X / s: (Xq uint8 codes [M, K], x_scale fp32 [M])."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    _need_smooth(smooth_s, K)
    Xq, sx = _row_outputs(out, M, K, torch.uint8, X.device)
    _check(lib().fp8_quantize_act(_ptr(X), _ptr(smooth_s), M, K, _ptr(Xq), _ptr(sx), _stream(X)))
    return Xq, sx


def fp8_gemm(Xq: torch.Tensor, x_scale: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
             out: torch.Tensor | None = None):
    """Y fp16 [M, N] = fp16((e4m3(Xq) e4m3(Wq)^T) * x_scale[m] * w_scale[n]), fp32 sums."""
    _need(Xq, torch.uint8, "Xq", 2)
    _need(Wq, torch.uint8, "Wq", 2)
    _need(x_scale, torch.float32, "x_scale", 1)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = Xq.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or x_scale.numel() != M or w_scale.numel() != N:
        raise ValueError("fp8_gemm: shape mismatch")
    Y = _output(out, M, N, Xq.device)
    _check(lib().fp8_gemm(_ptr(Xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), M, N, K, _ptr(Y),
                          _stream(Xq)))
    return Y


def fp8_linear(X: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor,
               smooth_s: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               out: torch.Tensor | None = None):
    """FP8 E4M3 linear layer: per-token E4M3 of X / s, E4M3 GEMM, fp16 epilogue."""
    _need(X, torch.float16, "X", 2)
    _need(Wq, torch.uint8, "Wq", 2)
    _need(w_scale, torch.float32, "w_scale", 1)
    M, K = X.shape
    N = Wq.shape[0]
    _need_smooth(smooth_s, K)
    if Wq.shape[1] != K or w_scale.numel() != N:
        raise ValueError("fp8_linear: Wq must be [N, K] and w_scale [N]")
    if workspace is None:
        workspace = w8a8_workspace(M, K, X.device)
    _need(workspace, torch.uint8, "workspace", 1)
    Y = _output(out, M, N, X.device)
    _check(lib().fp8_linear(_ptr(X), M, N, K, _ptr(Wq), _ptr(w_scale), _ptr(smooth_s), _ptr(Y),
                            _ptr(workspace), workspace.numel(), _stream(X)))
    return Y


# --- MXFP4 weights with E4M3 activations (W4A8) ---------------------------------

def mxfp4_quantize_weight(W: torch.Tensor, smooth_s: torch.Tensor | None = None):
    """MXFP4 of W diag(s): (codes uint8 [N, K/2], E8M0 scales uint8 [N, K/32])."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    _need_smooth(smooth_s, K)
    codes = _empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = _empty((N, K // 32), dtype=torch.uint8, device=W.device)
    _check(lib().mxfp4_quantize_weight(_ptr(W), _ptr(smooth_s), N, K, _ptr(codes), _ptr(scales),
                                       _stream(W)))
    return codes, scales


def _check_mxfp4(codes, scales, K: int) -> int:
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.uint8, "scales", 2)
    N = codes.shape[0]
    if codes.shape[1] * 2 != K or tuple(scales.shape) != (N, K // 32):
        raise ValueError(f"codes {tuple(codes.shape)} / scales {tuple(scales.shape)} do not match K={K}")
    return N


def mxfp4_gemm(Xq: torch.Tensor, x_scale: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
               out: torch.Tensor | None = None):
    """Y fp16 [M, N] = fp16(x_scale[m] * sum_k e4m3(Xq) e2m1(code) 2^(scale - 127))."""
    _need(Xq, torch.uint8, "Xq", 2)
    _need(x_scale, torch.float32, "x_scale", 1)
    M, K = Xq.shape
    N = _check_mxfp4(codes, scales, K)
    if x_scale.numel() != M:
        raise ValueError("x_scale must have M entries")
    Y = _output(out, M, N, Xq.device)
    _check(lib().mxfp4_gemm(_ptr(Xq), _ptr(x_scale), _ptr(codes), _ptr(scales), M, N, K, _ptr(Y),
                            _stream(Xq)))
    return Y


def mxfp4_linear(X: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                 smooth_s: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None):
    """W4A8 linear layer: per-token E4M3 of X / s, MXFP4 weight, fp16 out."""
    _need(X, torch.float16, "X", 2)
    M, K = X.shape
    N = _check_mxfp4(codes, scales, K)
    _need_smooth(smooth_s, K)
    if workspace is None:
        workspace = w8a8_workspace(M, K, X.device)
    _need(workspace, torch.uint8, "workspace", 1)
    Y = _output(out, M, N, X.device)
    _check(lib().mxfp4_linear(_ptr(X), M, N, K, _ptr(codes), _ptr(scales), _ptr(smooth_s), _ptr(Y),
                              _ptr(workspace), workspace.numel(), _stream(X)))
    return Y


# --- NF4 weights ------------------------------------------------------------------

def nf4_levels():
    """The library's 16 NF4 levels (numpy float16, ascending)."""
    import numpy as np
    out = (ctypes.c_uint16 * 16)()
    lib().nf4_levels(ctypes.cast(out, _vp))
    return np.array(out[:], dtype=np.uint16).view(np.float16)


def nf4_quantize(W: torch.Tensor):
    """NF4 of W fp16 [N, K]: (codes uint8 [N, K/2], scales fp32 [N, K/64])."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    codes = _empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = _empty((N, max(K // 64, 0)), dtype=torch.float32, device=W.device)
    _check(lib().nf4_quantize(_ptr(W), N, K, _ptr(codes), _ptr(scales), _stream(W)))
    return codes, scales


def nf4_linear(X: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None):
    """Y fp16 [M, N] = X W_hat^T with W_hat = level[code] * scale (NF4)."""
    _need(X, torch.float16, "X", 2)
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.float32, "scales", 2)
    M, K = X.shape
    N = codes.shape[0]
    if codes.shape[1] * 2 != K or tuple(scales.shape) != (N, K // 64):
        raise ValueError(f"codes {tuple(codes.shape)} / scales {tuple(scales.shape)} do not match K={K}")
    Y = _output(out, M, N, X.device)
    _check(lib().nf4_linear(_ptr(X), M, N, K, _ptr(codes), _ptr(scales), _ptr(Y), _stream(X)))
    return Y


def nvfp4_quantize(W: torch.Tensor):
    """NVFP4 of W fp16 [N, K]: (codes uint8 [N, K/2], E4M3 scale bytes uint8 [N, K/16])."""
    _need(W, torch.float16, "W", 2)
    N, K = W.shape
    codes = _empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = _empty((N, max(K // 16, 0)), dtype=torch.uint8, device=W.device)
    _check(lib().nvfp4_quantize(_ptr(W), N, K, _ptr(codes), _ptr(scales), _stream(W)))
    return codes, scales


def nvfp4_linear(X: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None):
    """Y fp16 [M, N] = X W_hat^T with W_hat = e2m1(code) * e4m3(scale) (NVFP4)."""
    _need(X, torch.float16, "X", 2)
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.uint8, "scales", 2)
    M, K = X.shape
    N = codes.shape[0]
    if codes.shape[1] * 2 != K or tuple(scales.shape) != (N, K // 16):
        raise ValueError(f"codes {tuple(codes.shape)} / scales {tuple(scales.shape)} do not match K={K}")
    Y = _output(out, M, N, X.device)
    _check(lib().nvfp4_linear(_ptr(X), M, N, K, _ptr(codes), _ptr(scales), _ptr(Y), _stream(X)))
    return Y
