"""CPU oracle for the group-quantized linear layer (NumPy front end).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library in ``quantized_gemm_q4_amd`` and the HIP library never
calls it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE binary32 quantizers, exact
fp64 / int64 GEMM references); this module only marshals NumPy arrays. Each
function names the passage of the quantization pages it follows; the C file
spells the steps out.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, brute-force searches and
independent library routines. No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # ORACLE_LIB names another build of oracle.c (the sanitizer build the
    # test suite runs the oracle's pins against)
    path = os.environ.get("ORACLE_LIB") or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(path)
    sig = {
        "orc_h2f": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f2h": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_h2f_array": (None, [_u16p, _i64, _f32p]),
        "orc_f2h_array": (None, [_f32p, _i64, _u16p]),
        "orc_q4_quantize_pack": (_int, [_u16p, _i64, _i64, _int, _int, _u8p, _u16p, _u8p]),
        "orc_q4_dequant_rows": (None, [_u8p, _u16p, _u8p, _i64, _int, _i64, _i64, _f64p]),
        "orc_w4a16_ref": (None, [_u16p, _i64, _i64, _u8p, _u16p, _u8p, _i64, _int,
                                 _i64p, _i64, _f64p, _f64p]),
        "orc_awq_scale_weight": (None, [_u16p, _f32p, _i64, _i64, _u16p]),
        "orc_awq_scale_act": (None, [_u16p, _f32p, _i64, _i64, _u16p]),
        "orc_q8_quantize_weight": (None, [_u16p, _f32p, _i64, _i64, _i8p, _f32p]),
        "orc_q8_quantize_act": (None, [_u16p, _f32p, _i64, _i64, _i8p, _f32p]),
        "orc_int8_gemm": (_i64, [_i8p, _i64, _i64, _i8p, _i64, _i64p, _i64, _i64p, _i64p]),
        "orc_w8a8_epilogue": (None, [_i64p, _i64p, _f32p, _i64p, _i64, _f32p, _i64,
                                     _f64p, _f64p, _u16p]),
        "orc_smooth_scales": (None, [_u16p, _i64, _u16p, _i64, _i64, ctypes.c_float, _f32p]),
        "orc_e4m3_decode": (ctypes.c_float, [ctypes.c_uint]),
        "orc_e5m2_decode": (ctypes.c_float, [ctypes.c_uint]),
        "orc_e2m1_decode": (ctypes.c_float, [ctypes.c_uint]),
        "orc_e4m3_encode": (ctypes.c_uint, [ctypes.c_float]),
        "orc_fp8_quantize_weight": (None, [_u16p, _f32p, _i64, _i64, _u8p, _f32p]),
        "orc_fp8_quantize_act": (None, [_u16p, _f32p, _i64, _i64, _u8p, _f32p]),
        "orc_fp8_gemm": (None, [_u8p, _i64, _i64, _u8p, _i64, _i64p, _i64, _f64p, _f64p]),
        "orc_e2m1_encode": (ctypes.c_uint, [ctypes.c_float]),
        "orc_mxfp4_quantize_weight": (None, [_u16p, _f32p, _i64, _i64, _u8p, _u8p]),
        "orc_mxfp4_gemm": (None, [_u8p, _i64, _i64, _u8p, _u8p, _i64, _i64p, _i64, _f64p, _f64p]),
        "orc_nf4_quantize": (None, [_u16p, _i64, _i64, _u16p, _u8p, _f32p]),
        "orc_nf4_ref": (None, [_u16p, _i64, _i64, _u8p, _f32p, _u16p, _i64, _i64p, _i64, _f64p, _f64p]),
        "orc_nvfp4_quantize": (None, [_u16p, _i64, _i64, _u8p, _u8p]),
        "orc_nvfp4_ref": (None, [_u16p, _i64, _i64, _u8p, _u8p, _i64, _i64p, _i64, _f64p, _f64p]),
        "orc_layernorm_quant_smooth": (None, [_u16p, _f32p, _f32p, _f32p, ctypes.c_double, _i64, _i64,
                                              _i8p, _f32p, _f32p, _f64p]),
        "orc_layernorm_quant_smooth_fp8": (None, [_u16p, _f32p, _f32p, _f32p, ctypes.c_double, _i64, _i64,
                                                  _u8p, _f32p]),
        "orc_u128_to_double": (ctypes.c_double, [ctypes.c_uint64, ctypes.c_uint64]),
        "orc_num_threads": (_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.cast(None, ctype)
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctype)


def _half_bits(a) -> np.ndarray:
    """fp16 array (np.float16 or its uint16 bit pattern) -> contiguous uint16."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, f"expected fp16 data, got {a.dtype}"
    return np.ascontiguousarray(a)


def _rows(rows):
    if rows is None:
        return None
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


# --- binary16 -------------------------------------------------------------

def h2f(h) -> np.ndarray:
    """binary16 bit patterns -> float32 (IEEE 754 binary16 definition)."""
    h = _half_bits(h)
    out = np.empty(h.shape, np.float32)
    _load().orc_h2f_array(_ptr(h.reshape(-1), _u16p), h.size, _ptr(out.reshape(-1), _f32p))
    return out


def f2h(x) -> np.ndarray:
    """float32 -> binary16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint16)
    _load().orc_f2h_array(_ptr(x.reshape(-1), _f32p), x.size, _ptr(out.reshape(-1), _u16p))
    return out


# --- INT4 group quantizer ---------------------------------------------------

def q4_quantize_pack(W, g: int = 128, sym: bool = False):
    """Group-wise RTN INT4 quantize + pack (Core ideas §2.2; Quantization
    operators guide §2.1, §2.2 per-group; Quantization notes item (1)).

    W: fp16 [N, K]. Returns (codes u8 [N, K/2], scales fp16 [N, K/g],
    zeros u8 [N, ceil(K/g/2)] or None when sym).
    """
    W = _half_bits(W)
    N, K = W.shape
    G = K // g
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, G), np.uint16)
    zeros = None if sym else np.empty((N, (G + 1) // 2), np.uint8)
    rc = _load().orc_q4_quantize_pack(_ptr(W, _u16p), N, K, g, int(bool(sym)),
                                      _ptr(codes, _u8p), _ptr(scales, _u16p),
                                      _ptr(zeros, _u8p))
    if rc != 0:
        raise ValueError(f"oracle rejects shape N={N} K={K} g={g}")
    return codes, scales.view(np.float16), zeros


def q4_dequant(codes, scales, zeros, K: int, g: int = 128, rows=None) -> np.ndarray:
    """w_hat = (u - zp) * s in fp64 (Core ideas §2.2 dequantization)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _half_bits(scales)
    zeros = None if zeros is None else np.ascontiguousarray(zeros, dtype=np.uint8)
    N = codes.shape[0]
    n0, n1 = (0, N) if rows is None else rows
    out = np.empty((n1 - n0, K), np.float64)
    _load().orc_q4_dequant_rows(_ptr(codes, _u8p), _ptr(scales, _u16p), _ptr(zeros, _u8p),
                                K, g, n0, n1, _ptr(out, _f64p))
    return out


def w4a16_ref(X, codes, scales, zeros, g: int = 128, rows=None):
    """fp64 reference of Y = X W_hat^T and the error scale B = |X| |W_hat|^T.

    X: fp16 [M, K]; rows: optional subset of M. Returns (Y, B) as
    [len(rows) or M, N] float64.
    """
    X = _half_bits(X)
    M, K = X.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _half_bits(scales)
    zeros = None if zeros is None else np.ascontiguousarray(zeros, dtype=np.uint8)
    N = codes.shape[0]
    r = _rows(rows)
    n_rows = M if r is None else r.size
    Y = np.empty((n_rows, N), np.float64)
    B = np.empty((n_rows, N), np.float64)
    _load().orc_w4a16_ref(_ptr(X, _u16p), M, K, _ptr(codes, _u8p), _ptr(scales, _u16p),
                          _ptr(zeros, _u8p), N, g, _ptr(r, _i64p), n_rows,
                          _ptr(Y, _f64p), _ptr(B, _f64p))
    return Y, B


# --- AWQ-style per-input-channel scaling (W4A16) -----------------------------

def awq_scale_weight(W, s) -> np.ndarray:
    """w'' = f2h(h2f(W) * s[k]) (fp32 multiply, then binary16). fp16 bits [N, K]."""
    W = _half_bits(W)
    N, K = W.shape
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float32))
    assert s.shape == (K,)
    out = np.empty((N, K), np.uint16)
    _load().orc_awq_scale_weight(_ptr(W, _u16p), _ptr(s, _f32p), N, K, _ptr(out, _u16p))
    return out


def awq_scale_act(X, s) -> np.ndarray:
    """x'' = f2h(h2f(X) / s[k]) (fp32 division, then binary16). fp16 bits [M, K]."""
    X = _half_bits(X)
    M, K = X.shape
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float32))
    assert s.shape == (K,)
    out = np.empty((M, K), np.uint16)
    _load().orc_awq_scale_act(_ptr(X, _u16p), _ptr(s, _f32p), M, K, _ptr(out, _u16p))
    return out


# --- INT8 path ----------------------------------------------------------------

def _smooth(s):
    if s is None:
        return None
    return np.ascontiguousarray(np.asarray(s, dtype=np.float32))


def q8_quantize_weight(W, s=None):
    """Per-output-channel INT8 of W diag(s). Returns (Wq int8 [N,K], sw f32 [N])."""
    W = _half_bits(W)
    N, K = W.shape
    s = _smooth(s)
    Wq = np.empty((N, K), np.int8)
    sw = np.empty(N, np.float32)
    _load().orc_q8_quantize_weight(_ptr(W, _u16p), _ptr(s, _f32p), N, K,
                                   _ptr(Wq, _i8p), _ptr(sw, _f32p))
    return Wq, sw


def q8_quantize_act(X, s=None):
    """Per-token dynamic INT8 of X / s. Returns (Xq int8 [M,K], sx f32 [M])."""
    X = _half_bits(X)
    M, K = X.shape
    s = _smooth(s)
    Xq = np.empty((M, K), np.int8)
    sx = np.empty(M, np.float32)
    _load().orc_q8_quantize_act(_ptr(X, _u16p), _ptr(s, _f32p), M, K,
                                _ptr(Xq, _i8p), _ptr(sx, _f32p))
    return Xq, sx


def int8_gemm(Xq, Wq, rows=None):
    """Exact acc = Xq Wq^T in int64 (+ sum |qx||qw|, + count outside int32)."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    M, K = Xq.shape
    N = Wq.shape[0]
    r = _rows(rows)
    n_rows = M if r is None else r.size
    acc = np.empty((n_rows, N), np.int64)
    aacc = np.empty((n_rows, N), np.int64)
    ovf = _load().orc_int8_gemm(_ptr(Xq, _i8p), M, K, _ptr(Wq, _i8p), N, _ptr(r, _i64p),
                                n_rows, _ptr(acc, _i64p), _ptr(aacc, _i64p))
    return acc, aacc, int(ovf)


def w8a8_epilogue(acc, abs_acc, sx, sw, rows=None):
    """Y = sx sw acc (fp64), its error scale B, and the fp32 expression
    ((float)acc * sx) * sw rounded to fp16 (bit patterns)."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    abs_acc = np.ascontiguousarray(abs_acc, dtype=np.int64)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    r = _rows(rows)
    n_rows, N = acc.shape
    Y = np.empty((n_rows, N), np.float64)
    B = np.empty((n_rows, N), np.float64)
    y16 = np.empty((n_rows, N), np.uint16)
    _load().orc_w8a8_epilogue(_ptr(acc, _i64p), _ptr(abs_acc, _i64p), _ptr(sx, _f32p),
                              _ptr(r, _i64p), n_rows, _ptr(sw, _f32p), N,
                              _ptr(Y, _f64p), _ptr(B, _f64p), _ptr(y16, _u16p))
    return Y, B, y16


def smooth_scales(Xcal, W, alpha: float = 0.5) -> np.ndarray:
    """SmoothQuant s_j = max|X_j|^a / max|W_j|^(1-a) (Quantization operators
    guide §5.1; Core ideas §2.4)."""
    Xcal = _half_bits(Xcal)
    W = _half_bits(W)
    R, K = Xcal.shape
    N, K2 = W.shape
    assert K == K2
    s = np.empty(K, np.float32)
    _load().orc_smooth_scales(_ptr(Xcal, _u16p), R, _ptr(W, _u16p), N, K,
                              ctypes.c_float(alpha), _ptr(s, _f32p))
    return s


# --- small-float formats (Core ideas §2.1) ---------------------------------

def e4m3_decode(code: int) -> float:
    return float(_load().orc_e4m3_decode(code))


def e5m2_decode(code: int) -> float:
    return float(_load().orc_e5m2_decode(code))


def e2m1_decode(code: int) -> float:
    return float(_load().orc_e2m1_decode(code))


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code to x (ties to even, saturating at +-448)."""
    return int(_load().orc_e4m3_encode(ctypes.c_float(x)))


# --- FP8 E4M3 path (Quantization operators guide §4.1, §4.2) ------------------

def fp8_quantize_weight(W, s=None):
    """Per-output-channel E4M3 of W diag(s): (Wq uint8 codes [N,K], sw f32 [N]),
    sw = max|w'| / 448."""
    W = _half_bits(W)
    N, K = W.shape
    s = _smooth(s)
    Wq = np.empty((N, K), np.uint8)
    sw = np.empty(N, np.float32)
    _load().orc_fp8_quantize_weight(_ptr(W, _u16p), _ptr(s, _f32p), N, K,
                                    _ptr(Wq, _u8p), _ptr(sw, _f32p))
    return Wq, sw


def fp8_quantize_act(X, s=None):
    """Per-token dynamic E4M3 of X / s: (Xq uint8 codes [M,K], sx f32 [M])."""
    X = _half_bits(X)
    M, K = X.shape
    s = _smooth(s)
    Xq = np.empty((M, K), np.uint8)
    sx = np.empty(M, np.float32)
    _load().orc_fp8_quantize_act(_ptr(X, _u16p), _ptr(s, _f32p), M, K,
                                 _ptr(Xq, _u8p), _ptr(sx, _f32p))
    return Xq, sx


def fp8_gemm(Xq, Wq, rows=None):
    """Exact acc = e4m3(Xq) e4m3(Wq)^T in fp64 and sum |products| ([rows or M, N])."""
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    M, K = Xq.shape
    N = Wq.shape[0]
    r = _rows(rows)
    n_rows = M if r is None else r.size
    acc = np.empty((n_rows, N), np.float64)
    aacc = np.empty((n_rows, N), np.float64)
    _load().orc_fp8_gemm(_ptr(Xq, _u8p), M, K, _ptr(Wq, _u8p), N, _ptr(r, _i64p), n_rows,
                         _ptr(acc, _f64p), _ptr(aacc, _f64p))
    return acc, aacc


def fp8_reference(acc, abs_acc, sx, sw, rows=None):
    """Y = sx sw acc and its error scale B = sx sw sum|products| (fp64)
    (Quantization operators guide §4.2: C = scale_A scale_B (A_fp8 @ B_fp8))."""
    sx = np.asarray(sx, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    if rows is not None:
        sx = sx[np.asarray(rows)]
    scale = sx[:, None] * sw[None, :]
    return scale * acc, scale * abs_acc


# --- MXFP4 weights (Quantization operators guide §4.3) ------------------------

def e2m1_encode(x: float) -> int:
    """Nearest E2M1 code to x (ties to even, saturating at +-6, sign kept on zero)."""
    return int(_load().orc_e2m1_encode(ctypes.c_float(x)))


def mxfp4_quantize_weight(W, s=None):
    """MXFP4 of W diag(s): (codes uint8 [N, K/2], E8M0 scales uint8 [N, K/32])."""
    W = _half_bits(W)
    N, K = W.shape
    assert K % 32 == 0
    s = _smooth(s)
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    _load().orc_mxfp4_quantize_weight(_ptr(W, _u16p), _ptr(s, _f32p), N, K,
                                      _ptr(codes, _u8p), _ptr(scales, _u8p))
    return codes, scales


def mxfp4_dequant(codes, scales) -> np.ndarray:
    """fp64 values of an MXFP4 weight [N, K]."""
    lut = np.array([e2m1_decode(c) for c in range(16)])
    codes = np.asarray(codes, dtype=np.uint8)
    u = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return lut[u] * np.repeat(sc, 32, axis=1)


def mxfp4_gemm(Xq, codes, scales, rows=None):
    """Exact acc = e4m3(Xq) (MXFP4 W)^T in fp64 and sum |products| ([rows or M, N])."""
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M, K = Xq.shape
    N = codes.shape[0]
    r = _rows(rows)
    n_rows = M if r is None else r.size
    acc = np.empty((n_rows, N), np.float64)
    aacc = np.empty((n_rows, N), np.float64)
    _load().orc_mxfp4_gemm(_ptr(Xq, _u8p), M, K, _ptr(codes, _u8p), _ptr(scales, _u8p), N,
                           _ptr(r, _i64p), n_rows, _ptr(acc, _f64p), _ptr(aacc, _f64p))
    return acc, aacc


def mxfp4_reference(acc, abs_acc, sx, rows=None):
    """Y = sx acc and its error scale B = sx sum|products| (fp64)."""
    sx = np.asarray(sx, dtype=np.float64)
    if rows is not None:
        sx = sx[np.asarray(rows)]
    return sx[:, None] * acc, sx[:, None] * abs_acc


# --- NF4 weights (Quantization operators guide §3.4) ---------------------------

def nf4_levels() -> np.ndarray:
    """The guide's 16 NF4 levels: the N(0, 1) quantiles at the midpoints of 16
    equal-probability intervals, (i + 0.5) / 16, divided by the largest
    magnitude and rounded to fp16 (ascending)."""
    from scipy.stats import norm
    lv = norm.ppf((np.arange(16) + 0.5) / 16)
    return (lv / np.abs(lv).max()).astype(np.float16)


def nf4_quantize(W):
    """NF4 of W [N, K] (K % 64 == 0): (codes uint8 [N, K/2], scales f32 [N, K/64])."""
    W = _half_bits(W)
    N, K = W.shape
    assert K % 64 == 0
    lv = _half_bits(nf4_levels())
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.empty((N, K // 64), np.float32)
    _load().orc_nf4_quantize(_ptr(W, _u16p), N, K, _ptr(lv, _u16p), _ptr(codes, _u8p),
                             _ptr(scales, _f32p))
    return codes, scales


def nf4_dequant(codes, scales) -> np.ndarray:
    """fp64 w_hat = level[code] * scale of an NF4 weight [N, K]."""
    lv = nf4_levels().astype(np.float64)
    codes = np.asarray(codes, dtype=np.uint8)
    u = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    return lv[u] * np.repeat(np.asarray(scales, dtype=np.float64), 64, axis=1)


def nf4_ref(X, codes, scales, rows=None):
    """fp64 Y = X W_hat^T and B = |X| |W_hat|^T for an NF4 weight."""
    X = _half_bits(X)
    M, K = X.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    N = codes.shape[0]
    lv = _half_bits(nf4_levels())
    r = _rows(rows)
    n_rows = M if r is None else r.size
    Y = np.empty((n_rows, N), np.float64)
    B = np.empty((n_rows, N), np.float64)
    _load().orc_nf4_ref(_ptr(X, _u16p), M, K, _ptr(codes, _u8p), _ptr(scales, _f32p),
                        _ptr(lv, _u16p), N, _ptr(r, _i64p), n_rows, _ptr(Y, _f64p), _ptr(B, _f64p))
    return Y, B


# NVFP4 (Quantization notes, FP4 item: E2M1 values, one FP8 E4M3 scale per
# block of 16; orc_nvfp4_quantize states the steps and the reading of the
# sketch's rounding line)
def nvfp4_quantize(W):
    """NVFP4 of W [N, K] (K % 16 == 0): (codes uint8 [N, K/2], E4M3 scale bytes uint8 [N, K/16])."""
    W = _half_bits(W)
    N, K = W.shape
    assert K % 16 == 0
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    _load().orc_nvfp4_quantize(_ptr(W, _u16p), N, K, _ptr(codes, _u8p), _ptr(scales, _u8p))
    return codes, scales


def nvfp4_dequant(codes, scales) -> np.ndarray:
    """fp64 w_hat = e2m1(code) * e4m3(scale) of an NVFP4 weight [N, K]."""
    lut4 = np.array([e2m1_decode(c) for c in range(16)], np.float64)
    lut8 = np.array([e4m3_decode(c) for c in range(256)], np.float64)
    codes = np.asarray(codes, dtype=np.uint8)
    u = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    return lut4[u] * np.repeat(lut8[np.asarray(scales, dtype=np.uint8)], 16, axis=1)


def nvfp4_ref(X, codes, scales, rows=None):
    """fp64 Y = X W_hat^T and B = |X| |W_hat|^T for an NVFP4 weight."""
    X = _half_bits(X)
    M, K = X.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    N = codes.shape[0]
    r = _rows(rows)
    n_rows = M if r is None else r.size
    Y = np.empty((n_rows, N), np.float64)
    B = np.empty((n_rows, N), np.float64)
    _load().orc_nvfp4_ref(_ptr(X, _u16p), M, K, _ptr(codes, _u8p), _ptr(scales, _u8p), N,
                          _ptr(r, _i64p), n_rows, _ptr(Y, _f64p), _ptr(B, _f64p))
    return Y, B


# --- LayerNorm with the SmoothQuant divide and the per-token INT8 quantizer ---

def layernorm_quant_smooth(X, gamma, beta, s=None, eps: float = 1e-5, want_x: bool = False):
    """LayerNorm of each fp16 row of X (exact sums, fp64 statistics), the
    divide by s folded into the affine step, then per-token INT8 codes
    (Quantization operators guide §5.3, deployment fusion). Returns
    (Xq int8 [M,K], sx f32 [M]) and, with want_x, also x' f32 [M,K] and the
    row statistics f64 [M,3] (mean, biased variance, 1/sqrt(var + eps))."""
    X = _half_bits(X)
    M, K = X.shape
    gamma = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
    beta = np.ascontiguousarray(np.asarray(beta, dtype=np.float32))
    assert gamma.shape == (K,) and beta.shape == (K,) and eps > 0
    s = _smooth(s)
    Xq = np.empty((M, K), np.int8)
    sx = np.empty(M, np.float32)
    xs = np.empty((M, K), np.float32) if want_x else None
    st = np.empty((M, 3), np.float64) if want_x else None
    _load().orc_layernorm_quant_smooth(_ptr(X, _u16p), _ptr(gamma, _f32p), _ptr(beta, _f32p),
                                       _ptr(s, _f32p), float(eps), M, K, _ptr(Xq, _i8p),
                                       _ptr(sx, _f32p), _ptr(xs, _f32p), _ptr(st, _f64p))
    return (Xq, sx, xs, st) if want_x else (Xq, sx)


def layernorm_quant_smooth_fp8(X, gamma, beta, s=None, eps: float = 1e-5):
    """The same LayerNorm with per-token FP8 E4M3 codes (scale max|x'| / 448).
    Returns (Xq E4M3 bytes [M,K], sx f32 [M])."""
    X = _half_bits(X)
    M, K = X.shape
    gamma = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
    beta = np.ascontiguousarray(np.asarray(beta, dtype=np.float32))
    assert gamma.shape == (K,) and beta.shape == (K,) and eps > 0
    s = _smooth(s)
    Xq = np.empty((M, K), np.uint8)
    sx = np.empty(M, np.float32)
    _load().orc_layernorm_quant_smooth_fp8(_ptr(X, _u16p), _ptr(gamma, _f32p), _ptr(beta, _f32p),
                                           _ptr(s, _f32p), float(eps), M, K, _ptr(Xq, _u8p), _ptr(sx, _f32p))
    return Xq, sx


def u128_to_double(v: int) -> float:
    """The oracle's fp64 rounding of an unsigned 128-bit integer."""
    return _load().orc_u128_to_double(v >> 64, v & ((1 << 64) - 1))
