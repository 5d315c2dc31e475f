"""Seeded synthetic inputs for the group-quantized linear layer.

This module only draws random numbers: a NumPy PCG64 normal draw in fp32,
a scale by sigma, multipliers on a set of outlier channels, and a cast to fp16
(round to nearest even). It holds none of the quantization arithmetic, so both
the HIP path and the CPU oracle can take their inputs from it.

Workloads (Llama-shaped layers; K is the input width, N the output width):

  tiny      W [256, 512] ~ N(0, 0.02); X [8, 512] ~ N(0, 1) with input
            channels 0 and 1 scaled x40 and x10 (the outlier pattern of the
            smoothing experiment on the Method boundaries page); asym INT4 g128.
  decode    M = 1, K = 4096, N = 11008 and N = 4096; W ~ N(0, 0.02) with 1% of
            the K-channels x10; asym INT4 g128, packed ahead of time;
            X ~ N(0, 1).
  quant     W [11008, 4096] ~ N(0, 0.02) for the quantize + pack pass, then
            W4A16 at M = 16 and M = 64 with X ~ N(0, 1).
  prefill   M = 2048, K = 4096, N = 11008; sym INT4 g128; W ~ N(0, 0.02);
            X ~ N(0, 1) with 1% of the K-channels x30.
  w8a8      M = 2048, K = 8192, N = 8192; X ~ N(0, 1) with 1% of the
            K-channels x30; calibration X [512, 8192] from the same law and the
            same outlier channels; W ~ N(0, 0.02).
  layernorm the w8a8 workload's X read as the hidden state in front of the
            norm, with fp32 norm parameters gamma = 1 + 0.1 N(0, 1) (the
            outlier channels x30, where LLM norms carry their outliers),
            beta = 0.05 N(0, 1) and smoothing factors s = exp(0.5 N(0, 1))
            (seeds 5005, 6005, 7005).

Seeds: W 1000+c, X 2000+c, calibration X 3000+c, outlier permutation 4000+c,
for workload number c = 1..5 in the order above. The outlier set is the first
round(0.01 K) entries of a seeded permutation of range(K).
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny": dict(c=1, M=8, N=256, K=512, g=128, sym=False, x_outliers=((0, 40.0), (1, 10.0))),
    "decode": dict(c=2, M=1, N=(11008, 4096), K=4096, g=128, sym=False, w_outlier_mult=10.0),
    "quant": dict(c=3, M=(16, 64), N=11008, K=4096, g=128, sym=False),
    "prefill": dict(c=4, M=2048, N=11008, K=4096, g=128, sym=True, x_outlier_mult=30.0),
    "w8a8": dict(c=5, M=2048, N=8192, K=8192, R=512, x_outlier_mult=30.0),
}

W_SIGMA = 0.02


def seeds(c: int) -> dict:
    return dict(W=1000 + c, X=2000 + c, Xcal=3000 + c, outliers=4000 + c)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def outlier_channels(seed: int, K: int, frac: float = 0.01) -> np.ndarray:
    """First round(frac*K) entries of a seeded permutation of range(K)."""
    n = int(round(frac * K))
    return np.sort(rng(seed).permutation(K)[:n])


def normal_fp16(seed: int, shape, sigma: float = 1.0, col_mult=None) -> np.ndarray:
    """fp16 array: N(0, sigma) drawn in fp32, columns scaled by col_mult
    (a dict {column: multiplier} or (columns, multiplier)), cast RNE."""
    a = rng(seed).standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    if col_mult is not None:
        if isinstance(col_mult, dict):
            for col, mult in col_mult.items():
                a[..., col] *= np.float32(mult)
        else:
            cols, mult = col_mult
            a[..., cols] *= np.float32(mult)
    return a.astype(np.float16)


def tiny():
    w = WORKLOADS["tiny"]
    s = seeds(w["c"])
    W = normal_fp16(s["W"], (w["N"], w["K"]), W_SIGMA)
    X = normal_fp16(s["X"], (w["M"], w["K"]), 1.0, dict(w["x_outliers"]))
    return dict(W=W, X=X, g=w["g"], sym=w["sym"])


def decode(N: int = 11008):
    w = WORKLOADS["decode"]
    assert N in w["N"]
    s = seeds(w["c"])
    K = w["K"]
    cols = outlier_channels(s["outliers"], K)
    # Each N gets its own stream: the seed is offset by N so the two layers differ.
    W = normal_fp16(s["W"] * 100000 + N, (N, K), W_SIGMA, (cols, w["w_outlier_mult"]))
    X = normal_fp16(s["X"], (w["M"], K), 1.0)
    return dict(W=W, X=X, g=w["g"], sym=w["sym"], outliers=cols)


def quant(M: int | None = None):
    w = WORKLOADS["quant"]
    s = seeds(w["c"])
    W = normal_fp16(s["W"], (w["N"], w["K"]), W_SIGMA)
    out = dict(W=W, g=w["g"], sym=w["sym"])
    if M is not None:
        assert M in w["M"]
        out["X"] = normal_fp16(s["X"] * 100 + M, (M, w["K"]), 1.0)
    return out


def prefill():
    w = WORKLOADS["prefill"]
    s = seeds(w["c"])
    K = w["K"]
    cols = outlier_channels(s["outliers"], K)
    W = normal_fp16(s["W"], (w["N"], K), W_SIGMA)
    X = normal_fp16(s["X"], (w["M"], K), 1.0, (cols, w["x_outlier_mult"]))
    return dict(W=W, X=X, g=w["g"], sym=w["sym"], outliers=cols)


def w8a8():
    w = WORKLOADS["w8a8"]
    s = seeds(w["c"])
    K = w["K"]
    cols = outlier_channels(s["outliers"], K)
    W = normal_fp16(s["W"], (w["N"], K), W_SIGMA)
    X = normal_fp16(s["X"], (w["M"], K), 1.0, (cols, w["x_outlier_mult"]))
    Xcal = normal_fp16(s["Xcal"], (w["R"], K), 1.0, (cols, w["x_outlier_mult"]))
    return dict(W=W, X=X, Xcal=Xcal, outliers=cols)


def small_case(seed: int, M: int, N: int, K: int, x_outlier_mult: float = 30.0):
    """A small seeded W/X pair with the same laws as the full workloads
    (W ~ N(0, 0.02); X ~ N(0, 1) with 1% of the channels scaled)."""
    cols = outlier_channels(seed + 7, K)
    W = normal_fp16(seed, (N, K), W_SIGMA)
    X = normal_fp16(seed + 1, (M, K), 1.0, (cols, x_outlier_mult) if cols.size else None)
    return W, X


def layernorm_params(K: int, c: int = 5):
    """fp32 LayerNorm weight and bias and fp32 smoothing factors for a
    hidden width K (seeds 5000+c, 6000+c, 7000+c; gamma's outlier channels
    are the w8a8 workload's)."""
    gamma = np.float32(1.0) + np.float32(0.1) * rng(5000 + c).standard_normal(K, dtype=np.float32)
    gamma[outlier_channels(seeds(c)["outliers"], K)] *= np.float32(30.0)
    beta = np.float32(0.05) * rng(6000 + c).standard_normal(K, dtype=np.float32)
    s = np.exp(np.float32(0.5) * rng(7000 + c).standard_normal(K, dtype=np.float32)).astype(np.float32)
    return dict(gamma=gamma, beta=beta, s=s)
