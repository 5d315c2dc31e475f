"""Helpers for the GPU parity tests: host <-> device marshalling and the
accuracy criterion for fp16 GEMM outputs.

Criterion (W4A16 and W8A8 outputs) against the oracle's exact fp64 product
Y_ref over the dequantized operands, with B = sum_k |x| |w_hat|:
  elementwise  |Y - Y_ref| <= 2^-10 * B + 2^-25
  overall      ||Y - Y_ref||_2 / ||Y_ref||_2 <= 5e-4
Codes, scales, zero-points and int32 accumulators are compared bit for bit.
"""
import numpy as np
import torch

REL_L2_TOL = 5e-4
ELEM_REL = 2.0 ** -10
ELEM_ABS = 2.0 ** -25


def dev():
    return torch.device("cuda", 0)


def gpu(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).view(torch.float16).to(dev())
    return torch.from_numpy(a).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.float16)
    return t.numpy()


def check_gemm(Y: np.ndarray, Yref: np.ndarray, B: np.ndarray, what: str = ""):
    Yd = Y.astype(np.float64)
    assert np.isfinite(Yd).all(), f"{what}: non-finite output"
    err = np.abs(Yd - Yref)
    lim = ELEM_REL * B + ELEM_ABS
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over 2^-10*B; worst "
                           f"err/B = {float((err / np.maximum(B, 1e-300)).max()):.3e}")
    nref = np.linalg.norm(Yref)
    if nref > 0:
        rel = np.linalg.norm(Yd - Yref) / nref
        assert rel <= REL_L2_TOL, f"{what}: relative L2 {rel:.3e} > {REL_L2_TOL}"
        return rel
    assert np.all(Yd == 0), f"{what}: reference is zero but output is not"
    return 0.0


def sample_rows(M: int, n_random: int = 24, seed: int = 0):
    """Rows that span every tile edge plus a seeded random set."""
    fixed = {0, 1, 15, 16, 63, 64, 127, 128, M // 2, M - 2, M - 1}
    rng = np.random.default_rng(seed)
    rand = set(rng.choice(M, size=min(n_random, M), replace=False).tolist())
    return sorted(r for r in fixed | rand if 0 <= r < M)
