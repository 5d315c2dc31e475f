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


# (what, elements, worst err / B, relative L2) of every check_gemm call; the
# GPU run writes them out (conftest) for the accuracy-margin table
MARGINS = []


def check_gemm(Y: np.ndarray, Yref: np.ndarray, B: np.ndarray, what: str = ""):
    Yd = Y.astype(np.float64)
    assert np.isfinite(Yd).all(), f"{what}: non-finite output"
    err = np.abs(Yd - Yref)
    lim = ELEM_REL * B + ELEM_ABS
    bad = err > lim
    pos = B > 0
    worst = float((err[pos] / B[pos]).max()) if pos.any() else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements over 2^-10*B; worst "
                           f"err/B = {worst:.3e}")
    nref = np.linalg.norm(Yref)
    rel = 0.0
    if nref > 0:
        rel = float(np.linalg.norm(Yd - Yref) / nref)
        assert rel <= REL_L2_TOL, f"{what}: relative L2 {rel:.3e} > {REL_L2_TOL}"
    else:
        assert np.all(Yd == 0), f"{what}: reference is zero but output is not"
    MARGINS.append({"what": what, "elements": int(Yd.size), "worst_err_over_B": worst,
                    "rel_l2": rel})
    return rel


def sample_rows(M: int, n_random: int = 256, seed: int = 0):
    """Rows that span every tile edge (the first and last row of every
    16-, 32-, 64-, 128- and 256-row tile) plus a seeded random set of
    n_random more, so that at least 256 rows are checked whenever M allows."""
    fixed = {0, 1, M // 2, M - 2, M - 1}
    for t in (16, 32, 64, 128, 256):
        for b in range(0, M, t):
            fixed.update((b, min(b + t, M) - 1))
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(M), np.fromiter(fixed, dtype=np.int64))
    rand = set(rng.choice(rest, size=min(n_random, rest.size), replace=False).tolist())
    return sorted(r for r in fixed | rand if 0 <= r < M)


class GuardedAllocator:
    """Stand-in for the binding's output allocator in the GPU tests: every
    buffer gets PAD bytes of canary (0xA5) before and after it, and its own
    bytes start as 0xFF (NaN in fp16 / fp32, -1 in the integer types), so
    an element a kernel never wrote fails the comparison and a write past
    either end of a buffer is found by check(), which runs after each test.
    The canaries sit inside the same device allocation, so torch's caching
    allocator cannot hide such a write."""
    PAD = 4096
    CANARY = 0xA5

    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype, device):
        shape = tuple(int(d) for d in (shape if isinstance(shape, (tuple, list)) else (shape,)))
        itemsize = torch.empty((), dtype=dtype).element_size()
        nbytes = int(np.prod(shape, dtype=np.int64)) * itemsize
        buf = torch.empty(nbytes + 2 * self.PAD, dtype=torch.uint8, device=device)
        buf.fill_(self.CANARY)
        body = buf[self.PAD: self.PAD + nbytes]
        body.fill_(0xFF)
        self.bufs.append((buf, nbytes))
        return body.view(dtype).view(shape)

    def check(self):
        for buf, nbytes in self.bufs:
            head = buf[: self.PAD]
            tail = buf[self.PAD + nbytes:]
            bad_head = int((head != self.CANARY).sum())
            bad_tail = int((tail != self.CANARY).sum())
            assert bad_head == 0 and bad_tail == 0, (
                f"a kernel wrote outside a {nbytes}-byte output: {bad_head} bytes before it, "
                f"{bad_tail} bytes after it")
        self.bufs.clear()


def out_buffer(shape, dtype):
    """An output buffer for a test's own out= / acc_out= argument, from the
    binding's allocator (guarded during the GPU tests)."""
    import quantized_gemm_q4_amd as q4
    return q4._empty(shape, dtype, dev())


def poisoned(W: np.ndarray, seed: int, count: int = 6):
    """A copy of the fp16 matrix W with NaN, +Inf and -Inf written into
    `count` seeded cells (cycling through the three), the cells, and a clean
    copy with those cells set to 0: inputs for the flagged-group rule (a
    group holding a non-finite value gets the format's NaN scale and zero
    codes; every other group is quantized as in the clean copy)."""
    rng = np.random.default_rng(seed)
    Wp = np.array(W, dtype=np.float16, copy=True)
    clean = np.array(W, dtype=np.float16, copy=True)
    rows = rng.integers(0, W.shape[0], count)
    cols = rng.integers(0, W.shape[1], count)
    vals = [np.float16(np.nan), np.float16(np.inf), np.float16(-np.inf)]
    for i, (r, c) in enumerate(zip(rows, cols)):
        Wp[r, c] = vals[i % 3]
        clean[r, c] = 0
    return Wp, list(zip(rows.tolist(), cols.tolist())), clean


def flagged_mask(cells, shape, group: int):
    """[rows, K // group] bool: the groups that hold a poisoned cell."""
    m = np.zeros((shape[0], shape[1] // group), bool)
    for r, c in cells:
        m[r, c // group] = True
    return m
