"""Pins of the oracle's SmoothQuant migration factor (CPU only).

  * at alpha = 0.5 the factor balances the two sides: max|X_j| / s_j equals
    max|W_j| * s_j (the derivation on the Quantization notes page, SmoothQuant);
  * at alpha = 1 every smoothed activation channel has max 1 (all the
    difficulty moves to the weight; Quantization operators guide §5.1);
  * the transform is an identity of the product (Core ideas §2.4): in fp64,
    (X / s)(W diag(s))^T = X W^T up to rounding;
  * the smoothing experiment of the Method boundaries page (qualitative);
  * the alpha sweep of Core ideas §2.4 (trend: lowest error at alpha = 0.5).
"""
import numpy as np
import pytest

from golden_io import load, num


def _case(seed=31, R=256, N=64, K=128):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((R, K)).astype(np.float32)
    X[:, [3, 70]] *= 30
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return X.astype(np.float16), W.astype(np.float16)


def test_balance_at_half(orc):
    X, W = _case()
    s = orc.smooth_scales(X, W, 0.5).astype(np.float64)
    ax = np.abs(X.astype(np.float64)).max(0)
    aw = np.abs(W.astype(np.float64)).max(0)
    assert np.allclose(ax / s, aw * s, rtol=4 * 2.0 ** -23)
    assert np.allclose(ax / s, np.sqrt(ax * aw), rtol=4 * 2.0 ** -23)


def test_alpha_one_moves_everything(orc):
    X, W = _case()
    s = orc.smooth_scales(X, W, 1.0).astype(np.float64)
    assert np.allclose(np.abs(X.astype(np.float64) / s).max(0), 1.0, rtol=2.0 ** -22)


def test_zero_channel_floor(orc):
    X, W = _case()
    X[:, 5] = 0
    W[:, 9] = 0
    s = orc.smooth_scales(X, W, 0.5)
    assert np.isfinite(s).all() and (s > 0).all()
    ax9 = np.float32(np.abs(X[:, 9].astype(np.float32)).max())
    assert s[9] == np.sqrt(ax9) / np.sqrt(np.float32(1e-8))
    aw5 = np.float32(np.abs(W[:, 5].astype(np.float32)).max())
    assert s[5] == np.sqrt(np.float32(1e-8)) / np.sqrt(aw5)


def test_identity_fp64(orc):
    X, W = _case(R=64)
    s = orc.smooth_scales(X, W, 0.5).astype(np.float64)
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    lhs = (Xd / s) @ (Wd * s).T
    rhs = Xd @ Wd.T
    K = X.shape[1]
    bound = 4 * K * 2.0 ** -53 * (np.abs(Xd) @ np.abs(Wd).T)
    assert np.all(np.abs(lhs - rhs) <= bound)


def _fake_quant_per_tensor(x, qmax=127):
    scale = max(np.abs(x).max(), 1e-8) / qmax
    return np.clip(np.round(x / scale), -qmax, qmax) * scale


def test_method_boundaries_experiment(orc):
    ex = load("p4_smoothing_example.txt")
    rng = np.random.default_rng(239)
    x = rng.standard_normal((64, 8)).astype(np.float32)
    x[:, 0] *= 40
    x[:, 1] *= 10
    w = rng.standard_normal((8, 6)).astype(np.float32)      # [hidden, out]
    w[0] *= 0.08
    w[1] *= 0.2
    X16, W16 = x.astype(np.float16), w.T.copy().astype(np.float16)   # W as [N, K]
    s = orc.smooth_scales(X16, W16, 0.5)
    X = X16.astype(np.float32)
    Wk = W16.astype(np.float32).T                                     # [K, N]
    ref = X @ Wk
    xs, ws = X / s, Wk * s[:, None]
    rtol, atol = num(ex["identity_assert_rtol"]), num(ex["identity_assert_atol"])
    assert np.allclose(xs @ ws, ref, rtol=rtol, atol=atol)
    base = np.abs(_fake_quant_per_tensor(X) @ _fake_quant_per_tensor(Wk) - ref).mean()
    smooth = np.abs(_fake_quant_per_tensor(xs) @ _fake_quant_per_tensor(ws) - ref).mean()
    printed_ratio = num(ex["baseline_w8a8_mae"]) / num(ex["smoothed_w8a8_mae"])
    assert smooth < base
    assert base / smooth > printed_ratio / 3
    before = np.abs(X).max(0).max()
    after = np.abs(xs).max(0).max()
    printed = num(ex["activation_range_after"]) / num(ex["activation_range_before"])
    assert after / before < 3 * printed


def test_alpha_sweep_trend(orc):
    tab = load("p5_alpha_sweep.txt")
    alphas, printed = num(tab["alpha"]), num(tab["error"])
    rng = np.random.default_rng(0)
    K, N = 256, 256
    X = rng.standard_normal((512, K)).astype(np.float32)
    X[:, : K // 100] *= 30
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    X16, W16 = X.astype(np.float16), W.astype(np.float16)
    Xd, Wd = X16.astype(np.float64), W16.astype(np.float64)
    ref = Xd @ Wd.T
    errs = []
    for a in alphas:
        s = orc.smooth_scales(X16, W16, a).astype(np.float64)
        y = _fake_quant_per_tensor(Xd / s) @ _fake_quant_per_tensor(Wd * s).T
        errs.append(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    assert int(np.argmin(errs)) == alphas.index(0.5)
    assert errs[0] > errs[1] > errs[2] < errs[3] < errs[4]
    for e, p in zip(errs, printed):
        assert e == pytest.approx(p, rel=0.25)
