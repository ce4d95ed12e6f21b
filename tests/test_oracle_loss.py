"""Pins of the loss oracle (oracle/loss.py): L = (1 - lam) L1 + lam (1 - SSIM) of "Gaussian
splatting in PyTorch", section 7, with SSIM as in Wang et al. 2004 (11 x 11 Gaussian window,
sigma 1.5, zero padding, C1 = 0.01^2, C2 = 0.03^2). CPU only."""
import numpy as np
import pytest

from oracle import loss as L


def _imgs(seed, H=13, W=17):
    rng = np.random.default_rng(seed)
    x = rng.uniform(0, 1, (H, W, 3))
    y = np.clip(x + rng.normal(0, 0.2, (H, W, 3)), 0, 1)
    return x, y


def test_window():
    g = L.window_1d()
    assert g.shape == (11,) and g.sum() == pytest.approx(1.0, abs=1e-15)
    assert np.allclose(g, g[::-1])
    # Gaussian ratio: g[5 + k] / g[5] = exp(-k^2 / (2 * 1.5^2))
    for k in range(1, 6):
        assert g[5 + k] / g[5] == pytest.approx(np.exp(-k * k / 4.5), rel=1e-14)


def test_filter_matches_an_independent_filter():
    scipy_ndimage = pytest.importorskip("scipy.ndimage")
    rng = np.random.default_rng(0)
    img = rng.normal(size=(23, 31))
    g = L.window_1d()
    ref = scipy_ndimage.correlate1d(scipy_ndimage.correlate1d(img, g, axis=1, mode="constant", cval=0.0),
                                    g, axis=0, mode="constant", cval=0.0)
    assert np.allclose(L.filter2d(img), ref, atol=1e-14)
    # a centred delta gives the 2D window itself
    d = np.zeros((21, 21))
    d[10, 10] = 1.0
    assert np.allclose(L.filter2d(d)[5:16, 5:16], np.outer(g, g), atol=1e-17)


def test_identical_images():
    x, _ = _imgs(1)
    assert L.ssim(x, x) == pytest.approx(1.0, abs=1e-12)
    val, grad = L.loss_l1_ssim(x, x, 0.2)
    assert val == pytest.approx(0.0, abs=1e-12)
    # SSIM is maximal at x = y and sign(0) = 0: the gradient vanishes
    assert np.abs(grad).max() < 1e-12


def test_constant_images_closed_form():
    # away from the border the statistics of constants a, b are exact: sigma = 0 and
    # S = (2 a b + C1) C2 / ((a^2 + b^2 + C1) C2)
    a, b = 0.7, 0.3
    x = np.full((30, 30), a)
    y = np.full((30, 30), b)
    S = L.ssim_terms(x, y)[0]
    inner = S[5:-5, 5:-5]
    assert np.allclose(inner, (2 * a * b + L.C1) / (a * a + b * b + L.C1), rtol=1e-12)
    # at the border the zero padding lowers the window sums (S differs there)
    assert abs(S[0, 0] - inner[0, 0]) > 1e-6


def test_symmetry_and_l1_part():
    x, y = _imgs(2)
    assert L.ssim(x, y) == pytest.approx(L.ssim(y, x), rel=1e-14)
    # lam = 0 is plain L1 with the gradient sign(x - y) / (3 h w)
    val, grad = L.loss_l1_ssim(x, y, 0.0)
    assert val == pytest.approx(np.mean(np.abs(x - y)), rel=1e-14)
    assert np.array_equal(grad, np.sign(x - y) / x.size)


def test_gradient_finite_differences():
    x, y = _imgs(3, H=9, W=12)
    lam = 0.2
    _, grad = L.loss_l1_ssim(x, y, lam)
    h = 1e-6
    rng = np.random.default_rng(4)
    for _ in range(40):
        idx = (rng.integers(9), rng.integers(12), rng.integers(3))
        if abs(x[idx] - y[idx]) < 1e-4:
            continue  # keep the L1 kink out of the +-h step
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (L.loss_l1_ssim(xp, y, lam)[0] - L.loss_l1_ssim(xm, y, lam)[0]) / (2 * h)
        assert fd == pytest.approx(grad[idx], rel=1e-6, abs=1e-11)
