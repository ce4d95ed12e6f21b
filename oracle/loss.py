"""CPU oracle of the photometric training loss -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this module; the product path never does, and it imports nothing from the product path.

What it computes: the loss of "Gaussian splatting in PyTorch", section 7 (3DGS training):
    L = (1 - lam) L1 + lam (1 - SSIM),   lam = 0.2 in the lesson,
with L1 = mean |x - y| over the h * w * 3 values and SSIM the structural similarity of Wang,
Bovik, Sheikh and Simoncelli ("Image quality assessment: from error visibility to structural
similarity", 2004). The pages name SSIM without fixing its window; this reads it as that paper's
and 3DGS's choice: per channel, local statistics under an 11 x 11 Gaussian window of standard
deviation 1.5 (normalised to sum 1), the image padded with zeros ("same" size), constants
C1 = 0.01^2 and C2 = 0.03^2 (dynamic range 1), and SSIM the mean of the map over all pixels and
channels:
    mu_x = w * x, s_xx = w * (x x) - mu_x^2, s_xy = w * (x y) - mu_x mu_y (and likewise for y),
    S = (2 mu_x mu_y + C1)(2 s_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(s_xx + s_yy + C2)).
The gradient dL/dx is written out from that definition: with the maps' partial derivatives
dS/dmu_x, dS/de_xx, dS/de_xy (e_xx = w * (x x), e_xy = w * (x y)), the sum over the map of dS/dx
at pixel q is (w^T * dS/dmu_x)(q) + 2 x_q (w^T * dS/de_xx)(q) + y_q (w^T * dS/de_xy)(q), where
w^T (the adjoint of the zero-padded "same" filter) is the same symmetric window, zero padded.
L1's derivative is sign(x - y) / (3 h w) with sign(0) = 0.

Everything is float64. Parity pins: ``tests/test_oracle_loss.py`` (SSIM(x, x) = 1 with a zero
gradient, the closed form on constant images away from the border, symmetry, an independent
filter (scipy.ndimage) for the window statistics, central differences of the gradient).
"""
from __future__ import annotations

import numpy as np

WINDOW = 11
SIGMA = 1.5
C1 = 0.01 ** 2
C2 = 0.03 ** 2


def window_1d(size=WINDOW, sigma=SIGMA):
    """The normalised 1D Gaussian window (the 2D window is its outer product)."""
    r = np.arange(size, dtype=np.float64) - (size - 1) / 2.0
    g = np.exp(-(r * r) / (2.0 * sigma * sigma))
    return g / g.sum()


def filter2d(img, w=None):
    """Zero-padded 'same' filter of an [h, w] array with the separable window: sum over the
    window of w_i w_j img(r + i - 5, c + j - 5), terms outside the image being 0."""
    g = window_1d() if w is None else w
    h = (len(g) - 1) // 2
    img = np.asarray(img, np.float64)
    H, W = img.shape
    pad = np.zeros((H, W + 2 * h))
    pad[:, h:h + W] = img
    rows = sum(g[k] * pad[:, k:k + W] for k in range(len(g)))
    pad = np.zeros((H + 2 * h, W))
    pad[h:h + H, :] = rows
    return sum(g[k] * pad[k:k + H, :] for k in range(len(g)))


def ssim_terms(x, y):
    """Per channel maps of one pair of [h, w] images: S and its partials with respect to mu_x,
    e_xx and e_xy (float64)."""
    mx, my = filter2d(x), filter2d(y)
    exx, eyy, exy = filter2d(x * x), filter2d(y * y), filter2d(x * y)
    sxx, syy, sxy = exx - mx * mx, eyy - my * my, exy - mx * my
    A1 = 2.0 * mx * my + C1
    A2 = 2.0 * sxy + C2
    B1 = mx * mx + my * my + C1
    B2 = sxx + syy + C2
    S = (A1 * A2) / (B1 * B2)
    # S = A1 A2 / (B1 B2) with A2 = 2 (e_xy - mu_x mu_y) + C2, B2 = (e_xx - mu_x^2) + s_yy + C2
    d_mx = S * (2.0 * my / A1 - 2.0 * mx / B1 - 2.0 * my / A2 + 2.0 * mx / B2)
    d_exx = -S / B2
    d_exy = 2.0 * S / A2
    return S, d_mx, d_exx, d_exy


def ssim(image, target):
    """Mean SSIM over the [h, w, 3] images."""
    x = np.asarray(image, np.float64)
    y = np.asarray(target, np.float64)
    return float(np.mean([ssim_terms(x[..., ch], y[..., ch])[0] for ch in range(x.shape[-1])]))


def loss_l1_ssim(image, target, lam=0.2):
    """(1 - lam) L1 + lam (1 - SSIM) of [h, w, 3] images, and its gradient dL/dimage [h, w, 3]."""
    x = np.asarray(image, np.float64)
    y = np.asarray(target, np.float64)
    H, W, Cc = x.shape
    n = float(H * W * Cc)
    l1 = float(np.mean(np.abs(x - y)))
    grad = (1.0 - lam) * np.sign(x - y) / n
    s_sum = 0.0
    for ch in range(Cc):
        xc, yc = x[..., ch], y[..., ch]
        S, d_mx, d_exx, d_exy = ssim_terms(xc, yc)
        s_sum += float(S.sum())
        dS = filter2d(d_mx) + 2.0 * xc * filter2d(d_exx) + yc * filter2d(d_exy)
        grad[..., ch] += -lam * dS / n
    s = s_sum / n
    return (1.0 - lam) * l1 + lam * (1.0 - s), grad
