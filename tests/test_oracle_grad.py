"""The oracle's analytic backward against central finite differences in float64 (CPU only).

"Gaussian splatting in PyTorch", section 6: test differentiable code in float64 against finite
differences (float32 has too few digits for it). The loss is L = sum(W * image) with a seeded
W, so dL/dimage = W. Scenes are re-drawn until no blend decision lies near a threshold, so the
+-h perturbations cannot cross one.
"""
import numpy as np
import pytest

import oracle
from gaussian_splatting_tile_gs_amd import synth

PARAMS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def _scene(seed, sh_degree, n=10, W=32, H=32, f=40.0, with_clamped=True):
    sc = synth.random_scene(n, seed, width=W, height=H, focal=f, sh_degree=sh_degree, sh_rest_std=0.3)
    sc = {k: (np.asarray(v, np.float64) if k != "sh_degree" else v) for k, v in sc.items()}
    if with_clamped:
        # one large Gaussian beyond the widened frustum in x (x/z = 0.6 > 0.52): its J is
        # built at the clamp, but its footprint still reaches into the image
        sc["means"][0] = [0.6 * 3.0, 0.1, 3.0]
        sc["log_scales"][0] = [np.log(0.35), np.log(0.2), np.log(0.25)]
        sc["opacity_logits"][0] = 1.0
    return sc


def _loss(sc, cam, Wt):
    pr = oracle.project(sc, cam, np.float64)
    out = oracle.render(pr, cam, dtype=np.float64)
    return float(np.sum(out["image"] * Wt))


def _stable_scene(sh_degree, W=32, H=32, f=40.0):
    cam = synth.make_camera(np.eye(4), W, H, f, background=(0.1, 0.2, 0.3))
    for seed in range(100, 160):
        sc = _scene(seed, sh_degree, W=W, H=H, f=f)
        pr = oracle.project(sc, cam, np.float64)
        # decisions within ~1e-4 relative of a threshold are refused (band_eps scales the bound)
        out = oracle.render(pr, cam, dtype=np.float64, band_eps=5e-6)
        if not out["fragile"].any() and (pr["tiles_touched"] > 0).sum() >= 8:
            return sc, cam, pr
    raise RuntimeError("no stable scene found")


@pytest.mark.parametrize("sh_degree", [0, 3])
def test_finite_differences(sh_degree):
    sc, cam, pr = _stable_scene(sh_degree)
    W, H = cam["width"], cam["height"]
    Wt = synth.random_image_grad(H, W, seed=7).astype(np.float64)
    assert pr["tiles_touched"][0] > 0
    # the first Gaussian's J is clamped in x
    assert pr["means2d"][0, 0] > W
    _, _, _, _, raw = oracle.forward_backward(sc, cam, Wt, dtype=np.float64)
    h = 1e-6
    worst = 0.0
    for name in PARAMS:
        base = sc[name]
        an = raw[name].reshape(base.shape)
        for idx in np.ndindex(base.shape):
            plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in sc.items()}
            minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in sc.items()}
            plus[name][idx] += h
            minus[name][idx] -= h
            fd = (_loss(plus, cam, Wt) - _loss(minus, cam, Wt)) / (2 * h)
            err = abs(fd - an[idx])
            worst = max(worst, err / (1e-6 + 1e-5 * abs(an[idx])))
            assert err <= 1e-6 + 1e-5 * abs(an[idx]), (name, idx, fd, an[idx])
    assert worst <= 1.0


def test_gradient_invariants():
    sc, cam, pr = _stable_scene(0)
    Wt = synth.random_image_grad(cam["height"], cam["width"], seed=8).astype(np.float64)
    _, fwd, g2d, _, raw = oracle.forward_backward(sc, cam, Wt, dtype=np.float64)
    # the normalisation makes L invariant to |q|: q . dL/dq = 0
    q = sc["quats"]
    assert np.allclose(np.sum(q * raw["quats"], -1), 0.0, atol=1e-10 * (1 + np.abs(raw["quats"]).max()))
    # opacity = sigmoid(logit): dL/dlogit = o (1 - o) dL/do
    o = pr["opacities"]
    assert np.allclose(raw["opacity_logits"], o * (1 - o) * g2d[:, 5], rtol=1e-12, atol=1e-15)
    # degree-0 colour is the coefficient itself: dL/dsh = dL/dcolour
    assert np.allclose(raw["sh"][:, 0, :], g2d[:, 6:9], rtol=0, atol=0)
    # log-scale: dL/dl = s dL/ds, so scaling a Gaussian is the same direction for all axes sizes;
    # check against the colour rule C = sum c a T: dL/dc = sum_p a_p T_p W_p via a brute sum
    vis = pr["tiles_touched"] > 0
    assert np.all(g2d[~vis] == 0) and np.all(raw["means"][~vis] == 0)


def test_sparse_pixel_backward_matches_full():
    # A loss that is non-zero only on sampled pixels: the sampled-pixel backward (the one used at
    # full workload sizes) must equal the full-frame backward with the same sparse dL/dimage.
    sc, cam, pr = _stable_scene(3)
    W, H = cam["width"], cam["height"]
    pix = synth.sample_pixels(W, H, 200, seed=3)
    g = synth.random_image_grad(H, W, seed=9).astype(np.float64)
    sparse = np.zeros_like(g)
    sparse[pix[:, 0], pix[:, 1]] = g[pix[:, 0], pix[:, 1]]
    full2d, _ = oracle.render_backward(pr, cam, sparse, dtype=np.float64)
    samp2d, _ = oracle.render_backward(pr, cam, g[pix[:, 0], pix[:, 1]], pixels=pix, dtype=np.float64)
    assert np.allclose(full2d, samp2d, rtol=1e-12, atol=1e-14)
    fwd_full = oracle.render(pr, cam, dtype=np.float64)
    fwd_samp = oracle.render(pr, cam, pixels=pix, dtype=np.float64)
    assert np.array_equal(fwd_full["image"][pix[:, 0], pix[:, 1]], fwd_samp["image"])
