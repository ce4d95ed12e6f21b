"""Why the gradient tolerance's floor is the term-magnitude one (CPU only).

The backward of "Gaussian splatting in PyTorch" section 6 recovers each splat's transmittance back
to front by dividing by 1 - alpha, and forms dC/dalpha = c T_i - S_i / (1 - alpha_i) as a
difference. On a pixel where a splat's colour matches what lies behind it the two terms cancel:
the exact sum is far smaller than its terms, while fp32 rounding scales with the terms and grows
with the number of divisions. A floor of 1e-5 times the sum of the absolute per-pixel
contributions then asks for more digits than fp32 arithmetic in any order can give; the oracle's
term-magnitude floor (1e-5 times |c| T + |S| / (1 - alpha), widened by the transmittance's
rounding bound) does not.

This test builds such a pixel (many splats of nearly one colour on a background of that colour, so
T falls deep), replays the kernels' fp32 arithmetic on it in numpy (the forward's T products and
stop rule, the backward's reciprocal recovery of T, g.S carried as one scalar, dL/dalpha by a fused
multiply-add), and compares the resulting opacity gradients with the oracle's float64 ones: some
exceed the plain floor, none the term-magnitude floor.
"""
import numpy as np

import oracle

F = np.float32


def _fma(a, b, c):
    return F(np.float64(a) * np.float64(b) + np.float64(c))


def _scene(k, rng):
    # k isotropic splats a quarter pixel from the centre of pixel (16, 16) of a 32 x 32 view, at
    # distinct depths, their colours within 1e-5 of the background's
    z = np.linspace(2.0, 4.0, k)
    means = np.stack([np.full(k, (16.75 - 16.0) * z / 40.0), np.full(k, (16.75 - 16.0) * z / 40.0), z], -1)
    col = 0.5 + rng.uniform(-1e-5, 1e-5, (k, 1, 3))
    return {"means": means, "log_scales": np.full((k, 3), np.log(0.05)), "quats": np.tile([1.0, 0, 0, 0], (k, 1)),
            "opacity_logits": rng.normal(-2.0, 0.3, k), "sh": col, "sh_degree": 0}


def _kernel_fp32_dL_do(proj, cam, px, py, g):
    """The raster kernels' arithmetic at one pixel: per splat (depth order) dL/d opacity."""
    order = np.argsort(proj["depths"], kind="stable")
    order = order[proj["tiles_touched"][order] > 0]
    log2e = F(1.4426950408889634)
    alph, cols, G = [], [], []
    for i in order:
        mx, my = F(proj["means2d"][i, 0]), F(proj["means2d"][i, 1])
        A, B, C = (F(v) for v in proj["conics"][i])
        hA, B2, hC = F(F(0.5) * log2e) * A, log2e * B, F(F(0.5) * log2e) * C
        dx, dy = mx - F(px), my - F(py)
        s2 = _fma(_fma(hA, dx, B2 * dy), dx, (hC * dy) * dy)
        Gi = F(np.exp2(-np.float64(s2)))
        a = min(F(proj["opacities"][i]) * Gi, F(0.99))
        if s2 < 0 or a < F(1.0) / F(255.0):
            continue
        alph.append(a)
        cols.append(proj["colors"][i].astype(F))
        G.append(Gi)
    # forward: T products and the stop rule
    T = F(1.0)
    n = 0
    for a in alph:
        nT = T * (F(1.0) - a)
        if nT <= F(1e-4):
            break
        T = nT
        n += 1
    bg = np.full(3, F(0.5), F)
    gS = T * F((F(g[0] * bg[0]) + F(g[1] * bg[1])) + F(g[2] * bg[2]))
    out = np.zeros(n, np.float64)
    for j in range(n - 1, -1, -1):
        a, c = alph[j], cols[j]
        inv = F(1.0) / (F(1.0) - a)
        Ti = T * inv
        gc = _fma(F(g[0]), c[0], _fma(F(g[1]), c[1], F(g[2]) * c[2]))
        g_alpha = _fma(Ti, gc, -(gS * inv))
        wT = a * Ti
        gS = _fma(gc, wT, gS)
        T = Ti
        out[j] = np.float64(G[j]) * np.float64(g_alpha)
    return out, n


def test_term_floor_covers_the_fp32_error_the_plain_floor_does_not():
    rng = np.random.default_rng(3)
    sc = _scene(120, rng)
    cam = {"viewmat": np.eye(4), "fx": 40.0, "fy": 40.0, "cx": 16.0, "cy": 16.0, "width": 32, "height": 32,
           "near": 0.01, "background": (0.5, 0.5, 0.5)}
    proj = oracle.project(sc, cam, np.float32)
    g = np.array([1.0, -0.7, 0.4])
    pix = np.array([[16, 16]], np.int32)
    fwd = oracle.render(proj, cam, pixels=pix)
    assert not fwd["fragile"][0]
    assert fwd["final_T"][0] < 2e-3  # a deep pixel
    g2d, aref, aplain, _ = oracle.render_backward(proj, cam, g[None, :], pixels=pix, plain_floor=True)
    mine, n = _kernel_fp32_dL_do(proj, cam, 16.5, 16.5, g)
    order = np.argsort(proj["depths"], kind="stable")
    order = order[proj["tiles_touched"][order] > 0][:n]
    assert n == int(fwd["n_contrib"][0]) > 40
    exact = g2d[order, 5]
    err = np.abs(mine - exact)
    plain = 1e-5 * aplain[order, 5]
    terms = 1e-5 * aref[order, 5]
    # the colours nearly match the background: the exact gradients are small next to their terms
    assert np.median(np.abs(exact) / aref[order, 5]) < 1e-2
    assert (err > 1e-3 * np.abs(exact) + plain).sum() >= 5, "the plain floor would not be needed"
    assert np.all(err <= 1e-3 * np.abs(exact) + terms), "the term-magnitude floor does not cover fp32 rounding"
