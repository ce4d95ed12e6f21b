"""The raster kernels' quadrant masks never drop a reached quadrant (CPU emulation).

Each raster workgroup stages a splat together with the set of 8 x 8 quadrants of its 16 x 16 tile
where the splat can reach alpha >= 1/255 ("Gaussian splatting in PyTorch", section 5: alpha below
1/255 is skipped): per quadrant, the minimum over its box of pixel centres of
s2 = log2(e) sigma (0 inside the box, else the least of the four edge minima of a 1D quadratic)
is compared with log2(255 o) plus a slack of 0.02 + 4e-6 times the size of the quadratic's terms
over the tile. This test replays that bound in float32 (numpy, the kernel's operation order; the
hardware log2 is modelled one part in 2^20 low) for splats placed so that alpha = 1/255 falls
within 1e-3 px of a pixel centre on a quadrant's edge, and checks it against float64 alpha at
every pixel centre: a quadrant holding a centre with alpha >= 1/255 must be in the mask.
"""
import numpy as np

LOG2E = np.float32(1.4426950408889634)
F = np.float32


def _fma(a, b, c):
    # float32 fused multiply-add: the float64 product of two float32 values is exact
    return F(np.float64(a) * np.float64(b) + np.float64(c))


def mask_f32(mx, my, A, B, C, o, tx0, ty0):
    """The quadrant mask of a splat staged for the tile whose top-left pixel is (tx0, ty0)."""
    mx, my, A, B, C, o, tx0, ty0 = map(F, (mx, my, A, B, C, o, tx0, ty0))
    qa, qc, qb = F(F(0.5) * LOG2E) * A, F(F(0.5) * LOG2E) * C, LOG2E * B
    ia, ic = F(0.5) / qa, F(0.5) / qc
    ex0, ey0 = (tx0 + F(0.5)) - mx, (ty0 + F(0.5)) - my
    X = max(abs(ex0), abs(ex0 + F(15.0)))
    Y = max(abs(ey0), abs(ey0 + F(15.0)))
    terms = _fma(qa * X, X, _fma(abs(qb) * X, Y, (qc * Y) * Y))
    log2o = F(np.log2(np.float64(F(255.0) * o)) * (1.0 - 2.0 ** -20))  # the hardware log2, modelled low
    lim = log2o + _fma(F(4e-6), terms, F(0.02))

    def q2(x, y):
        return _fma(_fma(qa, x, qb * y), x, (qc * y) * y)

    m = 0
    for q in range(4):
        x_lo, y_lo = tx0 + F((q & 1) * 8) + F(0.5), ty0 + F((q >> 1) * 8) + F(0.5)
        x0, y0 = x_lo - mx, y_lo - my
        x1, y1 = x0 + F(7.0), y0 + F(7.0)
        s_l = q2(x0, min(max(-qb * x0 * ic, y0), y1))
        s_r = q2(x1, min(max(-qb * x1 * ic, y0), y1))
        s_t = q2(min(max(-qb * y0 * ia, x0), x1), y0)
        s_b = q2(min(max(-qb * y1 * ia, x0), x1), y1)
        inside = x0 <= 0 and x1 >= 0 and y0 <= 0 and y1 >= 0
        if inside or min(s_l, s_r, s_t, s_b) <= lim:
            m |= 1 << q
    return m


def alpha64(mx, my, A, B, C, o, xs, ys):
    dx, dy = mx - xs, my - ys
    sigma = 0.5 * (A * dx * dx + C * dy * dy) + B * dx * dy
    return np.minimum(0.99, o * np.exp(-sigma))


def test_masks_keep_every_quadrant_reached_at_the_threshold():
    rng = np.random.default_rng(11)
    tx0, ty0 = 32.0, 48.0
    checked = reached = 0
    for _ in range(4000):
        # a random dilated 2D covariance (the projection adds 0.3 to the diagonal) and its conic
        L = rng.normal(size=(2, 2)) * rng.uniform(0.3, 6.0)
        S = L @ L.T + 0.3 * np.eye(2)
        A, B, C = np.linalg.inv(S)[0, 0], np.linalg.inv(S)[0, 1], np.linalg.inv(S)[1, 1]
        # float32 conic and opacity as staged; the float64 truth uses the same values
        A, B, C = float(F(A)), float(F(B)), float(F(C))
        o = float(F(rng.uniform(1.0 / 255.0 * 1.05, 1.0)))
        q = int(rng.integers(4))
        # a pixel centre on the quadrant's boundary and a direction pointing away from the quadrant
        cx0, cy0 = tx0 + (q & 1) * 8 + 0.5, ty0 + (q >> 1) * 8 + 0.5
        edge = int(rng.integers(4))
        k = float(rng.integers(8))
        px, py = [(cx0, cy0 + k), (cx0 + 7, cy0 + k), (cx0 + k, cy0), (cx0 + k, cy0 + 7)][edge]
        ang = rng.uniform(0, 2 * np.pi)
        u = np.array([np.cos(ang), np.sin(ang)])
        out = [np.array([-1.0, 0]), np.array([1.0, 0]), np.array([0, -1.0]), np.array([0, 1.0])][edge]
        if u @ out < 0.2:
            u = out
        # alpha(p) = 1/255 at distance t along u: sigma = ln(255 o) = 0.5 t^2 u^T Sigma^-1 u
        quad = A * u[0] ** 2 + 2 * B * u[0] * u[1] + C * u[1] ** 2
        t = np.sqrt(2.0 * np.log(255.0 * o) / quad) + rng.uniform(-1e-3, 1e-3)
        mx, my = px + t * u[0], py + t * u[1]
        mask = mask_f32(mx, my, A, B, C, o, tx0, ty0)
        for qq in range(4):
            xs = tx0 + (qq & 1) * 8 + 0.5 + np.arange(8)
            ys = ty0 + (qq >> 1) * 8 + 0.5 + np.arange(8)
            X, Y = np.meshgrid(xs, ys)
            hit = (alpha64(mx, my, A, B, C, o, X, Y) >= 1.0 / 255.0).any()
            checked += 1
            reached += int(hit)
            assert not hit or (mask >> qq) & 1, (mx, my, A, B, C, o, qq, mask)
    assert reached > 1000  # the placements do sit on the threshold in many quadrants


def test_masks_drop_far_quadrants():
    # the bound is not vacuous: a small splat in one quadrant leaves the other three out
    A = C = 4.0  # alpha >= 1/255 within 1.7 px of the mean; the other quadrants start 4.5 px away
    m = mask_f32(36.0, 52.0, A, 0.0, C, 0.9, 32.0, 48.0)
    assert m == 0b0001
