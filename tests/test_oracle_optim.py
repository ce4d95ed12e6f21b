"""Pins of the optimizer oracle (oracle/optim.py) against closed forms, an independent
implementation and finite differences (CPU only).

Adam: Kingma and Ba 2015, Algorithm 1, as torch.optim.Adam implements it (the fitting loop of
"Gaussian splatting in PyTorch", section 7, calls torch.optim.Adam). The splat-size penalty of
"The backward pass I deleted" (its form read as lambda * mean_i sum_j exp(l_ij)).
"""
import numpy as np
import pytest

from oracle import optim

CFG = {"lr_means": 1.6e-4, "lr_log_scales": 5e-3, "lr_quats": 1e-3, "lr_opacity": 2.5e-2, "lr_sh_dc": 2.5e-3,
       "lr_sh_rest": 2.5e-3 / 20.0, "beta1": 0.9, "beta2": 0.999, "eps": 1e-15, "size_penalty": 0.0}


def test_first_step_moves_by_lr_times_sign():
    # from zero moments, m_hat = g and v_hat = g^2, so the step is lr g / (|g| + eps)
    rng = np.random.default_rng(0)
    g = rng.normal(size=1000) * 10.0 ** rng.uniform(-6, 3, size=1000)
    theta = rng.normal(size=1000)
    out, m, v = optim.adam_update(theta, g, np.zeros(1000), np.zeros(1000), 1, 0.01, 0.9, 0.999, 1e-12)
    assert np.allclose(out - theta, -0.01 * g / (np.abs(g) + 1e-12), rtol=1e-12, atol=0)
    assert np.allclose(m, 0.1 * g, rtol=1e-15) and np.allclose(v, 0.001 * g * g, rtol=1e-15)


def test_constant_gradient_steps_are_constant():
    # with g fixed, m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2: every bias-corrected step is the first
    g = np.array([3.0, -0.25, 1e-3])
    theta = np.zeros(3)
    m = np.zeros(3)
    v = np.zeros(3)
    for t in range(1, 51):
        new, m, v = optim.adam_update(theta, g, m, v, t, 0.1, 0.9, 0.999, 1e-12)
        assert np.allclose(new - theta, -0.1 * g / (np.abs(g) + 1e-12), rtol=1e-12, atol=0)
        theta = new


def test_zero_gradient_from_rest_keeps_parameters():
    theta = np.linspace(-1, 1, 7)
    out, m, v = optim.adam_update(theta, np.zeros(7), np.zeros(7), np.zeros(7), 1, 0.5, 0.9, 0.999, 1e-8)
    assert np.array_equal(out, theta) and not m.any() and not v.any()


def test_matches_torch_adam():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    theta0 = rng.normal(size=(64, 3))
    grads = [rng.normal(size=(64, 3)) * rng.uniform(0.01, 10) for _ in range(25)]
    p = torch.tensor(theta0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([p], lr=0.03, betas=(0.8, 0.99), eps=1e-7)
    theta, m, v = theta0.copy(), np.zeros_like(theta0), np.zeros_like(theta0)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        theta, m, v = optim.adam_update(theta, g, m, v, t, 0.03, 0.8, 0.99, 1e-7)
        assert np.allclose(theta, p.detach().numpy(), rtol=1e-12, atol=1e-14)


def test_size_penalty_gradient_is_its_derivative():
    rng = np.random.default_rng(2)
    ls = rng.uniform(-5, -1, size=(40, 3))
    lam = 0.7
    g = optim.size_penalty_grad(ls, lam)
    h = 1e-6
    for idx in [(0, 0), (7, 2), (39, 1)]:
        lp, lm = ls.copy(), ls.copy()
        lp[idx] += h
        lm[idx] -= h
        fd = (optim.size_penalty(lp, lam) - optim.size_penalty(lm, lam)) / (2 * h)
        assert abs(fd - g[idx]) <= 1e-7 * abs(g[idx]) + 1e-12
    # the penalty of one Gaussian with unit scales is lam * 3
    assert optim.size_penalty(np.zeros((1, 3)), lam) == pytest.approx(3 * lam)


def test_groups_take_their_own_rates_and_only_scales_the_penalty():
    rng = np.random.default_rng(3)
    n, deg = 5, 1
    K = (deg + 1) ** 2
    scene = {"means": rng.normal(size=(n, 3)), "log_scales": rng.uniform(-4, -2, (n, 3)),
             "quats": rng.normal(size=(n, 4)), "opacity_logits": rng.normal(size=n),
             "sh": rng.normal(size=(n, K, 3)), "sh_degree": deg}
    grads = {k: rng.normal(size=np.shape(scene[k])) for k in optim.GROUPS}
    cfg = dict(CFG, eps=1e-15)
    out = optim.adam_step(scene, grads, optim.new_state(scene), 1, cfg)
    lr = optim.learning_rates(cfg, deg, n)
    for k in optim.GROUPS:
        assert np.allclose(out[k] - scene[k], -lr[k] * np.sign(grads[k]), rtol=1e-9, atol=0), k
    assert np.all(lr["sh"][:, 0] == cfg["lr_sh_dc"]) and np.all(lr["sh"][:, 1:] == cfg["lr_sh_rest"])
    # with a penalty, the scales' first step follows the sign of g + lam exp(l) / n
    cfg2 = dict(cfg, size_penalty=50.0)
    out2 = optim.adam_step(scene, grads, optim.new_state(scene), 1, cfg2)
    gp = grads["log_scales"] + 50.0 * np.exp(scene["log_scales"]) / n
    assert np.allclose(out2["log_scales"] - scene["log_scales"], -cfg["lr_log_scales"] * np.sign(gp), rtol=1e-9)
    assert np.array_equal(out2["means"], out["means"])
