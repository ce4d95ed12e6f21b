"""CPU oracle of the optimizer step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this module; the product path never does, and it imports nothing from the product path.

What it computes ("Gaussian splatting in PyTorch", section 7 "Fitting splats with Adam", and the
distillation write-up "The backward pass I deleted"):

* Adam (Kingma and Ba, "Adam: A Method for Stochastic Optimization", 2015, Algorithm 1, in the
  form PyTorch's ``torch.optim.Adam`` uses, which the lesson's fitting loop calls): per element,
  m <- b1 m + (1 - b1) g, v <- b2 v + (1 - b2) g^2, and
  theta <- theta - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps), with step t >= 1 and m, v
  starting at 0. The optimizer updates the raw (unconstrained) parameters.
* Per-parameter learning rates: one rate per group (means, log-scales, quaternions, opacity
  logits, SH band 0, SH bands >= 1), as the lesson lists for 3DGS training.
* The splat-size penalty of the distillation write-up: the pages name the term but not its form;
  read here as lambda * mean over Gaussians of sum_j exp(l_j) (the mean of the three scales'
  sum), whose gradient lambda exp(l_j) / N is added to dL/dl_j before the Adam update.

Everything is float64. Parity pins: ``tests/test_oracle_optim.py`` (closed forms of the first
and of constant-gradient steps, an independent implementation (``torch.optim.Adam``), finite
differences of the penalty).
"""
from __future__ import annotations

import numpy as np

GROUPS = ("means", "log_scales", "quats", "opacity_logits", "sh")


def size_penalty_grad(log_scales, lam):
    """d/dl of lam * mean_i sum_j exp(l_ij): lam * exp(l) / N (float64)."""
    ls = np.asarray(log_scales, np.float64)
    n = ls.shape[0]
    return lam * np.exp(ls) / max(n, 1)


def size_penalty(log_scales, lam):
    """lam * mean over Gaussians of the sum of the three scales."""
    ls = np.asarray(log_scales, np.float64)
    return lam * np.exp(ls).sum(axis=-1).mean() if ls.shape[0] else 0.0


def adam_update(theta, g, m, v, t, lr, b1, b2, eps):
    """One Adam step on arrays (float64): returns (theta', m', v')."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(g, np.float64)
    m = b1 * np.asarray(m, np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, np.float64) + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    return theta - lr * m_hat / (np.sqrt(v_hat) + eps), m, v


def learning_rates(cfg, sh_degree, n):
    """Per-element learning rate of each group: {"means": [N,3], ..., "sh": [N,K,3]}."""
    K = (sh_degree + 1) ** 2
    sh = np.full((n, K, 3), cfg["lr_sh_rest"], np.float64)
    sh[:, 0, :] = cfg["lr_sh_dc"]
    return {"means": np.full((n, 3), cfg["lr_means"]), "log_scales": np.full((n, 3), cfg["lr_log_scales"]),
            "quats": np.full((n, 4), cfg["lr_quats"]), "opacity_logits": np.full((n,), cfg["lr_opacity"]),
            "sh": sh}


def adam_step(scene, grads, state, t, cfg):
    """Adam step t (>= 1) of every raw parameter group of a scene dictionary.

    scene: {"means", "log_scales", "quats", "opacity_logits", "sh", "sh_degree"}; grads: the same
    keys (dL/d raw parameter); state: {"m": {group: array}, "v": {group: array}} (zeros before
    step 1; updated in place); cfg: lr_* per group, beta1, beta2, eps, size_penalty.
    Returns the updated scene (a new dictionary, float64 arrays).
    """
    n = scene["means"].shape[0]
    lrs = learning_rates(cfg, scene["sh_degree"], n)
    out = dict(scene)
    for k in GROUPS:
        g = np.asarray(grads[k], np.float64)
        if k == "log_scales" and cfg.get("size_penalty", 0.0):
            g = g + size_penalty_grad(scene["log_scales"], cfg["size_penalty"])
        out[k], state["m"][k], state["v"][k] = adam_update(scene[k], g, state["m"][k], state["v"][k], t, lrs[k],
                                                           cfg["beta1"], cfg["beta2"], cfg["eps"])
    return out


def new_state(scene):
    """Zero moments for every group."""
    z = {k: np.zeros_like(np.asarray(scene[k], np.float64)) for k in GROUPS}
    return {"m": {k: v.copy() for k, v in z.items()}, "v": {k: v.copy() for k, v in z.items()}}
