"""Seeded synthetic scenes and cameras (the inputs both the HIP path and the oracle consume).

This module draws random numbers and builds look-at cameras; it holds none of the method's
arithmetic (no activation, projection, binning or blending). Everything is drawn in float64
with numpy's PCG64 (``default_rng(seed)``) and cast to float32.

The pages measure on real captures that are not available here (a 742,000-splat locomotive
scene, the Tanks & Temples "train" scene); the workloads below are synthetic stand-ins with the
Gaussian counts, resolutions, focal lengths and camera counts of those measurements.

Scene dict:  means [N,3], log_scales [N,3], quats [N,4] (w,x,y,z, un-normalised),
             opacity_logits [N], sh [N,(d+1)^2,3], sh_degree d.
Camera dict: viewmat [4,4] row-major world->camera with OpenCV axes (+x right, +y down,
             +z forward), fx, fy, cx = W/2, cy = H/2, width, height, near, background.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    sh_degree: int
    width: int
    height: int
    focal: float
    n_cameras: int
    log_scale_range: tuple
    logit_std: float
    layout: str                     # "box" (camera at the origin looking +z) or "clustered"
    scene_extent: float = 10.0      # L: blob centres ~ U[-L/2, L/2]^3
    blob_sigma: float = 0.3
    n_blobs: int = 64
    ring_radius: float = 12.0
    camera_mode: str = "ring"       # "ring", "ring_jitter" or "sphere_band"
    seed: int = 1
    sh_rest_std: float = 0.05
    teacher_n: int = 0
    loss: str = "l1"
    backward: bool = True
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # 1,024 Gaussians in a 2x2x2 box 4 m in front of one camera; the small parity case.
    "tiny_1k": Workload("tiny_1k", 1024, 0, 128, 128, 150.0, 1, (-4.5, -2.5), 1.5, "box", seed=1),
    # 30,000-splat distillation student, 60 ring cameras at 1280x720 (the headline workload).
    "distill_30k": Workload("distill_30k", 30000, 0, 1280, 720, 1000.0, 60, (-5.0, -2.5), 2.0,
                            "clustered", 10.0, 0.3, seed=2, teacher_n=300000),
    # 150,000 Gaussians with degree-3 SH, 980x545, 32 cameras, L1 + DSSIM loss.
    "mid_150k_sh3": Workload("mid_150k_sh3", 150000, 3, 980, 545, 580.0, 32, (-5.5, -3.0), 2.0,
                             "clustered", 10.0, 0.3, camera_mode="sphere_band", seed=3,
                             loss="l1_dssim"),
    # 742,000-Gaussian teacher at 1920x1080, 60 cameras inside the scene, forward only.
    "teacher_742k": Workload("teacher_742k", 742000, 0, 1920, 1080, 1400.0, 60, (-6.0, -2.5), 2.0,
                             "clustered", 20.0, 0.6, ring_radius=4.0, seed=4, backward=False),
    # 400,000 Gaussians, SH3, 1959x1090, large splats: more than 2^24 pairs per camera.
    "stress_400k_sh3": Workload("stress_400k_sh3", 400000, 3, 1959, 1090, 1160.0, 16, (-5.0, -1.5),
                                2.0, "clustered", 5.0, 0.15, ring_radius=6.0,
                                camera_mode="ring_jitter", seed=5),
}


def look_at(eye, target=(0.0, 0.0, 0.0), up=(0.0, 0.0, 1.0)):
    """World->camera [4,4] with OpenCV axes: rows (right, down, forward), t = -R eye."""
    eye = np.asarray(eye, np.float64)
    f = np.asarray(target, np.float64) - eye
    f /= np.linalg.norm(f)
    r = np.cross(f, np.asarray(up, np.float64))
    r /= np.linalg.norm(r)
    d = np.cross(f, r)
    R = np.stack([r, d, f])
    V = np.eye(4)
    V[:3, :3] = R
    V[:3, 3] = -R @ eye
    return V


def make_camera(viewmat, width, height, fx, fy=None, background=(0.0, 0.0, 0.0), near=0.01):
    return {"viewmat": np.asarray(viewmat, np.float64).astype(np.float32), "fx": float(fx),
            "fy": float(fx if fy is None else fy), "cx": width / 2.0, "cy": height / 2.0,
            "width": int(width), "height": int(height), "near": float(near),
            "background": tuple(float(b) for b in background)}


def _gaussians(rng, n, means, log_scale_range, logit_std, sh_degree, sh_rest_std):
    K = (sh_degree + 1) ** 2
    log_scales = rng.uniform(log_scale_range[0], log_scale_range[1], size=(n, 3))
    quats = rng.standard_normal((n, 4))
    logits = rng.normal(0.0, logit_std, size=n)
    sh = np.zeros((n, K, 3))
    sh[:, 0, :] = rng.uniform(0.0, 1.0, size=(n, 3))
    if K > 1:
        sh[:, 1:, :] = rng.normal(0.0, sh_rest_std, size=(n, K - 1, 3))
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {"means": f32(means), "log_scales": f32(log_scales), "quats": f32(quats),
            "opacity_logits": f32(logits), "sh": f32(sh), "sh_degree": int(sh_degree)}


def blob_centres(wl: Workload, seed: int):
    rng = np.random.default_rng(seed)
    L = wl.scene_extent
    return rng.uniform(-L / 2, L / 2, size=(wl.n_blobs, 3))


def make_scene(wl: Workload, seed: int | None = None, n: int | None = None, centres_seed=None):
    """Scene of workload ``wl``. ``centres_seed`` fixes the blob centres (the teacher shares
    the student's centres and draws its Gaussians with another seed)."""
    seed = wl.seed if seed is None else seed
    n = wl.n if n is None else n
    rng = np.random.default_rng(seed)
    if wl.layout == "box":
        means = np.stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(3, 5, n)], -1)
    else:
        centres = blob_centres(wl, wl.seed if centres_seed is None else centres_seed)
        pick = rng.integers(0, wl.n_blobs, size=n)
        means = centres[pick] + rng.normal(0.0, wl.blob_sigma, size=(n, 3))
    return _gaussians(rng, n, means, wl.log_scale_range, wl.logit_std, wl.sh_degree, wl.sh_rest_std)


def make_teacher(wl: Workload):
    """The distillation target scene: same blob centres, its own draws (seed + 100)."""
    return make_scene(wl, seed=wl.seed + 100, n=wl.teacher_n or wl.n, centres_seed=wl.seed)


def make_cameras(wl: Workload, seed: int | None = None):
    seed = wl.seed + 200 if seed is None else seed
    rng = np.random.default_rng(seed)
    W, H, f = wl.width, wl.height, wl.focal
    if wl.layout == "box":
        return [make_camera(np.eye(4), W, H, f)]
    cams = []
    for k in range(wl.n_cameras):
        if wl.camera_mode == "ring":
            az, el = 2 * np.pi * k / wl.n_cameras, 0.0
        elif wl.camera_mode == "ring_jitter":
            az, el = 2 * np.pi * k / wl.n_cameras + rng.uniform(0, 2 * np.pi / wl.n_cameras), 0.0
        else:  # sphere_band
            az, el = rng.uniform(0, 2 * np.pi), np.deg2rad(rng.uniform(-20.0, 20.0))
        R = wl.ring_radius
        eye = (R * np.cos(el) * np.cos(az), R * np.cos(el) * np.sin(az), R * np.sin(el))
        cams.append(make_camera(look_at(eye), W, H, f))
    return cams


def random_scene(n, seed, width=32, height=32, focal=40.0, depth=(2.5, 4.0), log_scales=(-3.0, -1.8),
                 logit_std=1.5, sh_degree=0, sh_rest_std=0.2, spread=0.6):
    """A small scene in front of an identity camera, for unit tests."""
    rng = np.random.default_rng(seed)
    z = rng.uniform(depth[0], depth[1], n)
    xy = rng.uniform(-spread, spread, size=(n, 2)) * z[:, None] * (width / 2.0) / focal
    means = np.concatenate([xy, z[:, None]], -1)
    return _gaussians(rng, n, means, log_scales, logit_std, sh_degree, sh_rest_std)


def sample_pixels(width, height, count, seed):
    """``count`` distinct (row, col) pixels, seeded."""
    rng = np.random.default_rng(seed)
    idx = rng.choice(width * height, size=min(count, width * height), replace=False)
    idx.sort()
    return np.stack([idx // width, idx % width], -1).astype(np.int32)


def random_image_grad(height, width, seed, scale=1.0):
    """A seeded dL/dimage [H,W,3] for backward parity (no loss function involved)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((height, width, 3)) * scale).astype(np.float32)
