"""CPU oracle for the tile-based 3D Gaussian Splatting rasterizer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this package. The product path (the HIP library and its binding) never imports, links or calls
it, and it imports nothing from the product path.

This module is argument marshalling around ``liboracle.so`` (built from ``gs_oracle.cpp`` by
``oracle/build.py``): numpy arrays in, numpy arrays out. The arithmetic and its citations live
in ``gs_oracle.cpp``. Scenes and cameras are the plain dictionaries produced by the seeded
input generators:

    scene  = {"means": [N,3], "log_scales": [N,3], "quats": [N,4] (w,x,y,z),
              "opacity_logits": [N], "sh": [N,K,3], "sh_degree": d}
    camera = {"viewmat": [4,4] row-major world->camera (OpenCV axes), "fx", "fy", "cx", "cy",
              "width", "height", "near", "background": [3]}

Every function takes ``dtype`` (np.float32: the kernel's precision for every decision, the
default; np.float64: the closed-form pins and finite-difference checks).

Parity status: every function here is pinned by tests in ``tests/test_oracle_*.py`` (worked
examples of the pages, closed forms, invariants, brute force and finite differences); none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# GS_ORACLE_LIB may name another build of gs_oracle.cpp (the sanitizer build of build.py --debug)
LIB_PATH = os.environ.get("GS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

# Unit roundoff of the fp32 implementation compared against (sets the fragility bands).
BAND_F32 = 2.0 ** -24


def load():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    for name in ("orc_exp_f32", "orc_log_f32"):
        getattr(lib, name).argtypes = [P, P, i64]
        getattr(lib, name).restype = None
    lib.orc_covariance_f64.argtypes = [P, P, P, P]
    lib.orc_covariance_f64.restype = None
    lib.orc_sh_basis_f64.argtypes = [i32, P, P, i64]
    lib.orc_sh_basis_f64.restype = None
    for name in ("orc_project_f32", "orc_project_f64"):
        getattr(lib, name).argtypes = [i32, i32] + [P] * 6 + [i32, i32] + [P] * 10
        getattr(lib, name).restype = ctypes.c_int
    lib.orc_bin.argtypes = [i32] + [P] * 6 + [i32, i32, i32, i64, P, P, P]
    lib.orc_bin.restype = i64
    for name in ("orc_render_f32", "orc_render_f64"):
        getattr(lib, name).argtypes = [i32] + [P] * 7 + [i32, i32, i32, P, i64, P, f64] + [P] * 7
        getattr(lib, name).restype = ctypes.c_int
    for name in ("orc_render_bwd_f32", "orc_render_bwd_f64"):
        getattr(lib, name).argtypes = [i32] + [P] * 7 + [i32, i32, i32, P, i64, P, f64, P, P, P, P, P]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("orc_project_bwd_f32", "orc_project_bwd_f64"):
        getattr(lib, name).argtypes = [i32, i32] + [P] * 6 + [i32, i32] + [P] * 8
        getattr(lib, name).restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _suffix(dtype):
    return "f32" if np.dtype(dtype) == np.float32 else "f64"


RADIUS_MODES = {"gsplat": 0, "3dgs": 1}


def camera_array(cam, dtype=np.float32):
    """Pack a camera dict into the oracle's 27-number layout. Options (section 4 of the PyTorch
    lesson): cam["radius_mode"] "gsplat" (default, the opacity-aware per-axis extent) or "3dgs"
    (ceil(3 sqrt(lambda_max)) on both axes); cam["antialiased"] (default False);
    cam["tight_tiles"] (default False: every tile of the rectangle; True: only the tiles whose
    pixel centres the splat's ellipse reaches)."""
    v = np.asarray(cam["viewmat"], dtype=np.float64).reshape(16)
    bg = np.asarray(cam.get("background", (0.0, 0.0, 0.0)), dtype=np.float64)
    opts = [RADIUS_MODES[cam.get("radius_mode", "gsplat")], 1.0 if cam.get("antialiased", False) else 0.0,
            1.0 if cam.get("tight_tiles", False) else 0.0]
    arr = np.concatenate([v, [cam["fx"], cam["fy"], cam["cx"], cam["cy"], cam.get("near", 0.01)], bg, opts])
    return _c(arr, dtype)


def _tight(cam):
    return 1 if cam.get("tight_tiles", False) else 0


def tiles_of(cam):
    return (int(cam["width"]) + 15) // 16, (int(cam["height"]) + 15) // 16


def num_threads():
    return int(load().orc_num_threads())


def set_num_threads(k):
    """Threads of the oracle's later parallel loops."""
    load().orc_set_num_threads(int(k))


# ---------------------------------------------------------------------------------------------
def exp_d1(x):
    """D1 exp on float32 input (the written-out Cody-Waite exp both sides implement)."""
    x = _c(x, np.float32).reshape(-1)
    y = np.empty_like(x)
    load().orc_exp_f32(_p(x), _p(y), x.size)
    return y


def log_d1(x):
    """D1 log on float32 input (atanh-series log)."""
    x = _c(x, np.float32).reshape(-1)
    y = np.empty_like(x)
    load().orc_log_f32(_p(x), _p(y), x.size)
    return y


def covariance(quat, log_scale):
    """Normalised rotation R [3,3] and Sigma = R S S^T R^T [3,3] in float64."""
    q = _c(quat, np.float64)
    ls = _c(log_scale, np.float64)
    R = np.empty(9)
    S = np.empty(9)
    load().orc_covariance_f64(_p(q), _p(ls), _p(R), _p(S))
    return R.reshape(3, 3), S.reshape(3, 3)


def sh_basis(degree, dirs):
    """SH basis values [n,16] (entries beyond (degree+1)^2 are 0) at unit directions [n,3]."""
    d = _c(dirs, np.float64).reshape(-1, 3)
    out = np.zeros((d.shape[0], 16))
    load().orc_sh_basis_f64(int(degree), _p(d), _p(out), d.shape[0])
    return out


# ---------------------------------------------------------------------------------------------
def project(scene, cam, dtype=np.float32):
    """Project every Gaussian (activations, Sigma, EWA, conic, radius, rectangle, colour).

    Returns a dict: means2d [N,2], conics [N,3], depths [N], radii [N,2] int32, opacities [N],
    colors [N,3], rects [N,4] int32 (x0,y0,x1,y1 in tiles), tiles_touched [N] uint32,
    cov2d [N,3] (dilated a,b,c), radius_3dgs [N] int32. Culled Gaussians are all zeros.
    """
    lib = load()
    n = int(np.asarray(scene["means"]).shape[0])
    deg = int(scene.get("sh_degree", 0))
    K = (deg + 1) ** 2
    means = _c(scene["means"], dtype).reshape(n, 3)
    ls = _c(scene["log_scales"], dtype).reshape(n, 3)
    q = _c(scene["quats"], dtype).reshape(n, 4)
    lg = _c(scene["opacity_logits"], dtype).reshape(n)
    sh = _c(scene["sh"], dtype).reshape(n, K, 3)
    camp = camera_array(cam, dtype)
    W, H = int(cam["width"]), int(cam["height"])
    out = {
        "means2d": np.empty((n, 2), dtype), "conics": np.empty((n, 3), dtype),
        "depths": np.empty(n, dtype), "radii": np.empty((n, 2), np.int32),
        "opacities": np.empty(n, dtype), "colors": np.empty((n, 3), dtype),
        "rects": np.empty((n, 4), np.int32), "tiles_touched": np.empty(n, np.uint32),
        "cov2d": np.empty((n, 3), dtype), "radius_3dgs": np.empty(n, np.int32),
    }
    fn = getattr(lib, "orc_project_" + _suffix(dtype))
    rc = fn(n, deg, _p(means), _p(ls), _p(q), _p(lg), _p(sh), _p(camp), W, H,
            _p(out["means2d"]), _p(out["conics"]), _p(out["depths"]), _p(out["radii"]),
            _p(out["opacities"]), _p(out["colors"]), _p(out["rects"]), _p(out["tiles_touched"]),
            _p(out["cov2d"]), _p(out["radius_3dgs"]))
    if rc != 0:
        raise ValueError("oracle project: bad arguments")
    return out


def bin_pairs(proj, cam):
    """Brute-force binning: (keys [P] uint64, ids [P] uint32, ranges [tiles,2] uint32)."""
    lib = load()
    tiles = _c(proj["tiles_touched"], np.uint32)
    rects = _c(proj["rects"], np.int32)
    depths = _c(proj["depths"], np.float32)
    n = tiles.shape[0]
    tx, ty = tiles_of(cam)
    P = int(tiles.astype(np.int64).sum())
    keys = np.empty(P, np.uint64)
    ids = np.empty(P, np.uint32)
    ranges = np.empty((tx * ty, 2), np.uint32)
    m2 = _c(proj["means2d"], np.float32)
    con = _c(proj["conics"], np.float32)
    op = _c(proj["opacities"], np.float32)
    got = lib.orc_bin(n, _p(tiles), _p(rects), _p(depths), _p(m2), _p(con), _p(op), _tight(cam), tx, ty, P,
                      _p(keys), _p(ids), _p(ranges))
    assert got == P
    return keys, ids, ranges


def _render_inputs(proj, dtype):
    return [_c(proj[k], dtype) for k in ("means2d", "conics", "opacities", "colors", "depths")] + [
        _c(proj["tiles_touched"], np.uint32), _c(proj["rects"], np.int32)]


def render(proj, cam, pixels=None, dtype=np.float32, band_eps=None):
    """Per-pixel render: every pixel walks, in one stable global depth order, the un-culled
    Gaussians whose tile list holds its tile (the tiled renderer's lists: the tile rectangle, or
    with cam["tight_tiles"] the tiles of it the ellipse reaches; with the default opacity-aware
    radius that is every Gaussian that can reach the pixel, i.e. the dense render).

    pixels: None (whole image, row-major) or int array [M,2] of (row, col).
    Returns dict image [M,3] f64, depth [M] f64 (the depth channel: camera z blended with the same
    weights, background depth 0), final_T [M] f64, last_id [M] int32 (-1: none),
    n_contrib [M] int32 (global count), fragile [M] bool, escapes (int), n_near (int).
    For pixels=None the arrays are reshaped to [H,W,...].
    """
    lib = load()
    if band_eps is None:
        band_eps = BAND_F32 if np.dtype(dtype) == np.float32 else 2.0 ** -40
    W, H = int(cam["width"]), int(cam["height"])
    ins = _render_inputs(proj, dtype)
    n = ins[0].shape[0]
    bg = _c(cam.get("background", (0, 0, 0)), dtype)
    if pixels is None:
        M = W * H
        pix = None
    else:
        pix = _c(pixels, np.int32).reshape(-1, 2)
        M = pix.shape[0]
    image = np.empty((M, 3))
    depth = np.empty(M)
    final_T = np.empty(M)
    last_id = np.empty(M, np.int32)
    n_contrib = np.empty(M, np.int32)
    fragile = np.empty(M, np.uint8)
    esc = ctypes.c_int64(0)
    nev = ctypes.c_int64(0)
    fn = getattr(lib, "orc_render_" + _suffix(dtype))
    fn(n, *[_p(a) for a in ins], _tight(cam), W, H, _p(bg), M, _p(pix), float(band_eps), _p(image), _p(final_T),
       _p(last_id), _p(n_contrib), _p(fragile), ctypes.byref(esc), ctypes.byref(nev), _p(depth))
    out = {"image": image, "depth": depth, "final_T": final_T, "last_id": last_id, "n_contrib": n_contrib,
           "fragile": fragile.astype(bool), "escapes": int(esc.value), "n_near": int(nev.value)}
    if pixels is None:
        out["image"] = image.reshape(H, W, 3)
        for k in ("depth", "final_T", "last_id", "n_contrib", "fragile"):
            out[k] = out[k].reshape(H, W)
    return out


GRAD2D_NAMES = ("mean2d_x", "mean2d_y", "conic_A", "conic_B", "conic_C", "opacity", "r", "g", "b", "depth")


def render_backward(proj, cam, dL_dimage, pixels=None, dtype=np.float32, band_eps=None, dL_ddepth=None,
                    plain_floor=False):
    """Analytic backward of the per-pixel render.

    dL_dimage: [H,W,3] (pixels=None) or [M,3] matching ``pixels``; dL_ddepth (optional): [H,W] or
    [M], the gradient on the depth channel.
    Returns (g2d [N,10] float64, aref [N,10] float64): per Gaussian d/d(mu'x, mu'y, A, B, C,
    opacity, r, g, b, depth) and the rounding scale of each (sum over pixels of the magnitudes of
    the terms each contribution is computed from, widened where the transmittance recovery loses
    digits). With plain_floor=True two more arrays [N,10] follow: the sum over pixels of the
    absolute per-pixel contribution, and the term magnitudes without the widening.
    """
    lib = load()
    if band_eps is None:
        band_eps = BAND_F32 if np.dtype(dtype) == np.float32 else 2.0 ** -40
    W, H = int(cam["width"]), int(cam["height"])
    ins = _render_inputs(proj, dtype)
    n = ins[0].shape[0]
    bg = _c(cam.get("background", (0, 0, 0)), dtype)
    if pixels is None:
        M = W * H
        pix = None
    else:
        pix = _c(pixels, np.int32).reshape(-1, 2)
        M = pix.shape[0]
    g = _c(dL_dimage, np.float64).reshape(M, 3)
    gd = _c(dL_ddepth, np.float64).reshape(M) if dL_ddepth is not None else None
    g2d = np.empty((n, 10))
    aref = np.empty((n, 10))
    aplain = np.empty((n, 10)) if plain_floor else None
    aterms = np.empty((n, 10)) if plain_floor else None
    fn = getattr(lib, "orc_render_bwd_" + _suffix(dtype))
    fn(n, *[_p(a) for a in ins], _tight(cam), W, H, _p(bg), M, _p(pix), float(band_eps), _p(g), _p(gd), _p(g2d),
       _p(aref), _p(aplain), _p(aterms))
    return (g2d, aref, aplain, aterms) if plain_floor else (g2d, aref)


def _pad10(a, n):
    """[N,9] (no depth channel) or [N,10] 2D gradients as [N,10]."""
    a = _c(a, np.float64).reshape(n, -1)
    if a.shape[1] == 9:
        a = np.concatenate([a, np.zeros((n, 1))], 1)
    return np.ascontiguousarray(a)


def project_backward(scene, cam, g2d, aref2d=None, dtype=np.float32):
    """Chain rule from the 2D gradients to the raw parameters (float64 arithmetic).

    Decisions (culling, J clamps, det clamp) are those of the ``dtype`` forward.
    Returns dict means [N,3], log_scales [N,3], quats [N,4], opacity_logits [N], sh [N,K,3]
    and, when aref2d is given, "aref" [N, 11 + 3K] (same order, flattened) -- a floor for
    tolerance checks: |Jacobian| times the 2D absolute sums.
    """
    lib = load()
    n = int(np.asarray(scene["means"]).shape[0])
    deg = int(scene.get("sh_degree", 0))
    K = (deg + 1) ** 2
    means = _c(scene["means"], dtype).reshape(n, 3)
    ls = _c(scene["log_scales"], dtype).reshape(n, 3)
    q = _c(scene["quats"], dtype).reshape(n, 4)
    lg = _c(scene["opacity_logits"], dtype).reshape(n)
    sh = _c(scene["sh"], dtype).reshape(n, K, 3)
    camp = camera_array(cam, dtype)
    W, H = int(cam["width"]), int(cam["height"])
    g = _pad10(g2d, n)
    ar = _pad10(aref2d, n) if aref2d is not None else None
    out = {"means": np.empty((n, 3)), "log_scales": np.empty((n, 3)), "quats": np.empty((n, 4)),
           "opacity_logits": np.empty(n), "sh": np.empty((n, K, 3))}
    aref_raw = np.empty((n, 11 + 3 * K)) if ar is not None else None
    fn = getattr(lib, "orc_project_bwd_" + _suffix(dtype))
    rc = fn(n, deg, _p(means), _p(ls), _p(q), _p(lg), _p(sh), _p(camp), W, H, _p(g), _p(ar),
            _p(out["means"]), _p(out["log_scales"]), _p(out["quats"]), _p(out["opacity_logits"]),
            _p(out["sh"]), _p(aref_raw))
    if rc != 0:
        raise ValueError("oracle project_backward: bad arguments")
    if aref_raw is not None:
        out["aref"] = aref_raw
    return out


def split_raw(flat, sh_degree):
    """Split a flattened [N, 11 + 3K] raw-gradient array into the named parameter arrays."""
    K = (sh_degree + 1) ** 2
    n = flat.shape[0]
    return {"means": flat[:, 0:3], "log_scales": flat[:, 3:6], "quats": flat[:, 6:10],
            "opacity_logits": flat[:, 10], "sh": flat[:, 11:].reshape(n, K, 3)}


def forward_backward(scene, cam, dL_dimage, pixels=None, dtype=np.float32, dL_ddepth=None):
    """Convenience: project, render, backward to raw parameters (with tolerance floors)."""
    proj = project(scene, cam, dtype)
    fwd = render(proj, cam, pixels, dtype)
    g2d, aref = render_backward(proj, cam, dL_dimage, pixels, dtype, dL_ddepth=dL_ddepth)
    raw = project_backward(scene, cam, g2d, aref, dtype)
    return proj, fwd, g2d, aref, raw
