"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding and compare it
with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle

BAND = oracle.BAND_F32
PIXEL_TOL = 1e-4      # absolute, per pixel channel (fp32)
GRAD_RTOL = 1e-3      # relative, per gradient component (fp32)
GRAD_FLOOR = 1e-5     # times the oracle's sum of absolute contributions


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu_project(gs, torch, scene, cam_dict):
    params = gs.scene_to_device(scene)
    cam = gs.make_camera(cam_dict)
    proj = gs.Projected.empty(params["n"])
    gs.gs_project(params["n"], params["sh_degree"], params["means"], params["log_scales"], params["quats"],
                  params["opacity_logits"], params["sh"], cam, proj)
    torch.cuda.synchronize()
    return params, cam, proj


def proj_to_numpy(proj):
    return {"means2d": proj.means2d.cpu().numpy(), "conics": proj.conics.cpu().numpy(),
            "depths": proj.depths.cpu().numpy(), "opacities": proj.opacities.cpu().numpy(),
            "colors": proj.colors.cpu().numpy(), "radii": proj.radii.cpu().numpy(),
            "tiles_touched": proj.tiles_touched.cpu().numpy().view(np.uint32)}


def proj_from_numpy(gs, torch, o):
    """Upload the oracle's projected records into a device Projected (stage isolation)."""
    n = o["means2d"].shape[0]
    p = gs.Projected.empty(n)
    p.means2d.copy_(torch.from_numpy(np.ascontiguousarray(o["means2d"], np.float32)))
    p.conics.copy_(torch.from_numpy(np.ascontiguousarray(o["conics"], np.float32)))
    p.depths.copy_(torch.from_numpy(np.ascontiguousarray(o["depths"], np.float32)))
    p.opacities.copy_(torch.from_numpy(np.ascontiguousarray(o["opacities"], np.float32)))
    p.colors.copy_(torch.from_numpy(np.ascontiguousarray(o["colors"], np.float32)))
    p.radii.copy_(torch.from_numpy(np.ascontiguousarray(o["radii"], np.int32)))
    p.tiles_touched.copy_(torch.from_numpy(np.ascontiguousarray(o["tiles_touched"], np.uint32).view(np.int32)))
    return p


def assert_projection_bit_exact(gpu, orc):
    vis = orc["tiles_touched"] > 0
    for k in ("radii", "tiles_touched"):
        assert np.array_equal(gpu[k], orc[k]), k
    for k in ("means2d", "conics", "depths", "opacities", "colors"):
        a = np.ascontiguousarray(gpu[k], np.float32)
        b = np.ascontiguousarray(orc[k], np.float32)
        same = a.view(np.uint32) == b.view(np.uint32)
        bad = ~same
        # the floats are written in the oracle's op order: expected bit for bit; report otherwise
        if bad.any():
            rel = np.abs(a.astype(np.float64) - b) / np.maximum(np.abs(b.astype(np.float64)), 1e-30)
            raise AssertionError(f"{k}: {int(bad.sum())} values differ, max rel {rel[bad].max():.3e}")
    return int(vis.sum())


def run_gpu_bin(gs, torch, params_n, proj, cam, capacity):
    keys = torch.empty(max(capacity, 1), device="cuda", dtype=torch.int64)
    ids = torch.empty(max(capacity, 1), device="cuda", dtype=torch.int32)
    tiles = ((cam.width + 15) // 16) * ((cam.height + 15) // 16)
    ranges = torch.empty(tiles, 2, device="cuda", dtype=torch.int32)
    plan = torch.full((gs.gs_raster_plan_words(cam),), -1, device="cuda", dtype=torch.int32)
    ws = torch.empty(gs.gs_bin_workspace_bytes(params_n, capacity, cam), device="cuda", dtype=torch.uint8)
    st, P = gs.gs_bin_and_sort(params_n, proj, cam, ws, capacity, keys, ids, ranges, plan=plan)
    torch.cuda.synchronize()
    return st, P, keys, ids, ranges, plan


def assert_raster_plan(plan_np, ranges_np, P):
    """The raster plan: tiles ordered by non-increasing bit length of their pair count (empty
    ones last), a chunk length L = the smallest power of two >= 256 with P <= 2048 L, and for
    every tile of k = ceil(count / L) >= 2 chunks k checkpoint slots (disjoint intervals that
    tile [0, slots)) and the extra work items (tile, 1 .. k - 1), in any order."""
    plan = plan_np.view(np.uint32).astype(np.int64)
    n = ranges_np.shape[0]
    L, n_extra, n_ck = plan[0], plan[1], plan[2]
    order = plan[4:4 + n]
    assert np.array_equal(np.sort(order), np.arange(n)), "tile order is not a permutation"
    cnt = ranges_np[:, 1].astype(np.int64) - ranges_np[:, 0]
    cls = np.where(cnt[order] > 0, np.floor(np.log2(np.maximum(cnt[order], 1))).astype(np.int64) + 1, 0)
    assert np.all(np.diff(cls) <= 0), "tile order is not heaviest class first"
    want_L = 256
    while want_L * 2048 < P:
        want_L *= 2
    assert L == want_L, (L, want_L)
    nch = (cnt + L - 1) // L
    multi = np.nonzero(nch >= 2)[0]
    assert n_extra == (nch[multi] - 1).sum() and n_ck == nch[multi].sum()
    assert n_extra < 2048
    base = plan[4 + n + multi]
    span = np.zeros(n_ck, np.int64)
    for t, b0 in zip(multi, base):
        assert 0 <= b0 and b0 + nch[t] <= n_ck
        span[b0:b0 + nch[t]] += 1
    assert np.all(span == 1), "checkpoint slots overlap"
    items = plan[4 + 2 * n:4 + 2 * n + 2 * n_extra].reshape(-1, 2)
    want = sorted((t, c) for t in multi for c in range(1, nch[t]))
    assert sorted(map(tuple, items.tolist())) == want, "extra work items differ"


def pixel_last_ids(nc, ids_np, ranges_np, pixels, width):
    """Gaussian id of each pixel's last added splat from the GPU's per-tile n_contrib (-1: none)."""
    rows, cols = pixels[:, 0], pixels[:, 1]
    tiles_x = (width + 15) // 16
    t = (rows // 16) * tiles_x + cols // 16
    start = ranges_np[t, 0].astype(np.int64)
    k = nc[rows, cols].astype(np.int64)
    out = np.full(len(rows), -1, np.int64)
    has = k > 0
    out[has] = ids_np[start[has] + k[has] - 1]
    return out


def compare_forward(img, final_T, nc, ids_np, ranges_np, orc_fwd, pixels, width):
    """Pixel parity off the fragile set; returns (max diff, fragile count)."""
    rows, cols = pixels[:, 0], pixels[:, 1]
    frag = orc_fwd["fragile"]
    ok = ~frag
    d = np.abs(img[rows, cols].astype(np.float64) - orc_fwd["image"])
    assert d[ok].max(initial=0.0) <= PIXEL_TOL, f"pixel diff {d[ok].max():.3e}"
    dT = np.abs(final_T[rows, cols].astype(np.float64) - orc_fwd["final_T"])
    assert dT[ok].max(initial=0.0) <= PIXEL_TOL, f"final_T diff {dT[ok].max():.3e}"
    last = pixel_last_ids(nc, ids_np, ranges_np, pixels, width)
    assert np.array_equal(last[ok], orc_fwd["last_id"][ok].astype(np.int64)), "last contributor differs"
    return float(d[ok].max(initial=0.0)), int(frag.sum())


def compare_grads(gpu_grads: dict, orc_raw: dict, sh_degree: int, label=""):
    aref = oracle.split_raw(orc_raw["aref"], sh_degree)
    worst = 0.0
    for k in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        g = gpu_grads[k].astype(np.float64).reshape(orc_raw[k].shape)
        r = orc_raw[k]
        tol = GRAD_RTOL * np.abs(r) + GRAD_FLOOR * aref[k].reshape(r.shape) + 1e-12
        err = np.abs(g - r)
        ratio = err / tol
        worst = max(worst, float(ratio.max(initial=0.0)))
        if (err > tol).any():
            i = np.unravel_index(np.argmax(ratio), ratio.shape)
            raise AssertionError(f"{label} {k}: {int((err > tol).sum())} components off; worst at {i}: "
                                 f"gpu {g[i]:.6e} oracle {r[i]:.6e} floor {aref[k].reshape(r.shape)[i]:.3e}")
    return worst
