"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding and compare it
with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle

BAND = oracle.BAND_F32
PIXEL_TOL = 1e-4      # absolute, per pixel channel (fp32)
GRAD_RTOL = 1e-3      # relative, per gradient component (fp32)
GRAD_FLOOR = 1e-5     # times the oracle's rounding scale of the component
# which rounding scale the gradient tolerance uses: "terms" (the magnitudes of the terms each
# per-pixel contribution is formed from, widened by the transmittance's rounding bound) or "plain"
# (the sum over pixels of the absolute per-pixel contributions)
FLOOR = "terms"


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


def tile_xcd(t, tiles_x):
    """The XCD the plan's order gives tile t: 2x1 blocks of tiles round the 8 XCDs along a row of
    blocks, each row of tiles shifted by three."""
    t = np.asarray(t, np.int64)
    return ((t % tiles_x) // 2 + 3 * (t // tiles_x)) % 8


def assert_raster_plan(plan_np, ranges_np, P, tiles_x):
    """The raster plan: per XCD (tile_xcd) a list of its tiles by non-increasing bit length of
    their pair count (empty ones last); slot 8 p + x holds place p of XCD x's list up to the
    shortest list's length m, the slots from 8 m on the longer lists' rest; a chunk length L = the
    smallest power of two >= 128 with P <= C L (C = the plan's chunk limit); for every tile of
    k = ceil(count / L) >= 2 chunks k checkpoint slots (disjoint intervals that tile [0, slots))
    and the extra work items (tile, 1 .. k - 1), in any order."""
    from gaussian_splatting_tile_gs_amd import gs as gs_mod
    plan = plan_np.view(np.uint32).astype(np.int64)
    n = ranges_np.shape[0]
    L, n_extra, n_ck = plan[0], plan[1], plan[2]
    order = plan[4:4 + n]
    assert np.array_equal(np.sort(order), np.arange(n)), "tile order is not a permutation"
    cnt = ranges_np[:, 1].astype(np.int64) - ranges_np[:, 0]
    cls_t = np.where(cnt > 0, np.floor(np.log2(np.maximum(cnt, 1))).astype(np.int64) + 1, 0)
    xcd = tile_xcd(np.arange(n), tiles_x)
    m = int(np.bincount(xcd, minlength=8).min())
    head = order[:8 * m].reshape(m, 8)
    assert np.all(xcd[head] == np.arange(8)[None, :]), "a slot below 8 m is not on its tile's XCD"
    for x in range(8):
        lc = cls_t[head[:, x]]
        assert np.all(np.diff(lc) <= 0), f"XCD {x}'s list is not heaviest class first"
        rest = order[8 * m:][xcd[order[8 * m:]] == x]
        if m and rest.size:
            assert cls_t[rest].max() <= lc[-1], f"XCD {x}'s rest is heavier than its list"
    want_L = 128
    C = gs_mod.plan_max_chunks()
    while want_L * C < P:
        want_L *= 2
    assert L == want_L, (L, want_L)
    nch = (cnt + L - 1) // L
    multi = np.nonzero(nch >= 2)[0]
    assert n_extra == (nch[multi] - 1).sum() and n_ck == nch[multi].sum()
    assert n_extra < C
    base = plan[4 + n + multi]
    span = np.zeros(n_ck, np.int64)
    for t, b0 in zip(multi, base):
        assert 0 <= b0 and b0 + nch[t] <= n_ck
        span[b0:b0 + nch[t]] += 1
    assert np.all(span == 1), "checkpoint slots overlap"
    items = plan[4 + 2 * n:4 + 2 * n + 2 * n_extra].reshape(-1, 2)
    want = sorted((t, c) for t in multi for c in range(1, nch[t]))
    assert sorted(map(tuple, items.tolist())) == want, "extra work items differ"
    # the training forward's split chunks: tiles of more than 512 entries and at least three
    # chunks of 2 L entries, their chunks after the first, each tile's together in order
    nb = (cnt + 2 * L - 1) // (2 * L)
    spl = np.nonzero((cnt > 512) & (nb >= 3))[0]
    n_split = plan[3]
    assert n_split == (nb[spl] - 1).sum() and n_split <= C // 2
    fitems = plan[4 + 2 * n + 2 * C:4 + 2 * n + 2 * C + 2 * n_split].reshape(-1, 2)
    assert sorted(map(tuple, fitems.tolist())) == sorted((t, c) for t in spl for c in range(1, nb[t])), \
        "split chunks differ"
    for t in spl:  # a tile's chunks in ascending order (a chunk waits only on earlier items)
        pos = np.nonzero(fitems[:, 0] == t)[0]
        assert np.array_equal(fitems[pos, 1], np.arange(1, nb[t])) and np.all(np.diff(pos) == 1)


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


def oracle_grads(scene, cam, o_proj, dL_dimage, pixels=None, dL_ddepth=None):
    """The oracle's 2D and raw gradients with both tolerance floors: raw["aref"] the term-magnitude
    floor, raw["aref_plain"] the sum over pixels of the absolute per-pixel contributions, each
    carried to the raw parameters through the absolute Jacobian. Returns (g2d, aref2d,
    aplain2d, raw)."""
    g2d, aref2d, aplain2d, aterms2d = oracle.render_backward(o_proj, cam, dL_dimage, pixels=pixels,
                                                             dL_ddepth=dL_ddepth, plain_floor=True)
    raw = oracle.project_backward(scene, cam, g2d, aref2d)
    raw["aref_plain"] = oracle.project_backward(scene, cam, g2d, aplain2d)["aref"]
    raw["aref_terms"] = oracle.project_backward(scene, cam, g2d, aterms2d)["aref"]
    return g2d, aref2d, aplain2d, raw


def grad_floor_stats(err, ref, floor):
    """(components that pass only because of the floor, components off, worst error/tolerance)
    for the tolerance GRAD_RTOL |ref| + GRAD_FLOOR floor."""
    rel = GRAD_RTOL * np.abs(ref)
    tol = rel + GRAD_FLOOR * floor + 1e-12
    return int(((err > rel) & (err <= tol)).sum()), int((err > tol).sum()), float((err / tol).max(initial=0.0))


def compare_grads(gpu_grads: dict, orc_raw: dict, sh_degree: int, label=""):
    """Raw gradients within GRAD_RTOL |g_ref| + GRAD_FLOOR A_ref per component. Logs, per case, how
    many components pass only because of the floor and, when the oracle gave both floors, the
    same under each; returns the worst error/tolerance ratio of the floor asserted."""
    floors = {"terms": oracle.split_raw(orc_raw["aref"], sh_degree)}
    if "aref_plain" in orc_raw:
        floors["plain"] = oracle.split_raw(orc_raw["aref_plain"], sh_degree)
    if "aref_terms" in orc_raw:
        floors["terms_unwidened"] = oracle.split_raw(orc_raw["aref_terms"], sh_degree)
    use = "plain" if ("plain" in floors and FLOOR == "plain") else "terms"
    stats = {f: [0, 0, 0.0] for f in floors}
    total = 0
    for k in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        g = gpu_grads[k].astype(np.float64).reshape(orc_raw[k].shape)
        r = orc_raw[k]
        err = np.abs(g - r)
        total += err.size
        for f, fl in floors.items():
            nf, noff, w = grad_floor_stats(err, r, fl[k].reshape(r.shape))
            stats[f][0] += nf
            stats[f][1] += noff
            stats[f][2] = max(stats[f][2], w)
        fl = floors[use][k].reshape(r.shape)
        tol = GRAD_RTOL * np.abs(r) + GRAD_FLOOR * fl + 1e-12
        if (err > tol).any():
            ratio = err / tol
            i = np.unravel_index(np.argmax(ratio), ratio.shape)
            raise AssertionError(f"{label} {k}: {int((err > tol).sum())} components off ({use} floor); worst at {i}: "
                                 f"gpu {g[i]:.6e} oracle {r[i]:.6e} floor {fl[i]:.3e}")
    log(f"[{label}] gradient floors over {total} components: " + "; ".join(
        f"{f}: {s_[0]} decided by the floor ({100.0 * s_[0] / max(total, 1):.3f}%), {s_[1]} off, "
        f"worst err/tol {s_[2]:.3f}" for f, s_ in stats.items()) + f" (asserted: {use})")
    return stats[use][2]
