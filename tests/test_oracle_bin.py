"""Binning, sort and ranges of the oracle against brute force and invariants (CPU only).

"SplatRs: The Week the Gap Closed", section "Throughput: the tile rasterizer": project, count,
emit, sort, range, blend, each stage gated bit-exact against a naive renderer. The key layout
(tile id | depth) and the per-tile ranges are what the HIP path must reproduce bit for bit.
"""
import numpy as np
import pytest

import oracle
from gaussian_splatting_tile_gs_amd import synth


def _workload_scene(name, cam_index=0, n=None):
    wl = synth.WORKLOADS[name]
    return synth.make_scene(wl, n=n), synth.make_cameras(wl)[cam_index]


def test_bin_invariants_tiny_workload():
    sc, cam = _workload_scene("tiny_1k")
    pr = oracle.project(sc, cam)
    keys, ids, ranges = oracle.bin_pairs(pr, cam)
    tx, ty = oracle.tiles_of(cam)
    P = int(pr["tiles_touched"].astype(np.int64).sum())
    assert keys.size == P == ids.size
    # keys are non-decreasing; equal keys keep ascending Gaussian id (stable sort)
    assert np.all(keys[1:] >= keys[:-1])
    eq = keys[1:] == keys[:-1]
    assert np.all(ids[1:][eq] > ids[:-1][eq])
    # key = tile << 32 | float bits of the depth
    depth_bits = pr["depths"].astype(np.float32).view(np.uint32)
    assert np.array_equal((keys & 0xFFFFFFFF).astype(np.uint32), depth_bits[ids])
    # ranges partition [0, P) in tile order; empty tiles are (0, 0)
    tile_of = (keys >> 32).astype(np.int64)
    counts = np.bincount(tile_of, minlength=tx * ty)
    for t in range(tx * ty):
        s, e = ranges[t]
        if counts[t] == 0:
            assert (s, e) == (0, 0)
        else:
            assert e - s == counts[t] and np.all(tile_of[s:e] == t)
    # brute force: tile t lists exactly the Gaussians whose rectangle contains it
    r = pr["rects"]
    for t in range(tx * ty):
        x, y = t % tx, t // tx
        want = np.nonzero((r[:, 0] <= x) & (x < r[:, 2]) & (r[:, 1] <= y) & (y < r[:, 3]))[0]
        s, e = ranges[t]
        got = ids[s:e] if counts[t] else np.array([], np.uint32)
        assert sorted(got.tolist()) == want.tolist()
        # within a tile: ascending depth, ties by id
        d = pr["depths"][got]
        order = np.lexsort((got, d))
        assert np.array_equal(order, np.arange(got.size))


def test_rect_covers_support_brute_force():
    # Every pixel centre where alpha >= 1/255 lies in a tile of the Gaussian's rectangle (the
    # opacity-aware radius makes the tiled renderer reach exactly the dense result).
    sc, cam = _workload_scene("tiny_1k")
    pr = oracle.project(sc, cam, np.float32)
    W, H = cam["width"], cam["height"]
    ys, xs = np.mgrid[0:H, 0:W] + 0.5
    tile_x, tile_y = (np.arange(W) // 16)[None, :], (np.arange(H) // 16)[:, None]
    vis = np.nonzero(pr["tiles_touched"] > 0)[0]
    for g in vis:
        mx, my = pr["means2d"][g].astype(np.float64)
        A, B, C = pr["conics"][g].astype(np.float64)
        dx, dy = mx - xs, my - ys
        sig = 0.5 * (A * dx * dx + C * dy * dy) + B * dx * dy
        alpha = np.minimum(0.99, pr["opacities"][g] * np.exp(-sig))
        hit = (alpha >= 1 / 255) & (sig >= 0)
        x0, y0, x1, y1 = pr["rects"][g]
        inside = (tile_x >= x0) & (tile_x < x1) & (tile_y >= y0) & (tile_y < y1)
        assert not np.any(hit & ~inside), g
    out = oracle.render(pr, cam)
    assert out["escapes"] == 0


@pytest.mark.parametrize("name", ["distill_30k", "mid_150k_sh3"])
def test_escapes_zero_on_sampled_pixels(name):
    sc, cam = _workload_scene(name, n=20000)
    pr = oracle.project(sc, cam)
    pix = synth.sample_pixels(cam["width"], cam["height"], 512, seed=1)
    out = oracle.render(pr, cam, pixels=pix)
    assert out["escapes"] == 0


def test_near_plane_and_empty_inputs():
    cam = synth.make_camera(np.eye(4), 32, 32, 40.0)
    empty = {"means": np.zeros((0, 3)), "log_scales": np.zeros((0, 3)), "quats": np.zeros((0, 4)),
             "opacity_logits": np.zeros(0), "sh": np.zeros((0, 1, 3)), "sh_degree": 0}
    pr = oracle.project(empty, cam)
    keys, ids, ranges = oracle.bin_pairs(pr, cam)
    assert keys.size == 0 and np.all(ranges == 0)
    out = oracle.render(pr, cam)
    assert np.all(out["image"] == 0) and np.all(out["final_T"] == 1) and np.all(out["last_id"] == -1)


def test_huge_splat_covers_every_tile():
    cam = synth.make_camera(np.eye(4), 70, 40, 40.0)
    sc = {"means": np.array([[0.0, 0.0, 2.0]]), "log_scales": np.full((1, 3), 1.0),
          "quats": np.array([[1.0, 0, 0, 0]]), "opacity_logits": np.array([2.0]),
          "sh": np.ones((1, 1, 3)), "sh_degree": 0}
    pr = oracle.project(sc, cam)
    tx, ty = oracle.tiles_of(cam)
    assert pr["tiles_touched"][0] == tx * ty == 15
    keys, ids, ranges = oracle.bin_pairs(pr, cam)
    assert np.array_equal(ranges[:, 0], np.arange(15)) and np.array_equal(ranges[:, 1], np.arange(1, 16))


def test_equal_depths_keep_ascending_id():
    # Many Gaussians at exactly the same depth: equal keys within a tile must keep ascending
    # Gaussian id (the stable sort of section 5's argsort(depths, stable=True)).
    wl = synth.WORKLOADS["tiny_1k"]
    sc = synth.make_scene(wl, n=3000)
    sc["means"][:, 2] = 4.0
    cam = synth.make_cameras(wl)[0]
    pr = oracle.project(sc, cam)
    keys, ids, _ = oracle.bin_pairs(pr, cam)
    eq = keys[1:] == keys[:-1]
    assert eq.sum() > 1000
    assert np.all(ids[1:][eq] > ids[:-1][eq])
