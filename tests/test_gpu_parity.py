"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded synthetic inputs.

Bar: projected integers (radii, tile counts) and the floats written in the oracle's op order are
bit-exact; pair counts, sorted keys/ids and tile ranges are bit-exact; pixels within 1e-4 per
channel off the oracle's fragile set (decisions within a rounding band of a threshold); raw
gradients within 1e-3 relative plus 1e-5 of the oracle's sum of absolute contributions.
Small cases are compared whole; the full workload sizes compare projection and binning whole and
pixels/gradients on a seeded pixel sample (a loss that is non-zero only on the sample, so the
oracle's gradients are exact).
"""
import math
import time

import numpy as np
import pytest

import oracle
from gaussian_splatting_tile_gs_amd import synth
from _gpu_util import (FLOOR, assert_projection_bit_exact, assert_raster_plan, compare_forward, compare_grads, log,
                       oracle_grads, proj_from_numpy, proj_to_numpy, run_gpu_bin, run_gpu_project)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    from gaussian_splatting_tile_gs_amd import gs

    gs.load()
    return gs, torch


def _full_pixels(cam):
    H, W = cam["height"], cam["width"]
    r, c = np.mgrid[0:H, 0:W]
    return np.stack([r.ravel(), c.ravel()], -1).astype(np.int32)


def _pipeline_case(env, scene, cam_dict, pixels=None, backward=True, grad_seed=7, label="", bwd="atomic",
                   depth=False):
    """Project, bin, forward (and backward) on the GPU; compare every stage with the oracle.
    bwd: "atomic" (gs_rasterize_bwd), "det" (gs_rasterize_bwd_deterministic, run twice over a
    scrambled workspace: the two results must be equal bit for bit), "det_tiles" (the same
    without the raster plan and checkpoints). depth: render the depth channel too (compared within
    1e-4 of the largest depth) and give the backward a seeded gradient on it."""
    gs, torch = env
    t0 = time.time()
    log(f"[{label}] n={scene['means'].shape[0]} {cam_dict['width']}x{cam_dict['height']} deg={scene['sh_degree']}")
    params, cam, proj = run_gpu_project(gs, torch, scene, cam_dict)
    o_proj = oracle.project(scene, cam_dict, np.float32)
    nvis = assert_projection_bit_exact(proj_to_numpy(proj), o_proj)
    # binning end to end (GPU projection) and stage-isolated (the oracle's projection uploaded)
    o_keys, o_ids, o_ranges = oracle.bin_pairs(o_proj, cam_dict)
    P_exp = int(o_keys.size)
    st, P, keys, ids, ranges, plan = run_gpu_bin(gs, torch, params["n"], proj, cam, P_exp + 17)
    assert st == gs.GS_OK and P == P_exp
    keys_np = keys.cpu().numpy()[:P].view(np.uint64)
    ids_np = ids.cpu().numpy()[:P].view(np.uint32)
    ranges_np = ranges.cpu().numpy().view(np.uint32)
    assert np.array_equal(keys_np, o_keys), "sorted keys differ"
    assert np.array_equal(ids_np, o_ids), "sorted ids differ"
    assert np.array_equal(ranges_np, o_ranges), "tile ranges differ"
    assert_raster_plan(plan.cpu().numpy(), ranges_np, P, (cam_dict["width"] + 15) // 16)
    iso = proj_from_numpy(gs, torch, o_proj)
    st2, P2, keys2, ids2, ranges2, _ = run_gpu_bin(gs, torch, params["n"], iso, cam, P_exp)
    assert st2 == gs.GS_OK and P2 == P_exp
    assert np.array_equal(keys2.cpu().numpy()[:P].view(np.uint64), o_keys)
    assert np.array_equal(ranges2.cpu().numpy().view(np.uint32), o_ranges)
    log(f"[{label}] visible={nvis} pairs={P} projection+binning bit-exact ({time.time() - t0:.1f}s)")

    # forward
    H, W = cam_dict["height"], cam_dict["width"]
    img = torch.empty(H, W, 3, device="cuda")
    fT = torch.empty(H, W, device="cuda")
    nc = torch.empty(H, W, device="cuda", dtype=torch.int32)
    evals = torch.zeros(1, device="cuda", dtype=torch.int64)
    rws = torch.zeros(gs.gs_raster_workspace_bytes(), device="cuda", dtype=torch.uint8)
    dep = torch.empty(H, W, device="cuda") if depth else None
    gs.gs_rasterize_fwd(params["n"], proj, cam, ids, ranges, img, fT, nc, evals, plan=plan, raster_ws=rws, depth=dep)
    torch.cuda.synchronize()
    pix = _full_pixels(cam_dict) if pixels is None else pixels
    o_fwd = oracle.render(o_proj, cam_dict, pixels=pix)
    if cam_dict.get("radius_mode", "gsplat") == "gsplat":
        assert o_fwd["escapes"] == 0  # the opacity-aware rectangle holds every reached pixel
    dmax, nfrag = compare_forward(img.cpu().numpy(), fT.cpu().numpy(), nc.cpu().numpy(), ids_np, ranges_np, o_fwd,
                                  pix, W)
    assert nfrag <= max(2, len(pix) // 50), f"{nfrag} fragile pixels"
    if depth:
        dg = dep.cpu().numpy().astype(np.float64)[pix[:, 0], pix[:, 1]]
        dref = o_fwd["depth"].reshape(-1)
        ok = ~o_fwd["fragile"].reshape(-1)
        dtol = 1e-4 * max(1.0, float(np.abs(dref).max()))
        assert np.all(np.abs(dg - dref)[ok] <= dtol), f"depth channel differs by {np.abs(dg - dref)[ok].max():.3e}"
    log(f"[{label}] forward: {len(pix)} px, max |diff| {dmax:.2e}, fragile {nfrag}, evals {int(evals.item())} "
        f"({time.time() - t0:.1f}s)")
    if not backward:
        return
    # backward: seeded dL/dimage on the compared pixels (zero elsewhere and on fragile pixels)
    g = synth.random_image_grad(H, W, seed=grad_seed)
    gsel = g[pix[:, 0], pix[:, 1]].astype(np.float64)
    gsel[o_fwd["fragile"]] = 0.0
    dimg = np.zeros((H, W, 3), np.float32)
    dimg[pix[:, 0], pix[:, 1]] = gsel
    pipe_grads = {k: torch.empty_like(v) for k, v in
                  (("means", params["means"]), ("log_scales", params["log_scales"]), ("quats", params["quats"]),
                   ("opacity_logits", params["opacity_logits"]), ("sh", params["sh"]))}
    g2d_out = torch.empty(params["n"], 2, device="cuda")
    det = bwd != "atomic"
    cap = P_exp + 17  # the capacity the pairs were binned with
    ws = torch.empty(gs.gs_bwd_det_workspace_bytes(params["n"], cap) if det else gs.gs_bwd_workspace_bytes(params["n"]),
                     device="cuda", dtype=torch.uint8)
    dimg_d = torch.from_numpy(dimg).cuda()
    gdsel = None
    gdep_d = None
    if depth:
        gdsel = synth.random_image_grad(H, W, seed=grad_seed + 1)[..., 0][pix[:, 0], pix[:, 1]].astype(np.float64)
        gdsel[o_fwd["fragile"].reshape(-1)] = 0.0
        gdep = np.zeros((H, W), np.float32)
        gdep[pix[:, 0], pix[:, 1]] = gdsel
        gdep_d = torch.from_numpy(gdep).cuda()
    use_plan = bwd != "det_tiles"

    def run_bwd():
        gs.gs_rasterize_bwd(params["n"], params["sh_degree"], params["means"], params["log_scales"],
                            params["quats"], params["opacity_logits"], params["sh"], cam, proj, ids, ranges, fT, nc,
                            dimg_d, ws, pipe_grads["means"], pipe_grads["log_scales"], pipe_grads["quats"],
                            pipe_grads["opacity_logits"], pipe_grads["sh"], g2d_out,
                            plan=plan if use_plan else None, raster_ws=rws if use_plan else None,
                            pair_capacity=cap if det else None, dL_ddepth=gdep_d)
        torch.cuda.synchronize()

    run_bwd()
    if det:
        first = {k: v.clone() for k, v in pipe_grads.items()}
        first["means2d"] = g2d_out.clone()
        ws.random_(0, 256)  # the records of every pair must be rewritten
        run_bwd()
        same = all(torch.equal(first[k], v) for k, v in pipe_grads.items()) and torch.equal(first["means2d"], g2d_out)
        assert same, "the deterministic backward gave different bits on a second run"
    g2d, aref2d, aplain2d, raw = oracle_grads(scene, cam_dict, o_proj, gsel, pixels=pix, dL_ddepth=gdsel)
    gpu = {k: v.cpu().numpy() for k, v in pipe_grads.items()}
    worst = compare_grads(gpu, raw, scene["sh_degree"], label)
    m2 = g2d_out.cpu().numpy().astype(np.float64)
    fl2d = aplain2d if FLOOR == "plain" else aref2d
    tol = 1e-3 * np.abs(g2d[:, :2]) + 1e-5 * fl2d[:, :2] + 1e-12
    assert np.all(np.abs(m2 - g2d[:, :2]) <= tol), "dL/dmean2d differs"
    culled = o_proj["tiles_touched"] == 0
    assert all(np.all(gpu[k][culled] == 0) for k in gpu), "culled Gaussians must get exactly zero"
    log(f"[{label}] backward ({bwd}): worst error/tolerance {worst:.3f} ({time.time() - t0:.1f}s)")


# ---- small cases, compared whole --------------------------------------------------------------
def test_tiny_workload_full_frame(env):
    wl = synth.WORKLOADS["tiny_1k"]
    _pipeline_case(env, synth.make_scene(wl), synth.make_cameras(wl)[0], label="tiny_1k")


def test_ragged_sh3_small(env):
    # 37 x 23: a ragged tail in both directions (3 x 2 tiles), degree-3 colour, a few culled ones
    sc = synth.random_scene(300, seed=21, width=37, height=23, focal=30.0, sh_degree=3, logit_std=2.0)
    sc["means"][:5, 2] = -1.0
    cam = synth.make_camera(np.eye(4), 37, 23, 30.0, background=(0.2, 0.4, 0.6))
    _pipeline_case(env, sc, cam, label="ragged_sh3")


@pytest.mark.parametrize("deg", [1, 2])
def test_sh_degrees_small(env, deg):
    sc = synth.random_scene(400, seed=30 + deg, width=64, height=48, focal=50.0, sh_degree=deg)
    V = synth.look_at((0.4, -0.3, -0.5), target=(0.0, 0.0, 3.0), up=(0.0, -1.0, 0.0))
    _pipeline_case(env, sc, synth.make_camera(V, 64, 48, 50.0), label=f"sh{deg}")


# ---- full workload sizes: whole projection/binning, sampled pixels ------------------------------
@pytest.mark.parametrize("name,cam_index,backward", [
    ("distill_30k", 0, True), ("distill_30k", 17, True), ("mid_150k_sh3", 0, True),
    ("teacher_742k", 0, False), ("stress_400k_sh3", 0, True)])
def test_workload_sampled(env, name, cam_index, backward):
    wl = synth.WORKLOADS[name]
    scene = synth.make_scene(wl)
    cam = synth.make_cameras(wl)[cam_index]
    pix = synth.sample_pixels(cam["width"], cam["height"], 4096, seed=cam_index + 1)
    _pipeline_case(env, scene, cam, pixels=pix, backward=backward, label=f"{name}#{cam_index}")


def test_stress_every_camera_exceeds_2_24_pairs(env):
    """The full-resolution stress workload exists to exercise the large sort ("SplatRs: We Gave
    the Model 4x More Pixels", lesson 2: past 2^24 keys a sort dispatch outgrows its limits): each
    of its 16 cameras bins more than 2^24 tile/Gaussian pairs, and every count equals the sum of the
    projection's tile counts."""
    gs, torch = env
    wl = synth.WORKLOADS["stress_400k_sh3"]
    params = gs.scene_to_device(synth.make_scene(wl))
    pipe = gs.Pipeline(params, wl.width, wl.height, pair_capacity=24 << 20)
    counts = []
    for i, cam_d in enumerate(synth.make_cameras(wl)):
        cam = gs.make_camera(cam_d)
        pipe.project(cam)
        P = pipe.bin(cam)
        assert P == int(pipe.proj.tiles_touched.to(torch.int64).sum().item()), i
        counts.append(P)
    log(f"[stress cameras] pairs per camera: min {min(counts)} max {max(counts)} (2^24 = {1 << 24})")
    assert len(counts) == 16 and min(counts) > (1 << 24), counts


# ---- deterministic backward: oracle parity and bitwise reproducibility ---------------------------
@pytest.mark.parametrize("case,bwd", [("tiny", "det"), ("tiny", "det_tiles"), ("ragged", "det"),
                                      ("distill_30k", "det"), ("mid_150k_sh3", "det"), ("stress_400k_sh3", "det")])
def test_deterministic_backward(env, case, bwd):
    if case == "tiny":
        wl = synth.WORKLOADS["tiny_1k"]
        _pipeline_case(env, synth.make_scene(wl), synth.make_cameras(wl)[0], label="tiny_1k", bwd=bwd)
    elif case == "ragged":
        sc = synth.random_scene(300, seed=21, width=37, height=23, focal=30.0, sh_degree=3, logit_std=2.0)
        cam = synth.make_camera(np.eye(4), 37, 23, 30.0, background=(0.2, 0.4, 0.6))
        _pipeline_case(env, sc, cam, label="ragged_sh3", bwd=bwd)
    else:
        wl = synth.WORKLOADS[case]
        cam = synth.make_cameras(wl)[0]
        pix = synth.sample_pixels(cam["width"], cam["height"], 4096, seed=1)
        _pipeline_case(env, synth.make_scene(wl), cam, pixels=pix, label=f"{case}#0", bwd=bwd)


def test_deterministic_backward_capacity_and_arguments(env):
    """Pairs beyond the record capacity: every gradient is zero (as after a binning overflow);
    bad capacities and a misaligned workspace are rejected before any launch."""
    gs, torch = env
    wl = synth.WORKLOADS["tiny_1k"]
    params = gs.scene_to_device(synth.make_scene(wl))
    cam = gs.make_camera(synth.make_cameras(wl)[0])
    pipe = gs.Pipeline(params, wl.width, wl.height, pair_capacity=1 << 16)
    pipe.project(cam)
    P = pipe.bin(cam)
    pipe.forward(cam)
    pipe.dL_dimage.copy_(torch.from_numpy(synth.random_image_grad(wl.height, wl.width, seed=3)))
    pipe.deterministic = True
    pipe.backward(cam)
    torch.cuda.synchronize()
    assert float(pipe.grads["means"].abs().sum()) > 0.0
    g = pipe.grads
    ws = torch.empty(gs.gs_bwd_det_workspace_bytes(params["n"], P - 1), device="cuda", dtype=torch.uint8)
    args = lambda cap, w: (params["n"], 0, params["means"], params["log_scales"], params["quats"],
                           params["opacity_logits"], params["sh"], cam, pipe.proj, pipe.ids, pipe.ranges, pipe.final_T,
                           pipe.n_contrib, pipe.dL_dimage, w, g["means"], g["log_scales"], g["quats"],
                           g["opacity_logits"], g["sh"], g["means2d"])
    gs.gs_rasterize_bwd(*args(P - 1, ws), plan=pipe.plan, raster_ws=pipe.raster_ws, pair_capacity=P - 1)
    torch.cuda.synchronize()
    assert all(float(v.abs().sum()) == 0.0 for v in g.values())
    for bad in (-1, 1 << 30):
        with pytest.raises(gs.GsError):
            gs.gs_rasterize_bwd(*args(bad, ws), pair_capacity=bad)
    big = torch.empty(ws.numel() + 256, device="cuda", dtype=torch.uint8)
    with pytest.raises(gs.GsError):
        gs.gs_rasterize_bwd(*args(P - 1, big[4:]), pair_capacity=P - 1)
    assert gs.gs_bwd_det_workspace_bytes(params["n"], -1) == 0


# ---- depth channel --------------------------------------------------------------------------------
@pytest.mark.parametrize("case,bwd", [("tiny", "atomic"), ("ragged", "det"), ("distill_30k", "atomic"),
                                      ("mid_150k_sh3", "det"), ("tiny", "det_tiles"), ("distill_30k+tight", "det"),
                                      ("ragged+tight", "atomic")])
def test_depth_channel(env, case, bwd):
    case, _, opt = case.partition("+")
    if case == "tiny":
        wl = synth.WORKLOADS["tiny_1k"]
        scene, cam, pix = synth.make_scene(wl), synth.make_cameras(wl)[0], None
    elif case == "ragged":
        scene = synth.random_scene(300, seed=21, width=37, height=23, focal=30.0, sh_degree=3, logit_std=2.0)
        cam, pix = synth.make_camera(np.eye(4), 37, 23, 30.0, background=(0.2, 0.4, 0.6)), None
    else:
        wl = synth.WORKLOADS[case]
        scene, cam = synth.make_scene(wl), synth.make_cameras(wl)[0]
        pix = synth.sample_pixels(cam["width"], cam["height"], 4096, seed=1)
    if opt == "tight":
        cam = dict(cam, tight_tiles=True)
    _pipeline_case(env, scene, cam, pixels=pix, label=f"{case} {opt} depth", bwd=bwd, depth=True)


# ---- tile-count variants (camera options) ---------------------------------------------------------
@pytest.mark.parametrize("case,opts,bwd", [
    ("tiny", {"antialiased": True}, "atomic"), ("tiny", {"radius_mode": "3dgs"}, "atomic"),
    ("ragged", {"antialiased": True, "radius_mode": "3dgs"}, "atomic"), ("tiny", {"antialiased": True}, "det"),
    ("distill_30k", {"antialiased": True}, "atomic"), ("mid_150k_sh3", {"radius_mode": "3dgs"}, "atomic"),
    ("tiny", {"tight_tiles": True}, "atomic"), ("ragged", {"tight_tiles": True, "antialiased": True}, "det"),
    ("needles", {"tight_tiles": True}, "det"), ("needles", {"tight_tiles": True, "radius_mode": "3dgs"}, "atomic"),
    ("giant", {"tight_tiles": True}, "det"), ("distill_30k", {"tight_tiles": True}, "det"),
    ("mid_150k_sh3", {"tight_tiles": True, "antialiased": True}, "atomic"),
    ("dim_corners", {"tight_tiles": True}, "det"), ("stress_400k_sh3", {"tight_tiles": True}, "det")])
def test_variants(env, case, opts, bwd):
    if case == "tiny":
        wl = synth.WORKLOADS["tiny_1k"]
        scene, cam, pix = synth.make_scene(wl), dict(synth.make_cameras(wl)[0]), None
    elif case == "dim_corners":
        # ordinary splats plus 24 dim (o = 1.02/255), sub-pixel ones on tile corners: rectangles
        # of four tiles, no pixel centre reached, so tight lists leave them undrawn
        W, f, z = 96, 80.0, 3.0
        scene = synth.random_scene(200, seed=41, width=W, height=W, focal=f)
        cam = synth.make_camera(np.eye(4), W, W, f, background=(0.1, 0.1, 0.2))
        o = 1.02 / 255.0
        corners = [(16.0 * i, 16.0 * j) for i in range(1, 6) for j in range(1, 6)][:24]
        m = np.array([[(x - cam["cx"]) * z / f, (y - cam["cy"]) * z / f, z] for x, y in corners])
        k = len(corners)
        scene["means"] = np.concatenate([scene["means"], m]).astype(scene["means"].dtype)
        scene["log_scales"] = np.concatenate([scene["log_scales"], np.full((k, 3), -7.0)]).astype(
            scene["log_scales"].dtype)
        scene["quats"] = np.concatenate([scene["quats"], np.tile([1.0, 0, 0, 0], (k, 1))]).astype(
            scene["quats"].dtype)
        scene["opacity_logits"] = np.concatenate([scene["opacity_logits"], np.full(k, math.log(o / (1 - o)))]).astype(
            scene["opacity_logits"].dtype)
        scene["sh"] = np.concatenate([scene["sh"], np.full((k,) + scene["sh"].shape[1:], 0.5)]).astype(
            scene["sh"].dtype)
        pix = None
    elif case in ("needles", "giant"):
        # needles: elongated rotated splats of up to ~20 tile rows (the per-lane and per-wave row
        # walks); giant: a few splats of thousands of tiles each on a 1600 x 1600 image, whose
        # row runs cross several 4096-pair emission chunks
        n, W, f, ls = (3000, 300, 200.0, (-4.0, -2.0)) if case == "needles" else (40, 1600, 900.0, (-2.5, -0.5))
        scene = synth.random_scene(n, seed=31, width=W, height=W, focal=f, log_scales=ls, logit_std=2.0)
        rng = np.random.default_rng(32)
        scene["log_scales"][:, 0] += rng.uniform(0.0, 2.5, n)
        cam = synth.make_camera(np.eye(4), W, W, f, background=(0.2, 0.3, 0.1))
        pix = synth.sample_pixels(W, W, 4096, seed=2)
    elif case == "ragged":
        scene = synth.random_scene(300, seed=21, width=37, height=23, focal=30.0, sh_degree=3, logit_std=2.0)
        cam, pix = synth.make_camera(np.eye(4), 37, 23, 30.0, background=(0.2, 0.4, 0.6)), None
    else:
        wl = synth.WORKLOADS[case]
        scene, cam = synth.make_scene(wl), dict(synth.make_cameras(wl)[0])
        pix = synth.sample_pixels(cam["width"], cam["height"], 4096, seed=1)
    cam.update(opts)
    _pipeline_case(env, scene, cam, pixels=pix, label=f"{case} {opts}", bwd=bwd)


# ---- edge cases ---------------------------------------------------------------------------------
def test_empty_and_all_culled(env):
    gs, torch = env
    cam_d = synth.make_camera(np.eye(4), 40, 24, 30.0, background=(0.3, 0.2, 0.1))
    cam = gs.make_camera(cam_d)
    for n in (0, 5, 40000):  # 40,000: the large-frame path, whose depth sort drops culled keys
        sc = synth.random_scene(max(n, 1), seed=3, width=40, height=24, focal=30.0)
        if n == 0:
            sc = {k: (v[:0] if isinstance(v, np.ndarray) else v) for k, v in sc.items()}
        else:
            sc["means"][:, 2] = -2.0  # all behind the camera
        params = gs.scene_to_device(sc)
        pipe = gs.Pipeline(params, 40, 24, pair_capacity=16)
        pipe.project(cam)
        assert pipe.bin(cam) == 0
        pipe.forward(cam)
        torch.cuda.synchronize()
        img = pipe.image.cpu().numpy()
        assert np.allclose(img, np.array([0.3, 0.2, 0.1], np.float32)) and np.all(pipe.final_T.cpu().numpy() == 1)
        assert np.all(pipe.ranges.cpu().numpy() == 0)
        if n:
            pipe.dL_dimage.fill_(1.0)
            pipe.backward(cam)
            torch.cuda.synchronize()
            assert all(np.all(v.cpu().numpy() == 0) for v in pipe.grads.values())


@pytest.mark.parametrize("visible_every", [10, 997])
def test_large_frame_mostly_culled(env, visible_every):
    """Above 36,864 Gaussians the depth sort's first pass drops the culled ones and the later
    passes, the scan and the emission run on the drawn ones only: a scene where one Gaussian in
    10 (or in 997) is in front of the camera bins, blends and back-propagates like the oracle."""
    n, W, f = 60000, 200, 160.0
    scene = synth.random_scene(n, seed=61, width=W, height=W, focal=f)
    behind = np.arange(n) % visible_every != 0
    scene["means"][behind, 2] *= -1.0
    cam = synth.make_camera(np.eye(4), W, W, f, background=(0.2, 0.1, 0.3))
    _pipeline_case(env, scene, cam, pixels=synth.sample_pixels(W, W, 4096, seed=3),
                   label=f"mostly culled 1/{visible_every}", bwd="det")


def test_capacity_overflow_contract(env):
    # P > capacity: GS_ERR_CAPACITY with P in full (host and device), every range empty, nothing
    # written past the capacity; the same without the host wait; capacity 0 with n > 0
    gs, torch = env
    wl = synth.WORKLOADS["tiny_1k"]
    cam_d = synth.make_cameras(wl)[0]
    params, cam, proj = run_gpu_project(gs, torch, synth.make_scene(wl), cam_d)
    need = int(proj.tiles_touched.sum().item())
    tiles = ((cam.width + 15) // 16) * ((cam.height + 15) // 16)
    for cap in (need - 1, need // 3, 0):
        for wait in (True, False):
            print(f"capacity {cap} of {need}, wait={wait}", flush=True)
            keys = torch.full((cap + 64,), -7, device="cuda", dtype=torch.int64)
            ids = torch.full((cap + 64,), -7, device="cuda", dtype=torch.int32)
            ranges = torch.full((tiles, 2), -7, device="cuda", dtype=torch.int32)
            pdev = torch.full((1,), -7, device="cuda", dtype=torch.int64)
            plan = torch.full((gs.gs_raster_plan_words(cam),), -1, device="cuda", dtype=torch.int32)
            ws = torch.empty(gs.gs_bin_workspace_bytes(params["n"], cap, cam), device="cuda", dtype=torch.uint8)
            ws.fill_(0xAB)  # the workspace's contents on entry are arbitrary
            st, P = gs.gs_bin_and_sort(params["n"], proj, cam, ws, cap, keys, ids, ranges, pdev, wait=wait,
                                       plan=plan)
            torch.cuda.synchronize()
            if wait:
                assert st == gs.GS_ERR_CAPACITY and P == need
            else:
                assert st == gs.GS_OK and P is None
            assert int(pdev.item()) == need
            assert torch.all(ranges == 0)
            pl = plan.cpu().numpy().view(np.uint32)
            assert np.array_equal(np.sort(pl[4:4 + tiles]), np.arange(tiles)) and pl[1] == 0 and pl[2] == 0
            assert torch.all(keys[cap:] == -7) and torch.all(ids[cap:] == -7)


def test_async_bin_matches_waiting_bin(env):
    gs, torch = env
    wl = synth.WORKLOADS["distill_30k"]
    params = gs.scene_to_device(synth.make_scene(wl))
    cam = gs.make_camera(synth.make_cameras(wl)[9])
    pipe = gs.Pipeline(params, wl.width, wl.height, pair_capacity=1 << 10)
    pipe.project(cam)
    P = pipe.bin(cam)  # regrows from 1024 pairs
    keys, ids, ranges = pipe.keys[:P].clone(), pipe.ids[:P].clone(), pipe.ranges.clone()
    pipe.keys.fill_(-1)
    pipe.ranges.fill_(-1)
    pipe.bin_ws.fill_(0x5A)
    pipe.bin(cam, wait=False)
    torch.cuda.synchronize()
    assert int(pipe.num_pairs_dev.item()) == P
    assert torch.equal(pipe.keys[:P], keys) and torch.equal(pipe.ids[:P], ids) and torch.equal(pipe.ranges, ranges)


def test_invalid_arguments(env):
    gs, torch = env
    cam_d = synth.make_camera(np.eye(4), 32, 32, 40.0)
    params = gs.scene_to_device(synth.random_scene(10, seed=1))
    proj = gs.Projected.empty(10)
    cam = gs.make_camera(cam_d)
    with pytest.raises(gs.GsError) as e:
        gs.gs_project(10, 4, params["means"], params["log_scales"], params["quats"], params["opacity_logits"],
                      params["sh"], cam, proj)
    assert e.value.status == gs.GS_ERR_INVALID_ARG
    bad = gs.make_camera(dict(cam_d, width=0))
    with pytest.raises(gs.GsError):
        gs.gs_project(10, 0, params["means"], params["log_scales"], params["quats"], params["opacity_logits"],
                      params["sh"], bad, proj)
    nan_cam = gs.make_camera(dict(cam_d, fx=float("nan")))
    with pytest.raises(gs.GsError):
        gs.gs_project(10, 0, params["means"], params["log_scales"], params["quats"], params["opacity_logits"],
                      params["sh"], nan_cam, proj)
    with pytest.raises(gs.GsError):
        gs.gs_project(-1, 0, params["means"], params["log_scales"], params["quats"], params["opacity_logits"],
                      params["sh"], cam, proj)
    for field in ("radius_mode", "antialiased"):
        opt = gs.make_camera(cam_d)
        setattr(opt, field, 2)
        with pytest.raises(gs.GsError):
            gs.gs_project(10, 0, params["means"], params["log_scales"], params["quats"],
                          params["opacity_logits"], params["sh"], opt, proj)
    # too small a workspace
    keys = torch.empty(100, device="cuda", dtype=torch.int64)
    ids = torch.empty(100, device="cuda", dtype=torch.int32)
    ranges = torch.empty(4, 2, device="cuda", dtype=torch.int32)
    ws = torch.empty(16, device="cuda", dtype=torch.uint8)
    with pytest.raises(gs.GsError):
        gs.gs_bin_and_sort(10, proj, cam, ws, 100, keys, ids, ranges)


def test_huge_splat_and_tile_edges(env):
    # one splat covering every tile of a ragged grid, plus splats centred exactly on tile edges
    sc = {"means": np.array([[0.0, 0.0, 2.0], [0.0, 0.0, 3.0], [16.0 / 40 * 3, 0.0, 3.0], [0.0, -16.0 / 40 * 3, 3.0]]),
          "log_scales": np.array([[1.0] * 3, [-2.5] * 3, [-2.5] * 3, [-2.5] * 3]),
          "quats": np.tile([1.0, 0, 0, 0], (4, 1)), "opacity_logits": np.array([-1.0, 3.0, 3.0, 3.0]),
          "sh": np.random.default_rng(1).uniform(0, 1, (4, 1, 3)), "sh_degree": 0}
    cam = synth.make_camera(np.eye(4), 70, 40, 40.0)
    _pipeline_case(env, sc, cam, label="huge+edges")


@pytest.mark.parametrize("width,height", [(3000, 1100), (4200, 4200)])
def test_many_tiles(env, width, height):
    # 12,972 tiles: more than one step of the tile-count finalizer holds; 69,169 tiles: three
    # pair-sort passes (17 tile-id bits), histograms of digits 1 and 2 from run boundaries
    sc = synth.random_scene(3000, seed=width, width=width, height=height, focal=width / 2.0)
    cam = synth.make_camera(np.eye(4), width, height, width / 2.0)
    pix = synth.sample_pixels(width, height, 4096, seed=5)
    _pipeline_case(env, sc, cam, pixels=pix, label=f"tiles {width}x{height}")


@pytest.mark.parametrize("n,tight", [(4096, False), (4097, True), (20000, False), (36864, False), (36864, True),
                                     (36865, False)])
def test_depth_order_block_sizes_ties_and_culled(env, n, tight):
    """Frames of at most 36,864 Gaussians take their depth order from sorted blocks of 4096 and
    merge ranks, larger ones from the radix passes: sizes at and across the block and path
    boundaries, a third of the Gaussians at one exactly equal depth (stable: ascending id), a tenth
    behind the camera and some fully transparent (not drawn, no pairs)."""
    sc = synth.random_scene(n, seed=n, width=640, height=360, focal=400.0, log_scales=(-4.5, -2.5))
    rng = np.random.default_rng(n + 1)
    sc["means"][rng.random(n) < 0.33, 2] = 3.25
    sc["means"][rng.random(n) < 0.1, 2] = -1.0
    sc["opacity_logits"][rng.random(n) < 0.05] = -30.0
    cam = synth.make_camera(np.eye(4), 640, 360, 400.0)
    if tight:
        cam["tight_tiles"] = True
    pix = synth.sample_pixels(640, 360, 4096, seed=3)
    _pipeline_case(env, sc, cam, pixels=pix, label=f"blocks n={n} tight={tight}")


def test_opacity_extremes(env):
    sc = synth.random_scene(200, seed=8, width=48, height=48, focal=50.0)
    sc["opacity_logits"][:40] = 30.0
    sc["opacity_logits"][40:60] = -30.0
    _pipeline_case(env, sc, synth.make_camera(np.eye(4), 48, 48, 50.0, background=(1.0, 1.0, 1.0)), label="opacity")


def test_forward_and_sort_deterministic(env):
    # the same schedule twice: bit-identical; chunked (per-chunk colour sums) vs whole tiles: the
    # same sort and contributor counts, images equal up to the order of the colour additions
    gs, torch = env
    wl = synth.WORKLOADS["distill_30k"]
    params = gs.scene_to_device(synth.make_scene(wl))
    cam = gs.make_camera(synth.make_cameras(wl)[5])
    pipe = gs.Pipeline(params, wl.width, wl.height, pair_capacity=1 << 18)
    outs = []
    for schedule in ("chunks", "chunks", "tiles"):
        pipe.schedule = schedule
        pipe.project(cam)
        pipe.bin(cam)
        pipe.forward(cam)
        torch.cuda.synchronize()
        outs.append((pipe.keys[:pipe.num_pairs].clone(), pipe.ids[:pipe.num_pairs].clone(), pipe.image.clone(),
                     pipe.n_contrib.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for i, (a, b) in enumerate(zip(outs[0], outs[2])):
        if i == 2:
            assert torch.allclose(a, b, rtol=0, atol=1e-6)
        else:
            assert torch.equal(a, b)


def test_loss_l1(env):
    gs, torch = env
    rng = np.random.default_rng(2)
    img = rng.uniform(0, 1, (37, 23, 3)).astype(np.float32)
    tgt = rng.uniform(0, 1, (37, 23, 3)).astype(np.float32)
    tgt[0, 0] = img[0, 0]  # sign(0) = 0
    dimg = torch.empty(37, 23, 3, device="cuda")
    loss = torch.empty(1, device="cuda")
    gs.gs_loss_l1(23, 37, torch.from_numpy(img).cuda(), torch.from_numpy(tgt).cuda(), dimg, loss)
    torch.cuda.synchronize()
    want = np.sign(img.astype(np.float64) - tgt) / img.size
    assert np.allclose(dimg.cpu().numpy(), want, rtol=1e-6, atol=0)
    assert loss.item() == pytest.approx(np.abs(img.astype(np.float64) - tgt).mean(), rel=1e-5)
    # arrays that are 4- but not 16-byte aligned (a target image inside a batch of odd-sized ones)
    big_i = torch.from_numpy(np.concatenate([[0.0], img.ravel()]).astype(np.float32)).cuda()
    big_t = torch.from_numpy(np.concatenate([[0.0], tgt.ravel()]).astype(np.float32)).cuda()
    big_g = torch.zeros(img.size + 1, device="cuda")
    gs.gs_loss_l1(23, 37, big_i[1:], big_t[1:], big_g[1:], loss)
    torch.cuda.synchronize()
    assert np.allclose(big_g[1:].cpu().numpy(), want.ravel(), rtol=1e-6, atol=0) and big_g[0].item() == 0.0
    assert loss.item() == pytest.approx(np.abs(img.astype(np.float64) - tgt).mean(), rel=1e-5)


@pytest.mark.parametrize("W,H,lam", [(37, 23, 0.2), (128, 128, 0.2), (980, 545, 0.2), (64, 48, 1.0), (64, 48, 0.0)])
def test_loss_l1_ssim(env, W, H, lam):
    """gs_loss_l1_ssim against the loss oracle (float64): the loss value and dL/dimage. The
    statistics run in fp32 (window sums of 121 terms, variances as e_xx - mu^2, hardware
    reciprocals), hence a tolerance of 1e-4 of each element plus 1e-4 of the largest SSIM-part
    magnitude."""
    from oracle import loss as oloss
    gs, torch = env
    rng = np.random.default_rng(W * 7 + H)
    x = rng.uniform(0, 1, (H, W, 3)).astype(np.float32)
    # a target that shares structure with the image (smooth blend plus noise), so S spans a range
    y = np.clip(0.6 * x + 0.4 * np.roll(x, 3, axis=1) + rng.normal(0, 0.05, x.shape), 0, 1).astype(np.float32)
    y[: H // 4] = x[: H // 4]  # a band of equal values: sign(0) = 0 and S = 1 there
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    ws = torch.empty(gs.gs_loss_ssim_workspace_bytes(W, H), device="cuda", dtype=torch.uint8)
    grad = torch.empty_like(xd)
    loss = torch.empty(1, device="cuda")
    gs.gs_loss_l1_ssim(W, H, xd, yd, lam, ws, grad, loss)
    torch.cuda.synchronize()
    val_ref, g_ref = oloss.loss_l1_ssim(x.astype(np.float64), y.astype(np.float64), lam)
    g = grad.cpu().numpy().astype(np.float64)
    ssim_part = g_ref - (1 - lam) * np.sign(x.astype(np.float64) - y.astype(np.float64)) / x.size
    tol = 1e-4 * np.abs(g_ref) + 1e-4 * np.abs(ssim_part).max() + 1e-12
    err = np.abs(g - g_ref)
    log(f"[loss_ssim {W}x{H} lam={lam}] loss {loss.item():.7f} vs {val_ref:.7f}; grad max err/tol "
        f"{(err / tol).max():.3f}")
    assert np.all(err <= tol)
    assert abs(loss.item() - val_ref) <= 1e-5 * abs(val_ref) + 1e-6
    # the loss value is summed in a fixed order: the same bits again
    first = loss.clone()
    ws.random_(0, 256)
    gs.gs_loss_l1_ssim(W, H, xd, yd, lam, ws, grad, loss)
    torch.cuda.synchronize()
    assert torch.equal(first, loss)


def test_concurrent_streams_match_sequential(env):
    """Camera iterations on four streams at once (own buffers, shared Gaussians, as the bench runs
    them) give the same images bit for bit, and the same deterministic gradients, as one at a time."""
    gs, torch = env
    wl = synth.WORKLOADS["distill_30k"]
    params = gs.scene_to_device(synth.make_scene(wl))
    cams = [gs.make_camera(c) for c in synth.make_cameras(wl)[:8]]
    tg = torch.rand(8, wl.height, wl.width, 3, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    pipes = [gs.Pipeline(params, wl.width, wl.height, pair_capacity=1 << 18) for _ in range(4)]
    for p in pipes:
        p.deterministic = True
    streams = [torch.cuda.Stream() for _ in range(4)]

    def run(i, k, st):
        with torch.cuda.stream(st):
            pipes[k].iteration(cams[i], tg[i], stream=st, wait=False)

    ref = []
    for i in range(8):
        run(i, 0, torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append((pipes[0].image.clone(), {k: v.clone() for k, v in pipes[0].grads.items()}))
    for first in (0, 4):
        for k in range(4):
            run(first + k, k, streams[k])
        torch.cuda.synchronize()
        for k in range(4):
            img, grads = ref[first + k]
            assert torch.equal(pipes[k].image, img), f"camera {first + k}: image differs"
            for name, v in grads.items():
                assert torch.equal(pipes[k].grads[name], v), f"camera {first + k}: {name} differs"


@pytest.mark.parametrize("name,depth", [("mid_150k_sh3", False), ("mid_150k_sh3", True), ("deep", False)])
def test_chunked_forward_matches_whole_tiles(env, name, depth):
    """A training forward (plan and raster workspace) blends the chunks of each tile of three or
    more chunks at once, every chunk starting from the product of the earlier chunks'
    transmittance factors. Its pixels match one workgroup per tile within rounding (the last
    added entry too, off the pixels whose stop decision sits within rounding of 1e-4), a second
    call gives the same bits, and the call leaves the workspace's synchronisation words zero."""
    gs, torch = env
    if name == "deep":
        # 40,000 splats over a ragged 150 x 90 image: tiles of thousands of entries (many chunks)
        W, H = 150, 90
        scene = synth.random_scene(40000, seed=51, width=W, height=H, focal=110.0, logit_std=1.5)
        cam = gs.make_camera(synth.make_camera(np.eye(4), W, H, 110.0, background=(0.3, 0.2, 0.1)))
    else:
        wl = synth.WORKLOADS[name]
        W, H, scene = wl.width, wl.height, synth.make_scene(wl)
        cam = gs.make_camera(synth.make_cameras(wl)[0])
    params = gs.scene_to_device(scene)
    p = gs.Pipeline(params, W, H, pair_capacity=1 << 20)
    p.project(cam)
    p.bin(cam)
    plan = p.plan.cpu().numpy().view(np.uint32)
    lens = np.diff(p.ranges.cpu().numpy().view(np.uint32).astype(np.int64), axis=1)[:, 0]
    nch = -(-lens // int(plan[0]))
    log(f"[{name}] L={plan[0]} tiles of >= 3 chunks: {(nch >= 3).sum()}, longest {nch.max()} chunks")
    assert (nch >= 3).sum() >= 10
    outs = []
    for ck in (False, True, True):
        dep = torch.empty(H, W, device="cuda") if depth else None
        p.forward(cam, checkpoints=ck, depth=dep)
        torch.cuda.synchronize()
        outs.append((p.image.clone(), p.final_T.clone(), p.n_contrib.clone(), dep))
        if ck:
            sync = p.raster_ws[-gs.raster_sync_bytes():]
            assert int(torch.count_nonzero(sync)) == 0, "synchronisation words left set"
    for a, b in zip(outs[1], outs[2]):
        assert a is None or torch.equal(a, b), "two chunked forwards differ"
    img0, T0, nc0, d0 = (x.cpu().numpy() if x is not None else None for x in outs[0])
    img1, T1, nc1, d1 = (x.cpu().numpy() if x is not None else None for x in outs[1])
    same = nc0 == nc1
    assert same.mean() >= 0.999, f"{(~same).sum()} pixels end at another entry"
    assert np.abs(img1 - img0)[same].max() <= 1e-5
    assert np.abs(T1 - T0)[same].max() <= 1e-6
    assert np.abs(img1 - img0).max() <= 1e-4 + 1e-6
    if depth:
        assert np.abs(d1 - d0)[same].max() <= 1e-5 * max(1.0, float(np.abs(d0).max()))
    log(f"[{name}] chunked forward: {(~same).sum()} pixels end at another entry, max |diff| "
        f"{np.abs(img1 - img0).max():.2e}")


@pytest.mark.parametrize("case", ["distill_30k", "ragged"])
def test_fused_l1_forward(env, case):
    """gs_rasterize_fwd_l1: the image, final T and counts are those of gs_rasterize_fwd, and the
    gradient it writes is gs_loss_l1's on that image, bit for bit; the L1 value it implies
    matches the oracle loss on the same image."""
    from oracle import loss as oloss
    gs, torch = env
    if case == "ragged":
        scene = synth.random_scene(300, seed=51, width=37, height=23, focal=30.0)
        cam_d = synth.make_camera(np.eye(4), 37, 23, 30.0, background=(0.2, 0.4, 0.6))
    else:
        wl = synth.WORKLOADS[case]
        scene, cam_d = synth.make_scene(wl), synth.make_cameras(wl)[3]
    W, H = cam_d["width"], cam_d["height"]
    cam = gs.make_camera(cam_d)
    params = gs.scene_to_device(scene)
    pipe = gs.Pipeline(params, W, H, pair_capacity=1 << 10)
    pipe.project(cam)
    pipe.bin(cam)
    rng = np.random.default_rng(52)
    target = torch.from_numpy(rng.uniform(0, 1, (H, W, 3)).astype(np.float32)).cuda()
    pipe.forward(cam)
    ref_img, ref_T, ref_nc = pipe.image.clone(), pipe.final_T.clone(), pipe.n_contrib.clone()
    ref_grad = torch.empty_like(ref_img)
    gs.gs_loss_l1(W, H, ref_img, target, ref_grad)
    pipe.dL_dimage.fill_(float("nan"))
    pipe.image.zero_()
    pipe.forward(cam, l1_target=target)
    torch.cuda.synchronize()
    assert torch.equal(pipe.image, ref_img) and torch.equal(pipe.final_T, ref_T)
    assert torch.equal(pipe.n_contrib, ref_nc)
    assert torch.equal(pipe.dL_dimage, ref_grad), "fused L1 gradient differs from gs_loss_l1"
    _, g_ref = oloss.loss_l1_ssim(ref_img.cpu().numpy().astype(np.float64), target.cpu().numpy().astype(np.float64),
                                  0.0)
    assert np.array_equal(pipe.dL_dimage.cpu().numpy().astype(np.float64), g_ref.astype(np.float32))
    # a NULL target is an argument error
    with pytest.raises(gs.GsError):
        gs.gs_rasterize_fwd_l1(pipe.n, pipe.proj, cam, pipe.ids, pipe.ranges, pipe.image, pipe.final_T,
                               pipe.n_contrib, None, pipe.dL_dimage)


@pytest.mark.parametrize("case,C,det", [("ragged", 2, False), ("tiny", 3, True), ("tiny", 1, False)])
def test_feature_channels(env, case, C, det):
    """Per-Gaussian features [n, C] blended with the colour's weights (background 0) and their
    backward, against the oracle run on the same geometry with the features as degree-0 colours:
    the rendered channels (1e-4 off the fragile pixels), dL/dfeatures and the geometry's share of
    the gradients (the stated gradient tolerance)."""
    gs, torch = env
    if case == "ragged":
        scene = synth.random_scene(300, seed=61, width=37, height=23, focal=30.0, sh_degree=3, logit_std=2.0)
        cam_d = synth.make_camera(np.eye(4), 37, 23, 30.0, background=(0.2, 0.4, 0.6))
    else:
        wl = synth.WORKLOADS["tiny_1k"]
        scene, cam_d = synth.make_scene(wl), synth.make_cameras(wl)[0]
    W, H = cam_d["width"], cam_d["height"]
    n = scene["means"].shape[0]
    rng = np.random.default_rng(62)
    feats = rng.normal(0, 1, (n, C)).astype(np.float32)
    cam = gs.make_camera(cam_d)
    params = gs.scene_to_device(scene)
    pipe = gs.Pipeline(params, W, H, pair_capacity=1 << 12)
    pipe.deterministic = det
    pipe.project(cam)
    pipe.bin(cam)
    pipe.forward(cam)
    fd = torch.from_numpy(feats).cuda()
    F = pipe.render_features(cam, fd).cpu().numpy()
    # the oracle: the same Gaussians with the features as view-independent colours, background 0
    f3 = np.zeros((n, 1, 3), np.float32)
    f3[:, 0, :C] = feats
    scene_f = dict(scene, sh=f3, sh_degree=0)
    cam_f = dict(cam_d, background=(0.0, 0.0, 0.0))
    o_proj = oracle.project(scene_f, cam_f, np.float32)
    o_fwd = oracle.render(o_proj, cam_f)
    ok = ~o_fwd["fragile"]
    d = np.abs(F.astype(np.float64) - o_fwd["image"][..., :C])
    assert d[ok].max() <= 1e-4, f"feature channels differ by {d[ok].max():.3e}"
    gF = rng.normal(0, 1, (H, W, C)).astype(np.float32)
    gF[~ok] = 0.0  # no gradient where a decision sits on its threshold
    out = pipe.features_backward(cam, fd, torch.from_numpy(gF).cuda())
    torch.cuda.synchronize()
    g3 = np.zeros((H, W, 3))
    g3[..., :C] = gF
    _, _, _, raw = oracle_grads(scene_f, cam_f, o_proj, g3)
    gsh = np.zeros((n, 1, 3), np.float32)
    gsh[:, 0, :C] = out["features"].cpu().numpy()
    gpu = {k: out[k].cpu().numpy() for k in ("means", "log_scales", "quats", "opacity_logits")}
    gpu["sh"] = gsh
    compare_grads(gpu, raw, 0, f"features {case} C={C}")
