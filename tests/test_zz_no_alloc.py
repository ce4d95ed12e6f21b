"""The allocation-free binning entry point (gs_bin_and_sort_noalloc, for callers that cannot
allocate: code under graph capture, tight loops) gives what gs_bin_and_sort gives with a
caller-allocated workspace, bit for bit: pair count, sorted keys and ids and tile ranges; the
raster plan's header (chunk length, extra work items, checkpoint slots) is equal and both plans
are valid (the order of tiles within a count class and the slot assignment are not unique). Two calls in a row share the static workspace, the second on a smaller frame, so
state left by the first call must not leak into the second. A frame whose workspace exceeds the
static maximum is refused with an error, before any work is enqueued."""
import numpy as np
import pytest

from gaussian_splatting_tile_gs_amd import synth
from _gpu_util import assert_raster_plan

pytestmark = pytest.mark.gpu


def _bin_both(gs, torch, scene, cam_d, capacity):
    params = gs.scene_to_device(scene)
    n = params["n"]
    cam = gs.make_camera(cam_d)
    proj = gs.Projected.empty(n)
    gs.gs_project(n, params["sh_degree"], params["means"], params["log_scales"], params["quats"],
                  params["opacity_logits"], params["sh"], cam, proj)
    tiles = ((cam_d["width"] + 15) // 16) * ((cam_d["height"] + 15) // 16)
    out = []
    for noalloc in (False, True):
        keys = torch.full((capacity,), -1, device="cuda", dtype=torch.int64)
        ids = torch.full((capacity,), -1, device="cuda", dtype=torch.int32)
        ranges = torch.full((tiles, 2), -1, device="cuda", dtype=torch.int32)
        plan = torch.full((gs.gs_raster_plan_words(cam),), -1, device="cuda", dtype=torch.int32)
        P = torch.zeros(1, device="cuda", dtype=torch.int64)
        if noalloc:
            gs.gs_bin_and_sort_noalloc(n, proj, cam, capacity, keys, ids, ranges, P, plan=plan)
        else:
            ws = torch.empty(gs.gs_bin_workspace_bytes(n, capacity, cam), device="cuda", dtype=torch.uint8)
            gs.gs_bin_and_sort(n, proj, cam, ws, capacity, keys, ids, ranges, P, wait=False, plan=plan)
        torch.cuda.synchronize()
        Pn = int(P.item())
        out.append((Pn, keys[:Pn].cpu().numpy(), ids[:Pn].cpu().numpy(), ranges.cpu().numpy(), plan.cpu().numpy(),
                    (cam_d["width"] + 15) // 16))
    return out


def _check_equal(a, b):
    assert a[0] == b[0] > 0
    for x, y, what in zip(a[1:4], b[1:4], ("keys", "ids", "ranges")):
        assert np.array_equal(x, y), what
    assert np.array_equal(a[4][:4], b[4][:4]), "plan header"
    for r in (a, b):
        assert_raster_plan(r[4], r[3].view(np.uint32), r[0], r[5])


def test_noalloc_matches_workspace_binning_twice(env_gpu):
    gs, torch = env_gpu
    big = synth.WORKLOADS["distill_30k"]
    first = _bin_both(gs, torch, synth.make_scene(big), synth.make_cameras(big)[3], 200_000)
    _check_equal(*first)
    small = synth.WORKLOADS["tiny_1k"]
    second = _bin_both(gs, torch, synth.make_scene(small), synth.make_cameras(small)[0], 8192)
    _check_equal(*second)
    assert second[0][0] < first[0][0]


def test_noalloc_refuses_a_frame_above_its_maximum(env_gpu):
    gs, torch = env_gpu
    wl = synth.WORKLOADS["stress_400k_sh3"]
    cam = gs.make_camera(synth.make_cameras(wl)[0])
    cap = 20_000_000
    assert gs.gs_bin_workspace_bytes(wl.n, cap, cam) > gs.gs_bin_noalloc_max_workspace_bytes()
    proj = gs.Projected.empty(wl.n)
    keys = torch.empty(1, device="cuda", dtype=torch.int64)
    ids = torch.empty(1, device="cuda", dtype=torch.int32)
    ranges = torch.empty(cam.width * cam.height // 256 + 512, 2, device="cuda", dtype=torch.int32)
    P = torch.zeros(1, device="cuda", dtype=torch.int64)
    with pytest.raises(gs.GsError) as e:
        gs.gs_bin_and_sort_noalloc(wl.n, proj, cam, cap, keys, ids, ranges, P)
    assert e.value.status == gs.GS_ERR_LIMIT


@pytest.fixture(scope="module")
def env_gpu():
    import torch

    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    from gaussian_splatting_tile_gs_amd import gs

    gs.load()
    return gs, torch
