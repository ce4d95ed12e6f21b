"""Host logic of the binding's Pipeline (CPU only: the entry points are replaced by recorders, so no
kernel runs). The backward may split long tiles at the forward's checkpoints only when the
checkpoints hold everything the chunked backward reads: with a depth gradient, the depth
channel's parts too."""
import ctypes

import numpy as np
import pytest
import torch

from gaussian_splatting_tile_gs_amd import gs, synth


@pytest.fixture()
def pipe(monkeypatch):
    calls = []
    monkeypatch.setattr(gs, "gs_rasterize_fwd", lambda *a, **k: calls.append(("fwd", k)))
    monkeypatch.setattr(gs, "gs_rasterize_fwd_l1", lambda *a, **k: calls.append(("fwd_l1", k)))
    monkeypatch.setattr(gs, "gs_rasterize_bwd", lambda *a, **k: calls.append(("bwd", k)))
    sc = synth.random_scene(8, seed=1, width=32, height=32, focal=30.0)
    params = gs.scene_to_device(sc, device="cpu")
    p = gs.Pipeline(params, 32, 32, pair_capacity=64, device="cpu")
    p.calls = calls
    return p


def _cam():
    return gs.make_camera(synth.make_camera(np.eye(4), 32, 32, 30.0))


def test_backward_uses_checkpoints_of_a_colour_forward(pipe):
    cam = _cam()
    pipe.forward(cam)
    pipe.backward(cam)
    assert pipe.calls[-1][1]["raster_ws"] is pipe.raster_ws


def test_depth_backward_after_a_forward_without_depth_walks_whole_tiles(pipe):
    cam = _cam()
    pipe.forward(cam)  # checkpoints of the colour only
    pipe.backward(cam, dL_ddepth=torch.zeros(32, 32))
    assert pipe.calls[-1][1]["raster_ws"] is None


def test_depth_backward_after_a_depth_forward_uses_checkpoints(pipe):
    cam = _cam()
    pipe.forward(cam, depth=torch.zeros(32, 32))
    pipe.backward(cam, dL_ddepth=torch.zeros(32, 32))
    assert pipe.calls[-1][1]["raster_ws"] is pipe.raster_ws


def test_backward_after_a_forward_without_checkpoints(pipe):
    cam = _cam()
    pipe.forward(cam, checkpoints=False)
    pipe.backward(cam)
    assert pipe.calls[-1][1]["raster_ws"] is None


class _Recorder:
    """Stands in for the library: records every call's raw arguments (pointers as addresses,
    structs passed by reference as their bytes) and returns GS_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            norm = []
            for a in args:
                if isinstance(a, ctypes.c_void_p):
                    norm.append(("ptr", a.value))
                elif type(a).__name__ == "CArgObject":
                    norm.append(("ref", bytes(a._obj)))
                else:
                    norm.append(a)
            self.calls.append((name, tuple(norm)))
            return 0
        return f


@pytest.mark.parametrize("det", [False, True])
def test_cached_iteration_passes_the_same_arguments(monkeypatch, det):
    """Pipeline.iteration without a host wait takes its unchanging arguments from a cache; the
    library must see exactly the calls and arguments of the general path, also after the pair
    buffers grow."""
    rec = _Recorder()
    monkeypatch.setattr(gs, "load", lambda: rec)
    monkeypatch.setattr(gs, "_ptr", lambda t: None if t is None else ctypes.c_void_p(t.data_ptr()))
    monkeypatch.setattr(gs, "_stream", lambda s: ctypes.c_void_p(7))
    sc = synth.random_scene(8, seed=1, width=32, height=32, focal=30.0)
    p = gs.Pipeline(gs.scene_to_device(sc, device="cpu"), 32, 32, pair_capacity=64, device="cpu")
    p.deterministic = det
    cams = [_cam(), gs.make_camera(synth.make_camera(np.eye(4), 32, 32, 25.0))]
    tgts = [torch.zeros(32, 32, 3), torch.ones(32, 32, 3)]

    def general(cam, tgt):
        p.project(cam)
        p.bin(cam, wait=False)
        p.forward(cam, l1_target=tgt)
        p.backward(cam)

    for grow in (False, True):
        if grow:
            p.reserve_pairs(4096)
        for cam, tgt in zip(cams, tgts):
            rec.calls.clear()
            general(cam, tgt)
            want = [c for c in rec.calls if not c[0].endswith("workspace_bytes")]
            rec.calls.clear()
            p.iteration(cam, tgt, wait=False)
            got = [c for c in rec.calls if not c[0].endswith("workspace_bytes")]
            assert got == want
