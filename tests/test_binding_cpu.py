"""Host logic of the binding's Pipeline (CPU only: the entry points are replaced by recorders, so no
kernel runs). The backward may split long tiles at the forward's checkpoints only when the
checkpoints hold everything the chunked backward reads: with a depth gradient, the depth
channel's parts too."""
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
