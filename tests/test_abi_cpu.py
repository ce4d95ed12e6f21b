"""The C-ABI library loads and exports every entry point include/gs.h declares (CPU only: no
compute call is made), and the host-only size helpers behave."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gs.h")
LIB = os.path.join(ROOT, "gaussian_splatting_tile_gs_amd", "libgs_hip.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from gaussian_splatting_tile_gs_amd import build

        build.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gs_project", "gs_bin_and_sort", "gs_rasterize_fwd", "gs_rasterize_bwd"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_host_only_helpers(lib):
    lib.gs_status_string.restype = ctypes.c_char_p
    lib.gs_status_string.argtypes = [ctypes.c_int]
    assert lib.gs_status_string(2) == b"GS_ERR_CAPACITY"
    lib.gs_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_bwd_workspace_bytes.argtypes = [ctypes.c_int32]
    assert lib.gs_bwd_workspace_bytes(1000) >= 1000 * 10 * 4
    from gaussian_splatting_tile_gs_amd import gs

    cam = gs.GsCamera()
    cam.width, cam.height = 1280, 720
    lib.gs_bin_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_bin_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(gs.GsCamera)]
    small = lib.gs_bin_workspace_bytes(1000, 10000, ctypes.byref(cam))
    big = lib.gs_bin_workspace_bytes(1000, 1000000, ctypes.byref(cam))
    assert 0 < small < big
    lib.gs_adam_state_floats.restype = ctypes.c_size_t
    lib.gs_adam_state_floats.argtypes = [ctypes.c_int32, ctypes.c_int32]
    # groups of 3n, 3n, 4n, n and 3Kn values, each rounded up to 64 floats
    for n, deg in ((1000, 0), (1001, 3), (1, 1)):
        sizes = [3 * n, 3 * n, 4 * n, n, 3 * (deg + 1) ** 2 * n]
        assert lib.gs_adam_state_floats(n, deg) == sum(-(-c // 64) * 64 for c in sizes)
    assert lib.gs_adam_state_floats(0, 0) == 0 and lib.gs_adam_state_floats(10, 4) == 0
    lib.gs_bwd_det_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_bwd_det_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64]
    # 40 B per pair record (ten gradient components) on top of the per-Gaussian arrays; invalid
    # capacities give 0
    a, b = lib.gs_bwd_det_workspace_bytes(1000, 10000), lib.gs_bwd_det_workspace_bytes(1000, 20000)
    assert abs((b - a) - 40 * 10000) < 256 and a >= 1000 * 44 + 40 * 10000
    assert lib.gs_bwd_det_workspace_bytes(1000, -1) == 0 and lib.gs_bwd_det_workspace_bytes(1000, 1 << 30) == 0
    lib.gs_loss_ssim_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_loss_ssim_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
    # nine partial planes of h*w floats plus a float2 per 16x16 tile, each part 256-byte aligned
    assert lib.gs_loss_ssim_workspace_bytes(980, 545) >= 980 * 545 * 36 + 62 * 35 * 8
    assert lib.gs_loss_ssim_workspace_bytes(0, 10) == 0
    lib.gs_raster_workspace_bytes.restype = ctypes.c_size_t
    # per checkpoint slot (two per plan chunk) and pixel (256): (T, r, g, b), depth part, factor,
    # last entry; then the synchronisation words the binding finds at the end
    slots = 2 * gs.plan_max_chunks()
    assert slots >= 4096
    assert lib.gs_raster_workspace_bytes() == slots * 256 * 28 + gs.raster_sync_bytes()
