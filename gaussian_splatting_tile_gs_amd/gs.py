"""ctypes binding of libgs_hip.so (include/gs.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does nothing but convert
torch CUDA tensors (device memory) and a torch stream into pointers, call the library and turn a
non-OK status into an exception. All arithmetic runs in the HIP kernels; there is no fallback:
if the library is missing, or no GPU is present, calls raise.

``Pipeline`` owns the device buffers of one scene/resolution and chains the entry points for a
forward+backward iteration (allocation and call order only).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # loads the HIP runtime the library binds to (same libamdhip64 soname)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgs_hip.so")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_CAPACITY, GS_ERR_LIMIT, GS_ERR_DEVICE = 0, 1, 2, 3, 4


class GsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_name(status)}: {msg}")
        self.status = status


class GsCamera(ctypes.Structure):
    _fields_ = [("viewmat", ctypes.c_float * 16), ("fx", ctypes.c_float), ("fy", ctypes.c_float),
                ("cx", ctypes.c_float), ("cy", ctypes.c_float), ("width", ctypes.c_int32),
                ("height", ctypes.c_int32), ("near_plane", ctypes.c_float), ("background", ctypes.c_float * 3),
                ("radius_mode", ctypes.c_int32), ("antialiased", ctypes.c_int32),
                ("tight_tiles", ctypes.c_int32)]


RADIUS_MODES = {"gsplat": 0, "3dgs": 1}


class GsProjected(ctypes.Structure):
    _fields_ = [("d_means2d", ctypes.c_void_p), ("d_conics", ctypes.c_void_p), ("d_depths", ctypes.c_void_p),
                ("d_opacities", ctypes.c_void_p), ("d_colors", ctypes.c_void_p), ("d_radii", ctypes.c_void_p),
                ("d_tiles_touched", ctypes.c_void_p)]


class GsAdamConfig(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("lr_means", "lr_log_scales", "lr_quats", "lr_opacity", "lr_sh_dc",
                                               "lr_sh_rest", "beta1", "beta2", "eps", "size_penalty")]


_lib = None


def load():
    """Load libgs_hip.so (built by gaussian_splatting_tile_gs_amd/build.py). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise GsError(GS_ERR_DEVICE, f"{LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cam_p, proj_p = ctypes.POINTER(GsCamera), ctypes.POINTER(GsProjected)
    sig = {
        "gs_project": (i32, [i32, i32, P, P, P, P, P, cam_p, proj_p, P]),
        "gs_bin_workspace_bytes": (sz, [i32, i64, cam_p]),
        "gs_raster_plan_words": (sz, [cam_p]),
        "gs_raster_workspace_bytes": (sz, []),
        "gs_bin_and_sort": (i32, [i32, proj_p, cam_p, P, sz, i64, P, P, P, P, P, ctypes.POINTER(ctypes.c_int64), P]),
        "gs_bin_noalloc_max_workspace_bytes": (sz, []),
        "gs_bin_and_sort_noalloc": (i32, [i32, proj_p, cam_p, i64, P, P, P, P, P, P]),
        "gs_rasterize_fwd": (i32, [i32, proj_p, cam_p, P, P, P, P, P, P, P, P, P, P]),
        "gs_rasterize_fwd_l1": (i32, [i32, proj_p, cam_p, P, P, P, P, P, P, P, P, P, P, P, P]),
        "gs_bwd_workspace_bytes": (sz, [i32]),
        "gs_bwd_det_workspace_bytes": (sz, [i32, i64]),
        "gs_rasterize_bwd_deterministic": (i32, [i32, i32, P, P, P, P, P, cam_p, proj_p, P, P, P, P, P, P, P, P,
                                                 i64, P, sz, P, P, P, P, P, P, P, P]),
        "gs_rasterize_bwd": (i32, [i32, i32, P, P, P, P, P, cam_p, proj_p, P, P, P, P, P, P, P, P, P, sz, P, P, P, P,
                                   P, P, P, P]),
        "gs_loss_l1": (i32, [i32, i32, P, P, P, P, P]),
        "gs_loss_ssim_workspace_bytes": (sz, [i32, i32]),
        "gs_loss_l1_ssim": (i32, [i32, i32, P, P, ctypes.c_float, P, sz, P, P, P]),
        "gs_adam_state_floats": (sz, [i32, i32]),
        "gs_adam_step": (i32, [i32, i32, i32, ctypes.POINTER(GsAdamConfig)] + [P] * 12 + [P]),
        "gs_status_string": (ctypes.c_char_p, [i32]),
        "gs_last_error": (ctypes.c_char_p, []),
        "gs_timing_enable": (i32, [i32]),
        "gs_timing_collect": (i32, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(status: int) -> str:
    try:
        return load().gs_status_string(status).decode()
    except GsError:
        return f"status {status}"


def _check(status: int, allow=()):
    if status != GS_OK and status not in allow:
        raise GsError(status, load().gs_last_error().decode())
    return status


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise GsError(GS_ERR_INVALID_ARG, "expected a contiguous CUDA tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_camera(cam: dict) -> GsCamera:
    """GsCamera from a camera dict (viewmat [4,4], fx, fy, cx, cy, width, height, near, background;
    optional radius_mode "gsplat" (default) or "3dgs", antialiased (default False), tight_tiles
    (default False: the whole tile rectangle; True: only the tiles the splat's ellipse reaches))."""
    c = GsCamera()
    v = np.asarray(cam["viewmat"], np.float32).reshape(16)
    for i in range(16):
        c.viewmat[i] = float(v[i])
    c.fx, c.fy, c.cx, c.cy = float(cam["fx"]), float(cam["fy"]), float(cam["cx"]), float(cam["cy"])
    c.width, c.height = int(cam["width"]), int(cam["height"])
    c.near_plane = float(cam.get("near", 0.01))
    bg = cam.get("background", (0.0, 0.0, 0.0))
    for i in range(3):
        c.background[i] = float(bg[i])
    c.radius_mode = RADIUS_MODES[cam.get("radius_mode", "gsplat")]
    c.antialiased = 1 if cam.get("antialiased", False) else 0
    c.tight_tiles = 1 if cam.get("tight_tiles", False) else 0
    return c


# ---- the entry points -------------------------------------------------------------------------
def gs_project(n, sh_degree, means, log_scales, quats, opacity_logits, sh, cam: GsCamera, out: "Projected",
               stream=None):
    return _check(load().gs_project(n, sh_degree, _ptr(means), _ptr(log_scales), _ptr(quats), _ptr(opacity_logits),
                                    _ptr(sh), ctypes.byref(cam), ctypes.byref(out.struct()), _stream(stream)))


def gs_bin_workspace_bytes(n, pair_capacity, cam: GsCamera) -> int:
    return int(load().gs_bin_workspace_bytes(n, pair_capacity, ctypes.byref(cam)))


def gs_raster_plan_words(cam: GsCamera) -> int:
    return int(load().gs_raster_plan_words(ctypes.byref(cam)))


def plan_max_chunks() -> int:
    """The most extra work items a raster plan holds, M (the plan is 4 + 2 tiles + 2 M + 2 (M / 2)
    words: the items, then the training forward's split chunks)."""
    cam = GsCamera()
    cam.width, cam.height = 16, 16
    return (gs_raster_plan_words(cam) - 4 - 2) // 3


def raster_sync_bytes() -> int:
    """The end of the raster workspace: the chunked forward's synchronisation words (two counters,
    then an arrival counter and a flag per checkpoint slot, two slots per plan chunk), zero
    between calls."""
    return 4 * (2 + 2 * 2 * plan_max_chunks())


def gs_raster_workspace_bytes() -> int:
    return int(load().gs_raster_workspace_bytes())


def gs_bin_and_sort(n, proj: "Projected", cam: GsCamera, workspace, pair_capacity, keys, ids, tile_ranges,
                    num_pairs_dev=None, stream=None, wait=True, plan=None):
    """With wait=True returns (status, P): status is GS_OK or GS_ERR_CAPACITY (P = the count
    needed). With wait=False nothing waits and it returns (GS_OK, None); P goes to num_pairs_dev
    (a one-element int64 CUDA tensor) when given."""
    P = ctypes.c_int64(0)
    st = _check(load().gs_bin_and_sort(n, ctypes.byref(proj.struct()), ctypes.byref(cam), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), pair_capacity, _ptr(keys),
                                       _ptr(ids), _ptr(tile_ranges), _ptr(plan), _ptr(num_pairs_dev),
                                       ctypes.byref(P) if wait else None, _stream(stream)),
                allow=(GS_ERR_CAPACITY,))
    return st, (int(P.value) if wait else None)


def gs_bin_noalloc_max_workspace_bytes() -> int:
    return int(load().gs_bin_noalloc_max_workspace_bytes())


def gs_bin_and_sort_noalloc(n, proj: "Projected", cam: GsCamera, pair_capacity, keys, ids, tile_ranges,
                            num_pairs_dev, stream=None, plan=None):
    """gs_bin_and_sort with the library's static workspace: no allocation and no host wait; P
    goes to num_pairs_dev (a one-element int64 CUDA tensor)."""
    return _check(load().gs_bin_and_sort_noalloc(n, ctypes.byref(proj.struct()), ctypes.byref(cam), pair_capacity,
                                                 _ptr(keys), _ptr(ids), _ptr(tile_ranges), _ptr(plan),
                                                 _ptr(num_pairs_dev), _stream(stream)))


def gs_rasterize_fwd(n, proj: "Projected", cam: GsCamera, ids, tile_ranges, image, final_T, n_contrib,
                     eval_count=None, stream=None, plan=None, raster_ws=None, depth=None):
    """depth: optional [h,w] output of the depth channel."""
    return _check(load().gs_rasterize_fwd(n, ctypes.byref(proj.struct()), ctypes.byref(cam), _ptr(ids),
                                          _ptr(tile_ranges), _ptr(plan), _ptr(raster_ws), _ptr(image), _ptr(depth),
                                          _ptr(final_T), _ptr(n_contrib), _ptr(eval_count), _stream(stream)))


def gs_rasterize_fwd_l1(n, proj: "Projected", cam: GsCamera, ids, tile_ranges, image, final_T, n_contrib, target,
                        dL_dimage, eval_count=None, stream=None, plan=None, raster_ws=None, depth=None):
    """gs_rasterize_fwd with the L1 gradient sign(image - target) / (3 h w) written into dL_dimage."""
    return _check(load().gs_rasterize_fwd_l1(n, ctypes.byref(proj.struct()), ctypes.byref(cam), _ptr(ids),
                                             _ptr(tile_ranges), _ptr(plan), _ptr(raster_ws), _ptr(image),
                                             _ptr(depth), _ptr(final_T), _ptr(n_contrib), _ptr(target),
                                             _ptr(dL_dimage), _ptr(eval_count), _stream(stream)))


def gs_bwd_workspace_bytes(n) -> int:
    return int(load().gs_bwd_workspace_bytes(n))


def gs_bwd_det_workspace_bytes(n, pair_capacity) -> int:
    return int(load().gs_bwd_det_workspace_bytes(n, pair_capacity))


def gs_rasterize_bwd(n, sh_degree, means, log_scales, quats, opacity_logits, sh, cam: GsCamera, proj: "Projected",
                     ids, tile_ranges, final_T, n_contrib, dL_dimage, workspace, grad_means, grad_log_scales,
                     grad_quats, grad_opacity_logits, grad_sh, grad_means2d=None, eval_count=None, stream=None,
                     plan=None, raster_ws=None, pair_capacity=None, dL_ddepth=None):
    """pair_capacity=None: gs_rasterize_bwd (fp32 atomics); else gs_rasterize_bwd_deterministic.
    dL_ddepth: optional [h,w] gradient on the depth channel."""
    if pair_capacity is not None:
        return _check(load().gs_rasterize_bwd_deterministic(
            n, sh_degree, _ptr(means), _ptr(log_scales), _ptr(quats), _ptr(opacity_logits), _ptr(sh),
            ctypes.byref(cam), ctypes.byref(proj.struct()), _ptr(ids), _ptr(tile_ranges), _ptr(plan),
            _ptr(raster_ws), _ptr(final_T), _ptr(n_contrib), _ptr(dL_dimage), _ptr(dL_ddepth), int(pair_capacity),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(grad_means), _ptr(grad_log_scales),
            _ptr(grad_quats), _ptr(grad_opacity_logits), _ptr(grad_sh), _ptr(grad_means2d), _ptr(eval_count),
            _stream(stream)))
    return _check(load().gs_rasterize_bwd(
        n, sh_degree, _ptr(means), _ptr(log_scales), _ptr(quats), _ptr(opacity_logits), _ptr(sh), ctypes.byref(cam),
        ctypes.byref(proj.struct()), _ptr(ids), _ptr(tile_ranges), _ptr(plan), _ptr(raster_ws), _ptr(final_T),
        _ptr(n_contrib), _ptr(dL_dimage), _ptr(dL_ddepth),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(grad_means), _ptr(grad_log_scales),
        _ptr(grad_quats), _ptr(grad_opacity_logits), _ptr(grad_sh), _ptr(grad_means2d), _ptr(eval_count),
        _stream(stream)))


def gs_loss_l1(width, height, image, target, dL_dimage, loss=None, stream=None):
    return _check(load().gs_loss_l1(width, height, _ptr(image), _ptr(target), _ptr(dL_dimage), _ptr(loss),
                                    _stream(stream)))


def gs_loss_ssim_workspace_bytes(width, height) -> int:
    return int(load().gs_loss_ssim_workspace_bytes(width, height))


def gs_loss_l1_ssim(width, height, image, target, lam, workspace, dL_dimage, loss=None, stream=None):
    return _check(load().gs_loss_l1_ssim(width, height, _ptr(image), _ptr(target), float(lam), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(dL_dimage), _ptr(loss),
                                         _stream(stream)))


def gs_timing_enable(on: bool):
    return _check(load().gs_timing_enable(1 if on else 0))


def gs_timing_collect(max_records=4096):
    names = (ctypes.c_char_p * max_records)()
    ms = (ctypes.c_float * max_records)()
    k = load().gs_timing_collect(names, ms, max_records)
    return [(names[i].decode(), float(ms[i])) for i in range(k)]


# ---- buffers ------------------------------------------------------------------------------------
def adam_config(lr_means=1.6e-4, lr_log_scales=5e-3, lr_quats=1e-3, lr_opacity=2.5e-2, lr_sh_dc=2.5e-3,
                lr_sh_rest=2.5e-3 / 20.0, beta1=0.9, beta2=0.999, eps=1e-15, size_penalty=0.0) -> GsAdamConfig:
    """Adam settings; the defaults are 3DGS's per-parameter rates (means: times the scene extent)."""
    return GsAdamConfig(lr_means, lr_log_scales, lr_quats, lr_opacity, lr_sh_dc, lr_sh_rest, beta1, beta2, eps,
                        size_penalty)


def gs_adam_state_floats(n, sh_degree) -> int:
    return int(load().gs_adam_state_floats(n, sh_degree))


def gs_adam_step(n, sh_degree, step, cfg: GsAdamConfig, params: dict, grads: dict, m, v, stream=None):
    """One Adam step on params (updated in place) from grads; m, v: the moment buffers."""
    _check(load().gs_adam_step(n, sh_degree, step, ctypes.byref(cfg),
                               *[_ptr(params[k]) for k in ("means", "log_scales", "quats", "opacity_logits", "sh")],
                               *[_ptr(grads[k]) for k in ("means", "log_scales", "quats", "opacity_logits", "sh")],
                               _ptr(m), _ptr(v), _stream(stream)))


_PROJ_FIELDS = ("means2d", "conics", "depths", "opacities", "colors", "radii", "tiles_touched")


@dataclass
class Projected:
    means2d: torch.Tensor
    conics: torch.Tensor
    depths: torch.Tensor
    opacities: torch.Tensor
    colors: torch.Tensor
    radii: torch.Tensor
    tiles_touched: torch.Tensor

    @staticmethod
    def empty(n, device="cuda"):
        f = dict(device=device, dtype=torch.float32)
        return Projected(torch.empty(n, 2, **f), torch.empty(n, 3, **f), torch.empty(n, **f), torch.empty(n, **f),
                         torch.empty(n, 3, **f), torch.empty(n, 2, device=device, dtype=torch.int32),
                         torch.empty(n, device=device, dtype=torch.int32))

    def struct(self) -> GsProjected:
        """The C struct of the seven pointers, rebuilt only when one of them changed."""
        ptrs = tuple(getattr(self, f).data_ptr() for f in _PROJ_FIELDS)
        if getattr(self, "_keep_ptrs", None) != ptrs:
            s = GsProjected()
            for f, q in zip(_PROJ_FIELDS, ptrs):
                setattr(s, "d_" + f, q)
            self._keep, self._keep_ptrs = s, ptrs
        return self._keep


def scene_to_device(scene: dict, device="cuda"):
    """Raw parameters of a scene dict as contiguous fp32 CUDA tensors."""
    out = {}
    for k in ("means", "log_scales", "quats", "opacity_logits", "sh"):
        out[k] = torch.as_tensor(np.ascontiguousarray(scene[k], dtype=np.float32)).to(device).contiguous()
    out["sh_degree"] = int(scene.get("sh_degree", 0))
    out["n"] = int(out["means"].shape[0])
    return out


class Pipeline:
    """Device buffers for one scene at one image size, and the entry points in iteration order."""

    def __init__(self, params: dict, width: int, height: int, pair_capacity: int = 1 << 20, device="cuda"):
        self.p = params
        self.n = params["n"]
        self.width, self.height = width, height
        self.device = device
        self.tiles = ((width + 15) // 16) * ((height + 15) // 16)
        self.proj = Projected.empty(self.n, device)
        self.image = torch.empty(height, width, 3, device=device)
        self.final_T = torch.empty(height, width, device=device)
        self.n_contrib = torch.empty(height, width, device=device, dtype=torch.int32)
        self.dL_dimage = torch.zeros(height, width, 3, device=device)
        self.ranges = torch.empty(self.tiles, 2, device=device, dtype=torch.int32)
        cam0 = GsCamera()
        cam0.width, cam0.height = width, height
        self.plan = torch.empty(gs_raster_plan_words(cam0), device=device, dtype=torch.int32)
        self.raster_ws = torch.zeros(gs_raster_workspace_bytes(), device=device, dtype=torch.uint8)
        self.bwd_ws = torch.empty(gs_bwd_workspace_bytes(self.n), device=device, dtype=torch.uint8)
        K = (params["sh_degree"] + 1) ** 2
        f = dict(device=device, dtype=torch.float32)
        self.grads = {"means": torch.empty(self.n, 3, **f), "log_scales": torch.empty(self.n, 3, **f),
                      "quats": torch.empty(self.n, 4, **f), "opacity_logits": torch.empty(self.n, **f),
                      "sh": torch.empty(self.n, K, 3, **f), "means2d": torch.empty(self.n, 2, **f)}
        self.num_pairs = 0
        self.num_pairs_dev = torch.zeros(1, device=device, dtype=torch.int64)
        self.schedule = "chunks"  # "chunks": plan + checkpoints; "order": plan only; "tiles": neither
        self.deterministic = False  # True: the bitwise-reproducible backward
        self.ssim_lambda = 0.0  # > 0: the loss is (1 - lambda) L1 + lambda (1 - SSIM)
        self._alloc_pairs(pair_capacity)

    def _alloc_pairs(self, cap):
        self.capacity = int(cap)
        self.keys = torch.empty(max(self.capacity, 1), device=self.device, dtype=torch.int64)
        self.ids = torch.empty(max(self.capacity, 1), device=self.device, dtype=torch.int32)
        cam0 = GsCamera()
        cam0.width, cam0.height = self.width, self.height
        self.bin_ws = torch.empty(gs_bin_workspace_bytes(self.n, self.capacity, cam0), device=self.device,
                                  dtype=torch.uint8)

    def project(self, cam: GsCamera, stream=None):
        p = self.p
        gs_project(self.n, p["sh_degree"], p["means"], p["log_scales"], p["quats"], p["opacity_logits"], p["sh"],
                   cam, self.proj, stream)

    def bin(self, cam: GsCamera, stream=None, wait=True):
        """Bin and sort. wait=True reads P on the host and regrows the pair buffers when they
        overflow; wait=False only enqueues (P lands in self.num_pairs_dev; an overflow leaves every
        tile empty and shows as self.num_pairs_dev > self.capacity)."""
        if not wait:
            gs_bin_and_sort(self.n, self.proj, cam, self.bin_ws, self.capacity, self.keys, self.ids, self.ranges,
                            self.num_pairs_dev, stream, wait=False, plan=self.plan)
            self.num_pairs = None
            return None
        st, P = gs_bin_and_sort(self.n, self.proj, cam, self.bin_ws, self.capacity, self.keys, self.ids,
                                self.ranges, self.num_pairs_dev, stream, plan=self.plan)
        if st == GS_ERR_CAPACITY:
            self._alloc_pairs(int(P * 1.25) + 1024)
            st, P = gs_bin_and_sort(self.n, self.proj, cam, self.bin_ws, self.capacity, self.keys, self.ids,
                                    self.ranges, self.num_pairs_dev, stream, plan=self.plan)
        self.num_pairs = P
        return P

    def reserve_pairs(self, cap):
        """Grow the pair buffers to at least cap pairs (for runs that do not wait on bin)."""
        if cap > self.capacity:
            self._alloc_pairs(int(cap))

    def forward(self, cam: GsCamera, eval_count=None, stream=None, checkpoints=None, depth=None, l1_target=None):
        """Blend. checkpoints (default: the "chunks" schedule) stores the per-chunk state that lets
        the backward split long tiles; a render that no backward follows can leave it out.
        l1_target: also write the L1 gradient against it into self.dL_dimage (gs_rasterize_fwd_l1)."""
        ck = self.schedule == "chunks" if checkpoints is None else bool(checkpoints)
        self._ckpt_written = ck
        self._ckpt_depth = ck and depth is not None  # the checkpoints hold the depth channel's parts
        plan = self.plan if self.schedule != "tiles" else None
        ws = self.raster_ws if ck else None
        if l1_target is not None:
            gs_rasterize_fwd_l1(self.n, self.proj, cam, self.ids, self.ranges, self.image, self.final_T,
                                self.n_contrib, l1_target, self.dL_dimage, eval_count, stream, plan=plan,
                                raster_ws=ws, depth=depth)
        else:
            gs_rasterize_fwd(self.n, self.proj, cam, self.ids, self.ranges, self.image, self.final_T, self.n_contrib,
                             eval_count, stream, plan=plan, raster_ws=ws, depth=depth)

    def loss_l1(self, target, loss=None, stream=None):
        """The training loss's gradient into self.dL_dimage: L1, or with self.ssim_lambda > 0
        (1 - lambda) L1 + lambda (1 - SSIM)."""
        lam = getattr(self, "ssim_lambda", 0.0)
        if lam > 0.0:
            if getattr(self, "_ssim_ws", None) is None:
                self._ssim_ws = torch.empty(gs_loss_ssim_workspace_bytes(self.width, self.height), device=self.device,
                                            dtype=torch.uint8)
            gs_loss_l1_ssim(self.width, self.height, self.image, target, lam, self._ssim_ws, self.dL_dimage, loss,
                            stream)
        else:
            gs_loss_l1(self.width, self.height, self.image, target, self.dL_dimage, loss, stream)

    def backward(self, cam: GsCamera, dL_dimage=None, eval_count=None, stream=None, dL_ddepth=None):
        """self.deterministic selects gs_rasterize_bwd_deterministic (records sized by the pair
        capacity) over gs_rasterize_bwd (fp32 atomics). The backward splits long tiles at the last
        forward's checkpoints only when they hold what it reads: with dL_ddepth, the depth
        channel's parts too; otherwise it walks whole tiles."""
        p, g = self.p, self.grads
        use_ckpt = getattr(self, "_ckpt_written", False) and (dL_ddepth is None or getattr(self, "_ckpt_depth", False))
        det = getattr(self, "deterministic", False)
        ws = self.bwd_ws
        if det:
            ws = self._det_workspace()
        gs_rasterize_bwd(self.n, p["sh_degree"], p["means"], p["log_scales"], p["quats"], p["opacity_logits"],
                         p["sh"], cam, self.proj, self.ids, self.ranges, self.final_T, self.n_contrib,
                         self.dL_dimage if dL_dimage is None else dL_dimage, ws, g["means"], g["log_scales"],
                         g["quats"], g["opacity_logits"], g["sh"], g["means2d"], eval_count, stream,
                         plan=self.plan if self.schedule != "tiles" else None,
                         raster_ws=self.raster_ws if use_ckpt else None,
                         pair_capacity=self.capacity if det else None, dL_ddepth=dL_ddepth)

    # ---- feature channels: any per-Gaussian quantity blended with the colour's weights ----------
    def _feature_args(self, cam: GsCamera, features):
        """The camera with background 0 and the features laid out as three channels ([n, 3], the
        unused ones 0): the blend and its backward treat them as colours."""
        if features.dim() != 2 or features.shape[0] != self.n or not 1 <= features.shape[1] <= 3:
            raise ValueError("features must be [n, C] with 1 <= C <= 3 (render more in groups of three)")
        fcam = GsCamera()
        ctypes.memmove(ctypes.byref(fcam), ctypes.byref(cam), ctypes.sizeof(GsCamera))
        for i in range(3):
            fcam.background[i] = 0.0
        f3 = torch.zeros(self.n, 3, device=self.device, dtype=torch.float32)
        f3[:, : features.shape[1]] = features
        pr = self.proj
        proj = Projected(pr.means2d, pr.conics, pr.depths, pr.opacities, f3, pr.radii, pr.tiles_touched)
        return fcam, f3, proj

    def render_features(self, cam: GsCamera, features, stream=None):
        """F = sum_i f_i alpha_i T_i per pixel (background 0) for features [n, C], C <= 3, with this
        iteration's projection and pair lists (section 5 of the PyTorch lesson: any channel goes
        through the blend's weights). Returns [h, w, C]."""
        fcam, _, proj = self._feature_args(cam, features)
        img = torch.empty(self.height, self.width, 3, device=self.device, dtype=torch.float32)
        ft = torch.empty_like(self.final_T)
        nc = torch.empty_like(self.n_contrib)
        gs_rasterize_fwd(self.n, proj, fcam, self.ids, self.ranges, img, ft, nc, None, stream)
        return img[..., : features.shape[1]]

    def features_backward(self, cam: GsCamera, features, dL_dF, stream=None):
        """Gradients of a loss on render_features' output: dL/dfeatures [n, C] and the
        geometry's share (means, log_scales, quats, opacity_logits), from the forward's final T
        and counts. The colour loss's gradients come from backward(); the two add."""
        fcam, f3, proj = self._feature_args(cam, features)
        C = features.shape[1]
        g3 = torch.zeros(self.height, self.width, 3, device=self.device, dtype=torch.float32)
        g3[..., :C] = dL_dF
        f = dict(device=self.device, dtype=torch.float32)
        out = {"means": torch.empty(self.n, 3, **f), "log_scales": torch.empty(self.n, 3, **f),
               "quats": torch.empty(self.n, 4, **f), "opacity_logits": torch.empty(self.n, **f),
               "features": torch.empty(self.n, 1, 3, **f)}
        det = getattr(self, "deterministic", False)
        if det:
            need = gs_bwd_det_workspace_bytes(self.n, self.capacity)
            if getattr(self, "_det_ws", None) is None or self._det_ws.numel() < need:
                self._det_ws = torch.empty(need, device=self.device, dtype=torch.uint8)
        p = self.p
        gs_rasterize_bwd(self.n, 0, p["means"], p["log_scales"], p["quats"], p["opacity_logits"], f3.view(self.n, 1, 3),
                         fcam, proj, self.ids, self.ranges, self.final_T, self.n_contrib, g3,
                         self._det_ws if det else self.bwd_ws, out["means"], out["log_scales"], out["quats"],
                         out["opacity_logits"], out["features"], None, None, stream,
                         pair_capacity=self.capacity if det else None)
        out["features"] = out["features"].view(self.n, 3)[:, :C]
        return out

    def _det_workspace(self):
        need = gs_bwd_det_workspace_bytes(self.n, self.capacity)
        if getattr(self, "_det_ws", None) is None or self._det_ws.numel() < need:
            self._det_ws = torch.empty(need, device=self.device, dtype=torch.uint8)
        return self._det_ws

    def _iteration_args(self):
        """The arguments of a no-wait L1 iteration's four entry points except the camera, the target
        and the stream, built once per set of buffers (their pointers do not change between
        iterations, and rebuilding them was half of the host's time per iteration)."""
        det = getattr(self, "deterministic", False)
        key = (self.capacity, det, self.keys.data_ptr(), self.bin_ws.data_ptr(), id(self.p))
        if getattr(self, "_iter_key", None) == key:
            return self._iter_args
        p, g = self.p, self.grads
        P = _ptr
        proj = ctypes.byref(self.proj.struct())
        raw = (P(p["means"]), P(p["log_scales"]), P(p["quats"]), P(p["opacity_logits"]), P(p["sh"]))
        ws = self._det_workspace() if det else self.bwd_ws
        a = {
            "proj": proj,
            "project": (self.n, p["sh_degree"]) + raw,
            "bin": (ctypes.c_void_p(self.bin_ws.data_ptr()), self.bin_ws.numel() * self.bin_ws.element_size(),
                    self.capacity, P(self.keys), P(self.ids), P(self.ranges), P(self.plan), P(self.num_pairs_dev),
                    None),
            "fwd_pre": (P(self.ids), P(self.ranges), P(self.plan), P(self.raster_ws), P(self.image), None,
                        P(self.final_T), P(self.n_contrib)),
            "fwd_post": (P(self.dL_dimage), None),
            "bwd_pre": (self.n, p["sh_degree"]) + raw,
            "bwd_post": (P(self.ids), P(self.ranges), P(self.plan), P(self.raster_ws), P(self.final_T),
                         P(self.n_contrib), P(self.dL_dimage), None)
                        + ((int(self.capacity),) if det else ())
                        + (P(ws), ws.numel() * ws.element_size(), P(g["means"]), P(g["log_scales"]), P(g["quats"]),
                           P(g["opacity_logits"]), P(g["sh"]), P(g["means2d"]), None),
            "bwd": load().gs_rasterize_bwd_deterministic if det else load().gs_rasterize_bwd,
        }
        self._iter_key, self._iter_args = key, a
        return a

    def iteration(self, cam: GsCamera, target, stream=None, wait=True):
        """One fwd+bwd iteration: project, bin+sort, blend, loss gradient (L1 inside the blend, or the
        separate L1 + SSIM kernels), backward. wait=False runs
        it without any host wait (the pair buffers must already be large enough)."""
        if not wait and getattr(self, "ssim_lambda", 0.0) <= 0.0 and self.schedule == "chunks":
            # the same four calls as below, with the unchanging arguments taken from a cache
            lib, a = load(), self._iteration_args()
            cp, s, tp = ctypes.byref(cam), _stream(stream), _ptr(target)
            _check(lib.gs_project(*a["project"], cp, a["proj"], s))
            _check(lib.gs_bin_and_sort(self.n, a["proj"], cp, *a["bin"], s), allow=(GS_ERR_CAPACITY,))
            self.num_pairs = None
            _check(lib.gs_rasterize_fwd_l1(self.n, a["proj"], cp, *a["fwd_pre"], tp, *a["fwd_post"], s))
            self._ckpt_written, self._ckpt_depth = True, False
            _check(a["bwd"](*a["bwd_pre"], cp, a["proj"], *a["bwd_post"], s))
            return
        self.project(cam, stream)
        self.bin(cam, stream, wait=wait)
        if getattr(self, "ssim_lambda", 0.0) > 0.0:
            self.forward(cam, stream=stream)
            self.loss_l1(target, stream=stream)
        else:  # the L1 gradient formed in the blend
            self.forward(cam, stream=stream, l1_target=target)
        self.backward(cam, stream=stream)

    def adam_step(self, cfg: GsAdamConfig, stream=None):
        """Adam on the raw parameters (in place) from the last backward's gradients. The moment
        buffers are allocated (zeroed) at the first call and carried between calls."""
        if getattr(self, "_adam_m", None) is None:
            f = gs_adam_state_floats(self.n, self.p["sh_degree"])
            self._adam_m = torch.zeros(max(f, 1), device=self.device)
            self._adam_v = torch.zeros(max(f, 1), device=self.device)
            self._adam_t = 0
        self._adam_t += 1
        gs_adam_step(self.n, self.p["sh_degree"], self._adam_t, cfg, self.p, self.grads, self._adam_m, self._adam_v,
                     stream)
