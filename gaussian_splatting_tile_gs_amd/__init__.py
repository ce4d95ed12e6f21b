"""MI355X-native differentiable tile-based 3D Gaussian Splatting rasterizer.

The compute path is the C-ABI library ``libgs_hip.so`` (hand-written HIP for gfx950, declared in
``include/gs.h``); ``gaussian_splatting_tile_gs_amd.gs`` is its thin ctypes binding (argument
marshalling only). ``synth`` holds the seeded synthetic inputs. Nothing is imported eagerly so
that importing ``synth`` never loads the GPU library.
"""

__all__ = ["gs", "synth"]
