"""MoE dispatch / combine for one MI355X (gfx950).

The C ABI is include/ep.h; `_ffi` binds it with the same names and `ops`
adds torch tensors (device memory and the current stream) on top. Importing
this package does not load the library; the first call does, and fails if
libep.so has not been built (`python -m combine_ep_layout_10_amd.build`).
"""
from . import _ffi  # noqa: F401
