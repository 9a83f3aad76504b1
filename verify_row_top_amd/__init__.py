"""verify_row_top_amd: draft-tree construction and lossless verification on MI355X.

The hot path is libvrt.so (hand-written HIP for gfx950 behind the C ABI in
include/vrt.h); `vrt` is its thin ctypes binding.
"""
from . import vrt  # noqa: F401
