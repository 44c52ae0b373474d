"""relative_position_bias_amd — relative-bias GQA attention for MI355X (gfx950).

The compute path is librba.so (hand-written HIP kernels behind a C ABI, see
include/rba.h); `rba` is its thin ctypes binding. Importing the package does
not load the library; the first call does, and raises if it has not been
built.
"""
from . import rba  # noqa: F401
from .rba import (  # noqa: F401
    RbaError, decode, decode_combine, decode_noalloc, decode_relproj, decode_split, plan_splits, prefill,
    prefill_relproj, relproj_workspace_size, version, workspace_size)

__all__ = ["rba", "prefill", "prefill_relproj", "decode", "decode_relproj", "decode_split", "decode_combine",
           "decode_noalloc", "plan_splits", "workspace_size", "relproj_workspace_size", "version", "RbaError"]
