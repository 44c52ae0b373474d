"""relative_position_bias_amd — relative-bias GQA attention for MI355X (gfx950).

The compute path is librba.so (hand-written HIP kernels behind a C ABI, see
include/rba.h); `rba` is its thin ctypes binding and `workloads` the seeded
synthetic inputs. Importing the package does not load the library; the first
call does, and raises if it has not been built.
"""
from . import rba  # noqa: F401
from .rba import (  # noqa: F401
    RbaError, decode, decode_combine, decode_split, plan_splits, prefill, version, workspace_size)

__all__ = ["rba", "prefill", "decode", "decode_split", "decode_combine", "plan_splits",
           "workspace_size", "version", "RbaError"]
