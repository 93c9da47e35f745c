"""Block-causal GQA attention forward (MAGI-1's hot path) for AMD MI355X.

libmagi_bca.so (C ABI, include/magi_bca.h) holds the mask -> AttnSlice
builder, the atomic-free scheduler and the HIP kernels; ``ops`` is a thin
torch binding over it.
"""
from . import _lib  # noqa: F401
from .ops import (build_slices, default_tile_q, dtype_code, ffa_fwd, make_plan,  # noqa: F401
                  plan_for_videos, qknorm_rope, schedule, Plan)

__version__ = "0.1.0"
