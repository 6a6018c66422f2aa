"""Document-masked (varlen) causal grouped-query attention for MI355X (gfx950).

``fwd``/``bwd`` call the C ABI of libattn_varlen.so (include/attn_varlen.h);
the computation runs in hand-written HIP kernels.  ``flops`` holds the exact
work counts used for throughput.
"""
from . import flops
from ._binding import (LIBRARY_PATH, AttnError, bwd, bwd_static, delta_bwd, delta_bwd_workspace_size, delta_fwd,
                       delta_workspace_size, fwd, kda_bwd, kda_bwd_workspace_size, kda_fwd, kda_workspace_size,
                       load_library, new_workspace, profile_start, profile_stop, schedule,
                       strerror, workspace_size)

__all__ = ["LIBRARY_PATH", "AttnError", "bwd", "bwd_static", "delta_bwd", "delta_bwd_workspace_size", "delta_fwd",
           "delta_workspace_size", "flops", "fwd", "kda_bwd", "kda_bwd_workspace_size", "kda_fwd",
           "kda_workspace_size",
           "load_library", "new_workspace", "profile_start", "profile_stop", "schedule",
           "strerror", "workspace_size"]
