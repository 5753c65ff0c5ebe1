"""Placement-aware gradient reduction, global norm, clipping and fused AdamW
for MI355X (gfx950): a C-ABI library of hand-written HIP kernels
(libgro.so, declared in include/gro.h) with a thin ctypes binding.

The library is loaded on first use and there is no fallback: a missing
library raises.
"""
from .binding import (  # noqa: F401
    GroError, gro_accumulate, gro_accumulate_window, gro_clip_adamw, gro_last_error, gro_plan_bind, gro_plan_bucket,
    gro_plan_create, gro_plan_destroy, gro_plan_get_info, gro_plan_get_norm, gro_plan_tensor,
    gro_init_uniform, gro_reduce_norm, load,
)
