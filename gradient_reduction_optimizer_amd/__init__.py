"""Placement-aware gradient reduction, global norm, clipping and fused AdamW
for MI355X (gfx950): a C-ABI library of hand-written HIP kernels with a thin
ctypes binding.  The library is loaded on first use; there is no fallback.
"""
