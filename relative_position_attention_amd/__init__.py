"""Exact relative-position attention on MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in ``include/relpos.h``: it builds the
descriptor from a mechanism description, allocates the library's buffers with
torch (device memory only) and passes raw pointers plus the current HIP
stream.  Every step of the computation runs in the HIP library
``librelpos.so``; there is no fallback: if the library is missing, importing
works but every call raises.

Method: "Fast and Exact Relative-Position Attention via Structure-Aware
Kernels" (arXiv 2611.01182).
"""

from .binding import (  # noqa: F401
    RelposError,
    Problem,
    library,
    library_path,
    plan_sizes,
    plan_rows,
    project,
    project_noalloc,
    attn_fwd,
    attn_bwd,
    empty_grads,
    set_stage_events,
    segment_bounds,
    strerror,
    EXPORTED_SYMBOLS,
)
