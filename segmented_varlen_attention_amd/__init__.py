"""Segmented ("gapped") varlen attention for AMD Instinct MI355X (gfx950).

The compute lives in libgvattn.so (HIP kernels behind the C ABI declared in
include/gvattn.h); this package is its thin Python binding plus the seeded
synthetic workloads used by the tests and the benchmark.
"""

from .binding import (  # noqa: F401
    GVATTN_BF16,
    GVATTN_FP16,
    GVATTN_FP32,
    alloc_workspace,
    gvattn_bwd,
    gvattn_bwd_workspace_size,
    gvattn_fwd,
    gvattn_fwd_plan,
    gvattn_fwd_noalloc,
    gvattn_fwd_ranges,
    gvattn_fwd_run,
    gvattn_fwd_workspace_size,
    gvattn_lse_merge,
    gvattn_read_device_error,
    gvattn_version,
    load_library,
    status_string,
)
