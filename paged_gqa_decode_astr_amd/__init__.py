"""Paged grouped-query attention (decode + ragged prefill) for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels inside libastr_attn.so, reached
through a C ABI (include/astr_attn.h).  This package holds the ctypes binding
(``_lib``), device-memory plumbing (``tensors``), the seeded synthetic
workloads (``workloads``) and the build script (``build``).
"""
from ._lib import (AstrError, DEFAULT_MAX_SPLITS, astr_last_error, astr_paged_decode, astr_paged_prefill,
                   astr_plan_decode, astr_workspace_size, load_library)

__all__ = ["AstrError", "DEFAULT_MAX_SPLITS", "astr_last_error", "astr_paged_decode", "astr_paged_prefill",
           "astr_plan_decode", "astr_workspace_size", "load_library"]
