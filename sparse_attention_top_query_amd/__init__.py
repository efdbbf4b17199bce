"""Fathom per-query variable-depth key scan on MI355X (gfx950).

The compute path is libfathom.so (hand-written HIP kernels behind the C ABI in
include/fathom.h); this package is its thin Python binding.  There is no CPU
fallback: calls fail if the library has not been built.
"""

from .fathom import (  # noqa: F401
    HBM,
    HOST_DIRECT,
    HOST_STAGED,
    STATIC,
    TOPQ,
    WATERFILL,
    WATERFILL_GROUP,
    FathomError,
    allocate,
    attend,
    attend_workspace_bytes,
    device_address,
    load,
    pack,
    pack_blocks,
    pack_nibbles,
    page_table,
    prefix_bytes,
    record_bytes,
    scan_scores,
    scan_topk,
    scan_topk_append,
    scan_topk_nibbles,
    scan_topk_paged,
    workspace_bytes,
)

__all__ = ["HBM", "HOST_DIRECT", "HOST_STAGED", "STATIC", "TOPQ", "WATERFILL", "WATERFILL_GROUP", "FathomError", "allocate", "attend", "attend_workspace_bytes", "device_address", "load", "pack", "pack_blocks", "pack_nibbles", "page_table",
           "prefix_bytes", "record_bytes", "scan_scores", "scan_topk", "scan_topk_append", "scan_topk_nibbles", "scan_topk_paged", "workspace_bytes"]
