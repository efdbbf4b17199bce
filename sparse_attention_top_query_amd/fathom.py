"""Python binding of libfathom.so (ctypes): argument marshalling only.

Every function takes torch tensors for device (or pinned host) memory, checks
dtype, device and contiguity, and passes raw pointers plus the current HIP
stream to the C ABI declared in include/fathom.h.  All compute runs in the
library's HIP kernels; nothing here computes any part of the method.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfathom.so")

HBM = 0
HOST_DIRECT = 1
HOST_STAGED = 2
WATERFILL = 0
TOPQ = 1
WATERFILL_GROUP = 2
STATIC = 3

FLAG_KEY_NONFINITE = 1
FLAG_SCALE_OVERFLOW = 2
FLAG_Q_NONFINITE = 4
FLAG_SIGMA2_INVALID = 8
FLAG_IMPORTANCE_OVERFLOW = 16
FLAG_INDEX_RANGE = 32

STATUS_NAMES = {0: "FATHOM_OK", -1: "FATHOM_EINVAL", -2: "FATHOM_ESHAPE", -3: "FATHOM_EBUDGET",
                -5: "FATHOM_EWORKSPACE", -6: "FATHOM_EHIP", -7: "FATHOM_ERESIDENCY"}


class FathomError(RuntimeError):
    """A negative status from the library, with its message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libfathom.so (built in-tree by sparse_attention_top_query_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_attention_top_query_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "fathom_record_bytes": (S, [L]),
        "fathom_prefix_bytes": (S, [L, I]),
        "pack_bitplanes": (I, [P, I, L, I, P, P, P]),
        "allocate_depths": (I, [P, P, I, I, I, I, I, P, P, P, P]),
        "fathom_workspace_bytes": (S, [I, I, L, I, I, I]),
        "scan_topk": (I, [P, I, P, P, P, I, I, L, I, I, P, P, P, S, P]),
        "fathom_scan_scores": (I, [P, I, P, P, P, I, I, L, I, P, L, P, S, P]),
        "fathom_noalloc_scratch_bytes": (S, []),
        "scan_topk_noalloc": (I, [P, I, P, P, P, I, I, L, I, I, P, P, P]),
        "fathom_attend_workspace_bytes": (S, [I, I, I]),
        "pack_blocks": (I, [P, I, L, L, L, I, P, P, P]),
        "fathom_device_address": (I, [P, I, ctypes.POINTER(ctypes.c_void_p)]),
        "pack_nibbles": (I, [P, I, L, I, P, P, P, P]),
        "scan_topk_nibbles": (I, [P, P, I, P, P, P, I, I, L, I, I, P, P, P, S, P]),
        "scan_topk_paged": (I, [P, I, L, L, P, L, P, P, P, I, I, I, I, P, P, P, S, P]),
        "scan_topk_append": (I, [P, I, L, L, P, L, P, P, P, I, I, I, I, P, P, P, S, P]),
        "attend_topk": (I, [P, P, I, P, P, I, I, L, I, I, ctypes.c_float, P, P, P, P, S, P]),
        "fathom_last_error": (ctypes.c_char_p, []),
        "fathom_version": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise FathomError(status, load().fathom_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, ndim=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def record_bytes(n: int) -> int:
    return int(load().fathom_record_bytes(n))


def prefix_bytes(n: int, t: int) -> int:
    """Bytes of the contiguous run holding the scales and the first t planes."""
    return int(load().fathom_prefix_bytes(n, t))


def workspace_bytes(h_q: int, h_kv: int, n: int, d: int, k: int, residency: int = HBM) -> int:
    return int(load().fathom_workspace_bytes(h_q, h_kv, n, d, k, residency))


def pack(k: torch.Tensor, records: torch.Tensor | None = None, status: torch.Tensor | None = None):
    """pack_bitplanes: k float32 [h_kv, n, d] on device -> records uint8 [h_kv, d, R]."""
    _need(k, "k", torch.float32, 3)
    h_kv, n, d = k.shape
    r = record_bytes(n)
    if records is None:
        records = torch.empty((h_kv, d, r), dtype=torch.uint8, device=k.device)
    _need(records, "records", torch.uint8)
    if records.numel() < h_kv * d * r:
        raise ValueError("records buffer too small")
    if status is not None:
        _need(status, "status", torch.int32)
    _check(load().pack_bitplanes(_ptr(k), h_kv, n, d, _ptr(records), _ptr(status), _stream(k)))
    return records


def allocate(q: torch.Tensor, sigma2: torch.Tensor, budget: int, mode: int = WATERFILL,
             depth: torch.Tensor | None = None, union_depth: torch.Tensor | None = None,
             status: torch.Tensor | None = None):
    """allocate_depths: q [h_q, d], sigma2 [h_kv, d] -> (depth uint8 [h_q, d], union uint8 [h_kv, d])."""
    _need(q, "q", torch.float32, 2)
    _need(sigma2, "sigma2", torch.float32, 2)
    h_q, d = q.shape
    h_kv = sigma2.shape[0]
    if sigma2.shape[1] != d:
        raise ValueError("sigma2 and q disagree on d")
    if depth is None:
        depth = torch.empty((h_q, d), dtype=torch.uint8, device=q.device)
    if union_depth is None:
        union_depth = torch.empty((h_kv, d), dtype=torch.uint8, device=q.device)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    if status is not None:
        _need(status, "status", torch.int32)
    _check(load().allocate_depths(_ptr(q), _ptr(sigma2), h_q, h_kv, d, mode, budget, _ptr(depth),
                                  _ptr(union_depth), _ptr(status), _stream(q)))
    return depth, union_depth


def _residency_of(records: torch.Tensor) -> int:
    return HBM if records.is_cuda else HOST_DIRECT


def scan_topk(records: torch.Tensor, q: torch.Tensor, depth: torch.Tensor, union_depth: torch.Tensor,
              n: int, k: int, residency: int | None = None, workspace: torch.Tensor | None = None,
              idx: torch.Tensor | None = None, scores: torch.Tensor | None = None,
              want_scores: bool = False):
    """scan_topk: -> int32 [h_q, k] ascending key indices (and float32 scores if asked).

    ``records`` may be a device tensor (HBM residency) or a pinned host tensor
    (read in place over the host link by default; HOST_STAGED gathers the
    prefix runs into a ring of two KV heads' records in HBM first)."""
    _need(q, "q", torch.float32, 2)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    _need(records, "records", torch.uint8, device=False)
    if residency is None:
        residency = _residency_of(records)
    h_q, d = q.shape
    h_kv = union_depth.shape[0]
    if records.numel() < h_kv * d * record_bytes(n):
        raise ValueError("records buffer too small for (h_kv, d, n)")
    wsb = workspace_bytes(h_q, h_kv, n, d, k, residency)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if idx is None:
        idx = torch.empty((h_q, k), dtype=torch.int32, device=q.device)
    _need(idx, "idx", torch.int32)
    if want_scores and scores is None:
        scores = torch.empty((h_q, k), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores, "scores", torch.float32)
    _check(load().scan_topk(_ptr(records), residency, _ptr(q), _ptr(depth), _ptr(union_depth), h_q, h_kv,
                            n, d, k, _ptr(idx), _ptr(scores), _ptr(workspace), workspace.numel(),
                            _stream(q)))
    return (idx, scores) if want_scores or scores is not None else idx


def noalloc_scratch_bytes() -> int:
    """Size of the library's fixed device scratch used by scan_topk_noalloc."""
    return int(load().fathom_noalloc_scratch_bytes())


def scan_topk_noalloc(records: torch.Tensor, q: torch.Tensor, depth: torch.Tensor, union_depth: torch.Tensor,
                      n: int, k: int, idx: torch.Tensor, scores: torch.Tensor | None = None,
                      residency: int | None = None):
    """scan_topk_noalloc: scan_topk with the library's fixed scratch as workspace.
    The outputs are passed in (nothing is allocated here either)."""
    _need(q, "q", torch.float32, 2)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    _need(records, "records", torch.uint8, device=False)
    _need(idx, "idx", torch.int32)
    if scores is not None:
        _need(scores, "scores", torch.float32)
    if residency is None:
        residency = _residency_of(records)
    h_q, d = q.shape
    h_kv = union_depth.shape[0]
    if records.numel() < h_kv * d * record_bytes(n):
        raise ValueError("records buffer too small for (h_kv, d, n)")
    if idx.numel() < h_q * k or (scores is not None and scores.numel() < h_q * k):
        raise ValueError("idx/scores smaller than [h_q, k]")
    _check(load().scan_topk_noalloc(_ptr(records), residency, _ptr(q), _ptr(depth), _ptr(union_depth), h_q, h_kv,
                                    n, d, k, _ptr(idx), _ptr(scores), _stream(q)))
    return idx


def scan_scores(records: torch.Tensor, q: torch.Tensor, depth: torch.Tensor, union_depth: torch.Tensor,
                n: int, residency: int | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None):
    """fathom_scan_scores: -> float32 [h_q, n] scores (the scan stage alone)."""
    _need(q, "q", torch.float32, 2)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    _need(records, "records", torch.uint8, device=False)
    if residency is None:
        residency = _residency_of(records)
    h_q, d = q.shape
    h_kv = union_depth.shape[0]
    if out is None:
        out = torch.empty((h_q, max(n, 1)), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 2)
    if workspace is None and residency == HOST_STAGED:
        workspace = torch.empty(max(workspace_bytes(h_q, h_kv, n, d, 1, residency), 1), dtype=torch.uint8,
                                device=q.device)
    wsn = 0 if workspace is None else workspace.numel()
    _check(load().fathom_scan_scores(_ptr(records), residency, _ptr(q), _ptr(depth), _ptr(union_depth),
                                     h_q, h_kv, n, d, _ptr(out), out.shape[1], _ptr(workspace), wsn,
                                     _stream(q)))
    return out[:, :n]


def attend_workspace_bytes(h_q: int, d: int, k: int) -> int:
    return int(load().fathom_attend_workspace_bytes(h_q, d, k))


def attend(k_cache: torch.Tensor, v_cache: torch.Tensor, q: torch.Tensor, idx: torch.Tensor, scale: float,
           residency: int | None = None, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
           status: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """attend_topk: -> (float32 out [h_q, d], float32 lse [h_q]) attention over the selected keys.

    ``k_cache``/``v_cache``: bf16 [h_kv, n, d] (torch.bfloat16, or their bit
    patterns as int16/uint16), both device tensors (HBM) or both pinned host
    tensors (read in place).  ``idx``: int32 [h_q, k]."""
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError(f"{name} must be a bfloat16 (or 16-bit pattern) tensor")
        if not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous [h_kv, n, d] tensor")
    if k_cache.shape != v_cache.shape or k_cache.is_cuda != v_cache.is_cuda:
        raise ValueError("k_cache and v_cache must have one shape and one residency")
    _need(q, "q", torch.float32, 2)
    _need(idx, "idx", torch.int32, 2)
    h_kv, n, d = k_cache.shape
    h_q, k = idx.shape
    if q.shape != (h_q, d):
        raise ValueError("q must be [h_q, d] with h_q = idx.shape[0] and d = k_cache.shape[2]")
    if residency is None:
        residency = HBM if k_cache.is_cuda else HOST_DIRECT
    if out is None:
        out = torch.empty((h_q, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 2)
    if lse is None:
        lse = torch.empty(h_q, dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, 1)
    if status is not None:
        _need(status, "status", torch.int32)
    if workspace is None:
        workspace = torch.empty(max(attend_workspace_bytes(h_q, d, k), 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    _check(load().attend_topk(_ptr(k_cache), _ptr(v_cache), residency, _ptr(q), _ptr(idx), h_q, h_kv, n, d, k,
                              ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(status), _ptr(workspace),
                              workspace.numel(), _stream(q)))
    return out, lse


def pack_blocks(k: torch.Tensor, records: torch.Tensor, n_cap: int, block0: int,
                status: torch.Tensor | None = None):
    """pack_blocks: seal the blocks whose rows ``k`` float32 [h_kv, rows, d] holds,
    starting at block ``block0``, into ``records`` of capacity ``n_cap``."""
    _need(k, "k", torch.float32, 3)
    _need(records, "records", torch.uint8)
    h_kv, rows, d = k.shape
    nblocks = -(-rows // 128)
    if records.numel() < h_kv * d * record_bytes(n_cap):
        raise ValueError("records buffer too small for (h_kv, d, n_cap)")
    if rows != min(128 * nblocks, n_cap - 128 * block0):
        raise ValueError("k must hold whole blocks (or the capacity's last, shorter block)")
    if status is not None:
        _need(status, "status", torch.int32)
    _check(load().pack_blocks(_ptr(k), h_kv, n_cap, block0, nblocks, d, _ptr(records), _ptr(status), _stream(k)))
    return records


def scan_topk_append(records: torch.Tensor | None, n_cap: int, n_sealed: int, tail_k: torch.Tensor | None,
                     q: torch.Tensor, depth: torch.Tensor, union_depth: torch.Tensor, k: int,
                     residency: int | None = None, workspace: torch.Tensor | None = None,
                     idx: torch.Tensor | None = None, scores: torch.Tensor | None = None,
                     want_scores: bool = False):
    """scan_topk_append: top k over n_sealed sealed keys plus the exact open tail."""
    _need(q, "q", torch.float32, 2)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    h_q, d = q.shape
    h_kv = union_depth.shape[0]
    n_tail = 0
    if tail_k is not None:
        _need(tail_k, "tail_k", torch.float32, 3)
        n_tail = tail_k.shape[1]
    if records is not None:
        _need(records, "records", torch.uint8, device=False)
        if records.numel() < h_kv * d * record_bytes(n_cap):
            raise ValueError("records buffer too small for (h_kv, d, n_cap)")
    if residency is None:
        residency = HBM if records is None or records.is_cuda else HOST_DIRECT
    n = n_sealed + n_tail
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(h_q, h_kv, n, d, k, HBM), 1), dtype=torch.uint8,
                                device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if idx is None:
        idx = torch.empty((h_q, k), dtype=torch.int32, device=q.device)
    _need(idx, "idx", torch.int32)
    if want_scores and scores is None:
        scores = torch.empty((h_q, k), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores, "scores", torch.float32)
    _check(load().scan_topk_append(_ptr(records), residency, n_cap, n_sealed, _ptr(tail_k), n_tail, _ptr(q),
                                   _ptr(depth), _ptr(union_depth), h_q, h_kv, d, k, _ptr(idx), _ptr(scores),
                                   _ptr(workspace), workspace.numel(), _stream(q)))
    return (idx, scores) if want_scores or scores is not None else idx


def device_address(t: torch.Tensor, residency: int | None = None) -> int:
    """fathom_device_address: the address kernels use for tensor ``t`` (device
    memory, or pinned host memory read in place)."""
    if residency is None:
        residency = HBM if t.is_cuda else HOST_DIRECT
    out = ctypes.c_void_p()
    _check(load().fathom_device_address(_ptr(t), residency, ctypes.byref(out)))
    return int(out.value)


def page_table(pages, device="cuda:0", residency: int | None = None) -> torch.Tensor:
    """int64 [h_kv, npages] device tensor of page addresses from ``pages[g][p]``,
    uint8 tensors of [d, record_bytes(page_keys)] bytes each."""
    rows = [[device_address(pg, residency) for pg in head] for head in pages]
    if len({len(r) for r in rows}) != 1:
        raise ValueError("every KV head needs the same number of pages")
    return torch.tensor(rows, dtype=torch.int64, device=device)


def scan_topk_paged(table: torch.Tensor | None, page_keys: int, n_sealed: int, tail_k: torch.Tensor | None,
                    q: torch.Tensor, depth: torch.Tensor, union_depth: torch.Tensor, k: int,
                    residency: int = HOST_DIRECT, workspace: torch.Tensor | None = None,
                    idx: torch.Tensor | None = None, scores: torch.Tensor | None = None,
                    want_scores: bool = False):
    """scan_topk_paged: top k over n_sealed keys in paged records plus the exact open tail."""
    _need(q, "q", torch.float32, 2)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    h_q, d = q.shape
    h_kv = union_depth.shape[0]
    if table is not None:
        _need(table, "table", torch.int64, 2)
        if table.shape[0] != h_kv or table.shape[1] < -(-n_sealed // page_keys):
            raise ValueError("page table must be [h_kv, >= ceil(n_sealed / page_keys)]")
        if table.shape[1] != -(-n_sealed // page_keys):
            table = table[:, :-(-n_sealed // page_keys)].contiguous()
    n_tail = 0
    if tail_k is not None:
        _need(tail_k, "tail_k", torch.float32, 3)
        n_tail = tail_k.shape[1]
    n = n_sealed + n_tail
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(h_q, h_kv, n, d, k, HBM), 1), dtype=torch.uint8,
                                device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if idx is None:
        idx = torch.empty((h_q, k), dtype=torch.int32, device=q.device)
    _need(idx, "idx", torch.int32)
    if want_scores and scores is None:
        scores = torch.empty((h_q, k), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores, "scores", torch.float32)
    _check(load().scan_topk_paged(_ptr(table), residency, page_keys, n_sealed, _ptr(tail_k), n_tail, _ptr(q),
                                  _ptr(depth), _ptr(union_depth), h_q, h_kv, d, k, _ptr(idx), _ptr(scores),
                                  _ptr(workspace), workspace.numel(), _stream(q)))
    return (idx, scores) if want_scores or scores is not None else idx


def pack_nibbles(k: torch.Tensor, status: torch.Tensor | None = None):
    """pack_nibbles: float32 [h_kv, n, d] -> (codes uint8 [h_kv, n, d/2], scales fp16 [h_kv, nb, d])."""
    _need(k, "k", torch.float32, 3)
    h_kv, n, d = k.shape
    codes = torch.empty((h_kv, n, d // 2), dtype=torch.uint8, device=k.device)
    scales = torch.empty((h_kv, -(-n // 128), d), dtype=torch.float16, device=k.device)
    if status is not None:
        _need(status, "status", torch.int32)
    _check(load().pack_nibbles(_ptr(k), h_kv, n, d, _ptr(codes), _ptr(scales), _ptr(status), _stream(k)))
    return codes, scales


def scan_topk_nibbles(codes: torch.Tensor, scales: torch.Tensor, q: torch.Tensor, depth: torch.Tensor,
                      union_depth: torch.Tensor, k: int, residency: int | None = None,
                      workspace: torch.Tensor | None = None, idx: torch.Tensor | None = None,
                      scores: torch.Tensor | None = None, want_scores: bool = False):
    """scan_topk_nibbles: the scan over the token-major 4-bit copy (the free path)."""
    _need(q, "q", torch.float32, 2)
    _need(depth, "depth", torch.uint8)
    _need(union_depth, "union_depth", torch.uint8)
    _need(codes, "codes", torch.uint8, 3, device=False)
    if scales.dtype != torch.float16 or not scales.is_contiguous():
        raise TypeError("scales must be a contiguous float16 tensor")
    h_q, d = q.shape
    h_kv, n, _ = codes.shape
    if residency is None:
        residency = HBM if codes.is_cuda else HOST_DIRECT
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(h_q, h_kv, n, d, k, HBM), 1), dtype=torch.uint8,
                                device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if idx is None:
        idx = torch.empty((h_q, k), dtype=torch.int32, device=q.device)
    _need(idx, "idx", torch.int32)
    if want_scores and scores is None:
        scores = torch.empty((h_q, k), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores, "scores", torch.float32)
    _check(load().scan_topk_nibbles(_ptr(codes), _ptr(scales), residency, _ptr(q), _ptr(depth), _ptr(union_depth),
                                    h_q, h_kv, n, d, k, _ptr(idx), _ptr(scores), _ptr(workspace), workspace.numel(),
                                    _stream(q)))
    return (idx, scores) if want_scores or scores is not None else idx
