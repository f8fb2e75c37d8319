"""ctypes binding of libastr_attn.so (argument marshalling only).

The functions here carry the C names (astr_paged_decode, astr_paged_prefill,
astr_workspace_size, astr_plan_decode, astr_last_error).  They take torch
tensors, check dtype/device/layout, fill the C argument struct with raw
pointers, element strides and the current HIP stream, and call the library.
Every step of the attention runs in the library's HIP kernels; there is no
other implementation behind these calls.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libastr_attn.so")

ASTR_OK = 0
ASTR_ERR_INVALID_ARG = 1
ASTR_ERR_UNSUPPORTED = 2
ASTR_ERR_WORKSPACE = 3
ASTR_ERR_HIP = 4
DEFAULT_MAX_SPLITS = 256
NOALLOC_SCRATCH_BYTES = 32 << 20   # ASTR_NOALLOC_SCRATCH_BYTES
WORKSPACE_COUNTER_BYTES = 32768     # ASTR_WORKSPACE_COUNTER_BYTES: zeroed counter region opening a prefill workspace

EXPORTED = ("astr_workspace_size", "astr_plan_decode", "astr_paged_decode", "astr_paged_decode_noalloc",
            "astr_plan_prefill", "astr_paged_prefill",
            "astr_kv_append", "astr_paged_decode_append", "astr_decode_graph_create", "astr_decode_graph_launch",
            "astr_decode_graph_destroy", "astr_last_error", "astr_abi_version")


class AstrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"astr status {status}: {message}")
        self.status = status
        self.message = message


class PagedArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("o", ctypes.c_void_p), ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("lse_stride_tok", ctypes.c_int64),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("kv_stride_slot", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64), ("num_slots", ctypes.c_int64),
        ("req_to_token", ctypes.c_void_p), ("req_to_token_stride", ctypes.c_int64),
        ("kv_indptr", ctypes.c_void_p), ("kv_indptr_host", ctypes.c_void_p),
        ("qo_indptr", ctypes.c_void_p), ("qo_indptr_host", ctypes.c_void_p),
        ("num_splits", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
        ("timing_events", ctypes.c_void_p),
        ("non_causal", ctypes.c_int32), ("mask", ctypes.c_void_p),
        ("mask_stride_req", ctypes.c_int64), ("mask_stride_row", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
    ]


class NewKV(ctypes.Structure):
    _fields_ = [("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


class DecodePlan(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("num_partials", ctypes.c_int32), ("grid_x", ctypes.c_int32),
                ("grid_y", ctypes.c_int32), ("grid_z", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]


class PrefillPlan(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int32), ("split_tiles", ctypes.c_int32), ("chunk_tiles", ctypes.c_int32),
                ("max_chunks", ctypes.c_int32), ("partial_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_gqa_decode_astr_amd.build` "
                           "(there is no fallback implementation)")
    # Load torch's HIP runtime first so the process holds a single libamdhip64
    # (ours resolves to the already-loaded copy by soname).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.astr_workspace_size.restype = ctypes.c_size_t
    lib.astr_workspace_size.argtypes = [ctypes.c_int32] * 4
    lib.astr_plan_decode.restype = ctypes.c_int
    lib.astr_plan_decode.argtypes = [ctypes.POINTER(PagedArgs), ctypes.c_int32, ctypes.POINTER(DecodePlan)]
    for fn in ("astr_paged_decode", "astr_paged_prefill"):
        f = getattr(lib, fn)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(PagedArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.astr_paged_decode_noalloc.restype = ctypes.c_int
    lib.astr_paged_decode_noalloc.argtypes = [ctypes.POINTER(PagedArgs), ctypes.c_void_p]
    lib.astr_plan_prefill.restype = ctypes.c_int
    lib.astr_plan_prefill.argtypes = [ctypes.POINTER(PagedArgs), ctypes.c_int32, ctypes.POINTER(PrefillPlan)]
    lib.astr_kv_append.restype = ctypes.c_int
    lib.astr_kv_append.argtypes = [ctypes.POINTER(PagedArgs), ctypes.POINTER(NewKV), ctypes.c_void_p]
    lib.astr_paged_decode_append.restype = ctypes.c_int
    lib.astr_paged_decode_append.argtypes = [ctypes.POINTER(PagedArgs), ctypes.POINTER(NewKV), ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]
    lib.astr_decode_graph_create.restype = ctypes.c_int
    lib.astr_decode_graph_create.argtypes = [ctypes.POINTER(PagedArgs), ctypes.POINTER(NewKV), ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.POINTER(ctypes.c_void_p)]
    lib.astr_decode_graph_launch.restype = ctypes.c_int
    lib.astr_decode_graph_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.astr_decode_graph_destroy.restype = ctypes.c_int
    lib.astr_decode_graph_destroy.argtypes = [ctypes.c_void_p]
    lib.astr_last_error.restype = ctypes.c_char_p
    lib.astr_last_error.argtypes = []
    lib.astr_abi_version.restype = ctypes.c_int
    lib.astr_abi_version.argtypes = []
    _lib = lib
    return lib


def astr_last_error() -> str:
    return load_library().astr_last_error().decode()


def astr_workspace_size(batch: int, num_qo_heads: int, head_dim: int, max_splits: int = 0) -> int:
    return int(load_library().astr_workspace_size(batch, num_qo_heads, head_dim, max_splits))


def _check(status: int):
    if status != ASTR_OK:
        raise AstrError(status, astr_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _host_i32(x):
    """Host int32 copy of an index array (numpy or CPU tensor); kept alive by the caller."""
    if x is None:
        return None
    if isinstance(x, np.ndarray) and x.dtype == np.int32 and x.flags.c_contiguous:
        return x
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _np_ptr(a):
    return None if a is None else a.ctypes.data


def make_args(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, *, sm_scale,
              req_to_token_stride, lse=None, qo_indptr=None, qo_indptr_host=None, num_splits=0,
              max_q_len=0, timing_events=None, non_causal=False, mask=None, page_size=1):
    """Fill the C argument struct from tensors.  Returns (args, keepalive).

    mask: None, or a uint8 / bool tensor [B, kv_len] (2-D) or [B, q_len, kv_len] (3-D) with a
    contiguous last dimension; nonzero = visible."""
    import torch

    bf16, i32 = torch.bfloat16, torch.int32
    qs, ks, vs, os_ = q.stride(), k_pool.stride(), v_pool.stride(), o.stride()
    for name, t, st in (("q", q, qs), ("k_pool", k_pool, ks), ("v_pool", v_pool, vs), ("o", o, os_)):
        if t.dtype != bf16:
            raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")
        if len(st) != 3 or st[2] != 1:
            raise ValueError(f"{name} must be 3-D with a contiguous last dimension")
    for name, t in (("req_to_token", req_to_token), ("kv_indptr", kv_indptr), ("qo_indptr", qo_indptr)):
        if t is not None and (t.dtype != i32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous int32 tensor")
    lse_stride = 0
    if lse is not None:
        ls = lse.stride()
        if lse.dtype != torch.float32 or len(ls) != 2 or ls[1] != 1:
            raise TypeError("lse must be a 2-D float32 tensor with contiguous last dimension")
        lse_stride = ls[0]
    if ks != vs or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape and strides")
    kvh = _host_i32(kv_indptr_host)
    qoh = _host_i32(qo_indptr_host)
    mask_ptr, mask_req, mask_row = None, 0, 0
    if mask is not None:
        if mask.dtype not in (torch.uint8, torch.bool) or mask.dim() not in (2, 3) or mask.stride(-1) != 1:
            raise TypeError("mask must be a 2-D or 3-D uint8/bool tensor with a contiguous last dimension")
        mask_ptr = mask.data_ptr()
        mask_req = mask.stride(0)
        mask_row = mask.stride(1) if mask.dim() == 3 else 0
    ev, ev_ptr = None, None
    if timing_events is not None:
        ev = (ctypes.c_void_p * len(timing_events))(*[None if e is None else e.cuda_event for e in timing_events])
        ev_ptr = ctypes.addressof(ev)
    qshape = q.shape
    a = PagedArgs(
        batch=kv_indptr.numel() - 1, num_qo_heads=qshape[1], num_kv_heads=k_pool.shape[1], head_dim=qshape[2],
        sm_scale=float(sm_scale),
        q=q.data_ptr(), q_stride_tok=qs[0], q_stride_head=qs[1],
        o=o.data_ptr(), o_stride_tok=os_[0], o_stride_head=os_[1],
        lse=_ptr(lse), lse_stride_tok=lse_stride,
        k_pool=k_pool.data_ptr(), v_pool=v_pool.data_ptr(),
        kv_stride_slot=ks[0], kv_stride_head=ks[1], num_slots=k_pool.shape[0],
        req_to_token=req_to_token.data_ptr(), req_to_token_stride=int(req_to_token_stride),
        kv_indptr=kv_indptr.data_ptr(), kv_indptr_host=_np_ptr(kvh),
        qo_indptr=_ptr(qo_indptr), qo_indptr_host=_np_ptr(qoh),
        num_splits=int(num_splits), max_q_len=int(max_q_len), timing_events=ev_ptr,
        non_causal=1 if non_causal else 0, mask=mask_ptr, mask_stride_req=mask_req, mask_stride_row=mask_row,
        page_size=int(page_size))
    return a, (kvh, qoh, ev)


def _stream_handle(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def astr_plan_decode(args: PagedArgs, num_cus: int = 0) -> DecodePlan:
    plan = DecodePlan()
    _check(load_library().astr_plan_decode(ctypes.byref(args), int(num_cus), ctypes.byref(plan)))
    return plan


def astr_paged_decode(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, workspace, *,
                      sm_scale, req_to_token_stride, lse=None, num_splits=0, stream=None, timing_events=None,
                      mask=None, page_size=1):
    """Paged GQA decode: q [B, Hq, D] bf16 -> o [B, Hq, D] bf16 (+ lse [B, Hq] fp32).

    timing_events: optional 4 HipEvent or None (hip_events.py): start/end stamps of the
    split kernel, then of the combine kernel (None entries are skipped)."""
    if timing_events is not None and len(timing_events) != 4:
        raise ValueError("decode timing_events takes 4 events (split start/end, combine start/end)")
    lib = load_library()
    a, keep = make_args(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, sm_scale=sm_scale,
                        req_to_token_stride=req_to_token_stride, lse=lse, num_splits=num_splits,
                        timing_events=timing_events, mask=mask, page_size=page_size)
    ws_ptr = _ptr(workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.astr_paged_decode(ctypes.byref(a), ws_ptr, ws_bytes, _stream_handle(stream)))
    del keep


def astr_paged_decode_noalloc(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, *, sm_scale,
                              req_to_token_stride, lse=None, num_splits=0, stream=None, mask=None, page_size=1):
    """Allocation-free paged GQA decode: as astr_paged_decode, with the split partials in the
    library's fixed device scratch array instead of a caller workspace (no workspace argument)."""
    lib = load_library()
    a, keep = make_args(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, sm_scale=sm_scale,
                        req_to_token_stride=req_to_token_stride, lse=lse, num_splits=num_splits, mask=mask,
                        page_size=page_size)
    _check(lib.astr_paged_decode_noalloc(ctypes.byref(a), _stream_handle(stream)))
    del keep


def astr_plan_prefill(args: PagedArgs, num_cus: int = 0) -> PrefillPlan:
    plan = PrefillPlan()
    _check(load_library().astr_plan_prefill(ctypes.byref(args), int(num_cus), ctypes.byref(plan)))
    return plan


def astr_paged_prefill(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, qo_indptr, qo_indptr_host,
                       o, *, sm_scale, req_to_token_stride, lse=None, max_q_len=0, stream=None,
                       timing_events=None, non_causal=False, mask=None, page_size=1, workspace=None):
    """Ragged paged prefill: q [sum q_len, Hq, D] bf16 in qo_indptr order -> o (+ lse).

    workspace: None (every query tile whole) or a device tensor of at least astr_plan_prefill's
    workspace_bytes, zeroed before its first use (long query tiles are then split over several
    work groups).  timing_events: optional 2 HipEvent (hip_events.py): start/end stamps of the
    prefill kernel."""
    if timing_events is not None and len(timing_events) != 2:
        raise ValueError("prefill timing_events takes 2 events (kernel start/end)")
    lib = load_library()
    a, keep = make_args(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, sm_scale=sm_scale,
                        req_to_token_stride=req_to_token_stride, lse=lse, qo_indptr=qo_indptr,
                        qo_indptr_host=qo_indptr_host, max_q_len=max_q_len, timing_events=timing_events,
                        non_causal=non_causal, mask=mask, page_size=page_size)
    ws_ptr = _ptr(workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.astr_paged_prefill(ctypes.byref(a), ws_ptr, ws_bytes, _stream_handle(stream)))
    del keep


def make_new_kv(k_new, v_new) -> NewKV:
    """C view of the new tokens' rows k_new / v_new [rows, Hkv, D] bf16 (same strides)."""
    import torch

    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be 3-D with a contiguous last dimension")
    if k_new.stride() != v_new.stride() or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have the same shape and strides")
    n = NewKV()
    n.k_new = _ptr(k_new)
    n.v_new = _ptr(v_new)
    n.stride_tok, n.stride_head = k_new.stride(0), k_new.stride(1)
    return n


def astr_kv_append(k_new, v_new, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, *,
                   req_to_token_stride, qo_indptr=None, qo_indptr_host=None, max_q_len=0, stream=None,
                   timing_events=None, page_size=1):
    """Write the new tokens' rows k_new / v_new [sum n_b, Hkv, D] bf16 into the pools (in place).

    kv_indptr counts the new tokens; n_b = 1 per request without qo_indptr (decode), else
    qo_indptr[b+1] - qo_indptr[b].  timing_events: optional 2 HipEvent (kernel start/end)."""
    import torch

    if timing_events is not None and len(timing_events) != 2:
        raise ValueError("append timing_events takes 2 events (kernel start/end)")
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
            raise TypeError(f"{name} must be a 3-D bfloat16 tensor with a contiguous last dimension")
    if k_pool.stride() != v_pool.stride() or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape and strides")
    if k_new.shape[1:] != k_pool.shape[1:]:
        raise ValueError(f"new rows {tuple(k_new.shape)} do not match the pool rows {tuple(k_pool.shape)}")
    for name, t in (("req_to_token", req_to_token), ("kv_indptr", kv_indptr), ("qo_indptr", qo_indptr)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous int32 tensor")
    lib = load_library()
    kvh = _host_i32(kv_indptr_host)
    qoh = _host_i32(qo_indptr_host)
    rows = int(qoh[-1]) if qoh is not None else kv_indptr.numel() - 1
    if k_new.shape[0] != rows:
        raise ValueError(f"k_new has {k_new.shape[0]} rows; the new-token counts need {rows}")
    a = PagedArgs()
    a.batch = kv_indptr.numel() - 1
    a.num_kv_heads = k_pool.shape[1]
    a.num_qo_heads = k_pool.shape[1]
    a.head_dim = k_pool.shape[2]
    a.k_pool = _ptr(k_pool)
    a.v_pool = _ptr(v_pool)
    a.kv_stride_slot, a.kv_stride_head = k_pool.stride(0), k_pool.stride(1)
    a.num_slots = k_pool.shape[0]
    a.req_to_token = _ptr(req_to_token)
    a.req_to_token_stride = int(req_to_token_stride)
    a.kv_indptr = _ptr(kv_indptr)
    a.kv_indptr_host = _np_ptr(kvh)
    a.qo_indptr = _ptr(qo_indptr)
    a.qo_indptr_host = _np_ptr(qoh)
    a.max_q_len = int(max_q_len)
    a.page_size = int(page_size)
    ev = None
    if timing_events is not None:
        ev = (ctypes.c_void_p * 2)(*[None if e is None else e.cuda_event for e in timing_events])
        a.timing_events = ctypes.cast(ev, ctypes.c_void_p)
    nkv = make_new_kv(k_new, v_new)
    _check(lib.astr_kv_append(ctypes.byref(a), ctypes.byref(nkv), _stream_handle(stream)))
    del kvh, qoh, ev


def astr_paged_decode_append(q, k_new, v_new, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o,
                             workspace, *, sm_scale, req_to_token_stride, lse=None, num_splits=0, stream=None,
                             timing_events=None, mask=None, page_size=1):
    """Fused KV append + paged decode: writes k_new / v_new [B, Hkv, D] (request b's new token, its last
    position) into the pools and decodes q [B, Hq, D] -> o (+ lse), bit-identical to astr_kv_append
    followed by astr_paged_decode.  timing_events as astr_paged_decode."""
    if timing_events is not None and len(timing_events) != 4:
        raise ValueError("decode timing_events takes 4 events (split start/end, combine start/end)")
    if k_new.shape[0] != q.shape[0] or k_new.shape[1:] != k_pool.shape[1:]:
        raise ValueError(f"new rows {tuple(k_new.shape)} must be [B, Hkv, D] for q {tuple(q.shape)} and pool "
                         f"{tuple(k_pool.shape)}")
    lib = load_library()
    a, keep = make_args(q, k_pool, v_pool, req_to_token, kv_indptr, kv_indptr_host, o, sm_scale=sm_scale,
                        req_to_token_stride=req_to_token_stride, lse=lse, num_splits=num_splits,
                        timing_events=timing_events, mask=mask, page_size=page_size)
    nkv = make_new_kv(k_new, v_new)
    ws_ptr = _ptr(workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.astr_paged_decode_append(ctypes.byref(a), ctypes.byref(nkv), ws_ptr, ws_bytes,
                                        _stream_handle(stream)))
    del keep


class DecodeGraph:
    """A captured multi-layer decode step (astr_decode_graph_*): warm-up, capture, replay.

    layers: one dict per layer with the astr_paged_decode tensors (q, k_pool, v_pool, req_to_token,
    kv_indptr, kv_indptr_host, o, and optionally lse, mask, k_new / v_new for the fused append) plus
    sm_scale, req_to_token_stride and optionally page_size.  The graph holds the device addresses it
    was captured with, so this object keeps a reference to every layer tensor and the workspace until
    close(); a launch reads their current contents.  num_splits fixes the plan (required for capture)."""

    def __init__(self, layers, workspace, *, num_splits, stream):
        lib = load_library()
        n = len(layers)
        arr = (PagedArgs * n)()
        keep = []
        fused = [("k_new" in L and L["k_new"] is not None) for L in layers]
        if any(fused) and not all(fused):
            raise ValueError("either every layer or no layer takes new rows")
        nkv = (NewKV * n)() if all(fused) else None
        for i, L in enumerate(layers):
            a, k = make_args(L["q"], L["k_pool"], L["v_pool"], L["req_to_token"], L["kv_indptr"],
                             L["kv_indptr_host"], L["o"], sm_scale=L["sm_scale"],
                             req_to_token_stride=L["req_to_token_stride"], lse=L.get("lse"), num_splits=num_splits,
                             mask=L.get("mask"), page_size=L.get("page_size", 1))
            arr[i] = a
            keep.append(k)
            if nkv is not None:
                nkv[i] = make_new_kv(L["k_new"], L["v_new"])
        self._stream = stream
        self._handle = None
        self._keep = None
        handle = ctypes.c_void_p()
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib.astr_decode_graph_create(arr, nkv, n, _ptr(workspace), ws_bytes, ctypes.c_void_p(stream.cuda_stream),
                                            ctypes.byref(handle)))
        self._handle = handle
        self.num_layers = n
        # The captured kernels read and write these tensors by address: keep them alive with the graph.
        self._keep = (list(layers), workspace, keep, arr, nkv)

    def launch(self, stream=None):
        s = self._stream if stream is None else stream
        _check(load_library().astr_decode_graph_launch(self._handle, ctypes.c_void_p(s.cuda_stream)))

    def close(self):
        if self._handle is not None and self._handle.value:
            _check(load_library().astr_decode_graph_destroy(self._handle))
        self._handle = None
        self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
