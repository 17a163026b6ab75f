"""ctypes binding of libdocmask_gqa.so: argument marshalling only.

Every computation runs in the HIP library; this module reads shapes from
torch tensors, checks dtypes/devices/contiguity, allocates outputs and the
workspace with torch (device memory plumbing) and passes raw device pointers
and the current HIP stream through the C ABI declared in
include/docmask_gqa.h.  If the library is missing it raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
# DMGQA_LIBRARY selects another build of the same library (the host
# sanitizer build of the tests); there is no fallback either way.
LIB_PATH = os.environ.get("DMGQA_LIBRARY") or os.path.join(HERE, "libdocmask_gqa.so")

DMGQA_OK = 0
DMGQA_ERR_INVALID_ARG = -1
DMGQA_ERR_UNSUPPORTED = -2
DMGQA_ERR_WORKSPACE = -3
DMGQA_ERR_HIP = -4

DMGQA_BWD_PATH_RECOMPUTE = 0
DMGQA_BWD_PATH_STASH = 1
DMGQA_BWD_PATH_MIXED = 2

_lib = None

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

# (name, restype, argtypes) of every exported function.
SIGNATURES = {
    "docmask_gqa_fwd_workspace_size": (_sz, [_i32] * 7),
    "docmask_gqa_bwd_workspace_size": (_sz, [_i32] * 7),
    "docmask_gqa_bwd_workspace_size_min": (_sz, [_i32] * 7),
    "docmask_gqa_bwd_workspace_size_full": (_sz, [_i32] * 7),
    "docmask_gqa_bwd_path": (ctypes.c_int, [_i32] * 8 + [_sz]),
    "docmask_gqa_attn_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                            _sz, _vp]),
    "docmask_gqa_attn_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                            _vp, _vp, _vp, _sz, _vp]),
    "docmask_gqa_attn_fwd_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                                    _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                                    _vp, _vp]),
    "docmask_gqa_attn_fwd_bounds": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                                   _sz, _vp]),
    "docmask_gqa_attn_bwd_bounds": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                   _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                   _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "docmask_gqa_batch_plan_size": (_sz, [_i32] * 7),
    "docmask_gqa_batch_plan": (ctypes.c_int, [_vp, _vp] + [_i32] * 9 + [_vp, _sz, _vp]),
    "docmask_gqa_attn_fwd_plan": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                                 _sz, _vp]),
    "docmask_gqa_attn_bwd_plan": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                 _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                 _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "docmask_gqa_doc_bounds_size": (_sz, [_i32] * 3),
    "docmask_gqa_doc_bounds": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "docmask_gqa_check_docs": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "docmask_gqa_check_cu_seqlens": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "docmask_gqa_interval_bounds": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "docmask_gqa_check_intervals": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "docmask_gqa_fwd_cross_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "docmask_gqa_attn_fwd_cross": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "docmask_gqa_bwd_cross_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "docmask_gqa_bwd_cross_workspace_size_min": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "docmask_gqa_bwd_cross_path": (ctypes.c_int, [_i32] * 6 + [_sz]),
    "docmask_gqa_attn_bwd_cross": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                  _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                                  _vp, _vp, _sz, _vp]),
    "docmask_gqa_check_cross_intervals": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "docmask_gqa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "docmask_gqa_version": (ctypes.c_int, []),
    "docmask_gqa_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "docmask_gqa_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                               ctypes.POINTER(ctypes.c_int)]),
    "docmask_gqa_kernel_count": (ctypes.c_int, []),
    "docmask_gqa_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
}


class DocmaskGQAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m context_gqa_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().docmask_gqa_status_string(int(status)).decode()


def docmask_gqa_status_string(status: int) -> str:
    return status_string(status)


def docmask_gqa_fwd_workspace_size(B, S, Skv, Hq, Hkv, D, cp_size) -> int:
    return int(lib().docmask_gqa_fwd_workspace_size(B, S, Skv, Hq, Hkv, D, cp_size))


def docmask_gqa_bwd_workspace_size(B, S, Skv, Hq, Hkv, D, cp_size) -> int:
    return int(lib().docmask_gqa_bwd_workspace_size(B, S, Skv, Hq, Hkv, D, cp_size))


def docmask_gqa_bwd_workspace_size_min(B, S, Skv, Hq, Hkv, D, cp_size) -> int:
    return int(lib().docmask_gqa_bwd_workspace_size_min(B, S, Skv, Hq, Hkv, D, cp_size))


def docmask_gqa_bwd_workspace_size_full(B, S, Skv, Hq, Hkv, D, cp_size) -> int:
    return int(lib().docmask_gqa_bwd_workspace_size_full(B, S, Skv, Hq, Hkv, D, cp_size))


def docmask_gqa_bwd_path(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank, workspace_bytes) -> int:
    """DMGQA_BWD_PATH_* the backward takes with this workspace (or a negative
    status)."""
    return int(lib().docmask_gqa_bwd_path(B, S, Skv, Hq, Hkv, D, cp_size, cp_rank,
                                          int(workspace_bytes)))


def docmask_gqa_bwd_cross_path(B, S, Skv, Hq, Hkv, D, workspace_bytes) -> int:
    """DMGQA_BWD_PATH_* the cross-attention backward takes with this
    workspace (or a negative status)."""
    return int(lib().docmask_gqa_bwd_cross_path(B, S, Skv, Hq, Hkv, D, int(workspace_bytes)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, name, dtype, ndim):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _bounds_ok(bounds, doc_ids, cu_seqlens, B, S, Skv):
    import torch
    if doc_ids is not None or cu_seqlens is not None:
        raise ValueError("pass either bounds or doc_ids / cu_seqlens")
    _need(bounds, "bounds", torch.int32, 1)
    if bounds.numel() * 4 < docmask_gqa_doc_bounds_size(B, S, Skv):
        raise ValueError("bounds is smaller than docmask_gqa_doc_bounds_size(B, S, Skv)")


def _mask_form(doc_ids, cu_seqlens, bounds, plan, B, S, Skv, Hq, Hkv, D, cp_size):
    """Which masking input a call got: "docs" (doc_ids / cu_seqlens),
    "bounds" or "plan" (exactly one form)."""
    import torch
    if plan is not None:
        if bounds is not None or doc_ids is not None or cu_seqlens is not None:
            raise ValueError("pass plan alone, without bounds / doc_ids / cu_seqlens")
        _need(plan, "plan", torch.int32, 1)
        if plan.numel() * 4 < docmask_gqa_batch_plan_size(B, S, Skv, Hq, Hkv, D, cp_size):
            raise ValueError("plan is smaller than docmask_gqa_batch_plan_size")
        return "plan"
    if bounds is not None:
        _bounds_ok(bounds, doc_ids, cu_seqlens, B, S, Skv)
        return "bounds"
    return "docs"


def _docs(doc_ids, cu_seqlens, B, S):
    import torch
    if (doc_ids is None) == (cu_seqlens is None):
        raise ValueError("pass exactly one of doc_ids / cu_seqlens")
    if doc_ids is not None:
        _need(doc_ids, "doc_ids", torch.int32, 2)
        if tuple(doc_ids.shape) != (B, S):
            raise ValueError(f"doc_ids must be [B, S] = [{B}, {S}]")
        return doc_ids, None, 0
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    return None, cu_seqlens, cu_seqlens.numel() - 1


def docmask_gqa_doc_bounds_size(B, S, Skv) -> int:
    return int(lib().docmask_gqa_doc_bounds_size(B, S, Skv))


def docmask_gqa_doc_bounds(doc_ids=None, cu_seqlens=None, *, B: int, S: int, Skv: int,
                           out=None, stream=None):
    """Document bounds [2, B, Skv] int32 (first position of each key's
    document, one past its last), followed by scratch, as one int32 buffer
    for the attention calls' `bounds=` argument."""
    import torch
    doc_ids, cu_seqlens, n_docs = _docs(doc_ids, cu_seqlens, B, S)
    need = docmask_gqa_doc_bounds_size(B, S, Skv)
    dev = (doc_ids if doc_ids is not None else cu_seqlens).device
    if out is None:
        out = torch.empty(max(need // 4, 1), dtype=torch.int32, device=dev)
    _need(out, "bounds", torch.int32, 1)
    rc = lib().docmask_gqa_doc_bounds(_ptr(doc_ids), _ptr(cu_seqlens), n_docs, B, S, Skv,
                                      _ptr(out), out.numel() * 4, _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_doc_bounds")
    return out


def docmask_gqa_batch_plan_size(B, S, Skv, Hq, Hkv, D, cp_size) -> int:
    return int(lib().docmask_gqa_batch_plan_size(B, S, Skv, Hq, Hkv, D, cp_size))


def docmask_gqa_batch_plan(doc_ids=None, cu_seqlens=None, *, B: int, S: int, Skv: int, Hq: int,
                           Hkv: int, D: int, cp_size: int, cp_rank: int, out=None,
                           stream=None):
    """Bounds and query-tile orders of one batch layout as one int32 buffer,
    for the attention calls' `plan=` argument (its first 2 * B * Skv entries
    are the bounds array of docmask_gqa_doc_bounds)."""
    import torch
    doc_ids, cu_seqlens, n_docs = _docs(doc_ids, cu_seqlens, B, S)
    need = docmask_gqa_batch_plan_size(B, S, Skv, Hq, Hkv, D, cp_size)
    dev = (doc_ids if doc_ids is not None else cu_seqlens).device
    if out is None:
        out = torch.empty(max(need // 4, 1), dtype=torch.int32, device=dev)
    _need(out, "plan", torch.int32, 1)
    rc = lib().docmask_gqa_batch_plan(_ptr(doc_ids), _ptr(cu_seqlens), n_docs, B, S, Skv, Hq,
                                      Hkv, D, cp_size, cp_rank, _ptr(out), out.numel() * 4,
                                      _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_batch_plan")
    return out


def docmask_gqa_attn_fwd(q, k, v, doc_ids=None, cu_seqlens=None, *, cp_size: int,
                         cp_rank: int, softmax_scale: Optional[float] = None, out=None,
                         lse=None, workspace=None, stream=None,
                         bounds=None, plan=None) -> Tuple["object", "object"]:
    """out [B,Sq,Hq,D] bf16 and lse [B,Sq,Hq] fp32 of the rank's local rows.
    q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] bf16; doc_ids [B,S] or cu_seqlens
    [n_docs+1] int32 with S = Sq * cp_size, or bounds from
    docmask_gqa_doc_bounds, or a plan from docmask_gqa_batch_plan."""
    import torch
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Skv, Hkv, D] matching q")
    S = Sq * cp_size
    form = _mask_form(doc_ids, cu_seqlens, bounds, plan, B, S, Skv, Hq, Hkv, D, cp_size)
    if form == "docs":
        doc_ids, cu_seqlens, n_docs = _docs(doc_ids, cu_seqlens, B, S)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Sq, Hq, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    need = docmask_gqa_fwd_workspace_size(B, S, Skv, Hq, Hkv, D, cp_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if form == "docs":
        rc = lib().docmask_gqa_attn_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(doc_ids), _ptr(cu_seqlens), n_docs, B, S, Skv, Hq,
            Hkv, D, cp_size, cp_rank, float(softmax_scale), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    else:
        fn = lib().docmask_gqa_attn_fwd_bounds if form == "bounds" else \
            lib().docmask_gqa_attn_fwd_plan
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(bounds if form == "bounds" else plan), B, S,
                Skv, Hq, Hkv, D, cp_size, cp_rank, float(softmax_scale), _ptr(out), _ptr(lse),
                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_attn_fwd")
    return out, lse


def docmask_gqa_attn_fwd_noalloc(q, k, v, doc_ids=None, cu_seqlens=None, *, cp_size: int,
                                 cp_rank: int, out, lse, softmax_scale: Optional[float] = None,
                                 stream=None) -> Tuple["object", "object"]:
    """The forward with the library's fixed per-GPU scratch instead of a
    workspace (no allocation in the call; out and lse are the caller's).
    Calls overlapping on one GPU race."""
    import torch
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Skv, Hkv, D] matching q")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Sq, Hq):
        raise ValueError("out must match q and lse be [B, Sq, Hq]")
    S = Sq * cp_size
    doc_ids, cu_seqlens, n_docs = _docs(doc_ids, cu_seqlens, B, S)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rc = lib().docmask_gqa_attn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(doc_ids), _ptr(cu_seqlens), n_docs, B, S, Skv, Hq, Hkv,
        D, cp_size, cp_rank, float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_attn_fwd_noalloc")
    return out, lse


def docmask_gqa_attn_bwd(q, k, v, out, dout, lse, doc_ids=None, cu_seqlens=None, *,
                         cp_size: int, cp_rank: int, softmax_scale: Optional[float] = None,
                         dq=None, dk=None, dv=None, workspace=None, stream=None, bounds=None,
                         plan=None):
    """dq [B,Sq,Hq,D] bf16, dk/dv [B,Skv,Hkv,D] fp32.  Masking by doc_ids /
    cu_seqlens, by bounds from docmask_gqa_doc_bounds, or by a plan from
    docmask_gqa_batch_plan."""
    import torch
    for t, n in ((q, "q"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must match q")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must match")
    S = Sq * cp_size
    form = _mask_form(doc_ids, cu_seqlens, bounds, plan, B, S, Skv, Hq, Hkv, D, cp_size)
    if form == "docs":
        doc_ids, cu_seqlens, n_docs = _docs(doc_ids, cu_seqlens, B, S)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=k.device)
    if dv is None:
        dv = torch.empty(k.shape, dtype=torch.float32, device=k.device)
    _need(dq, "dq", torch.bfloat16, 4)
    _need(dk, "dk", torch.float32, 4)
    _need(dv, "dv", torch.float32, 4)
    need = docmask_gqa_bwd_workspace_size(B, S, Skv, Hq, Hkv, D, cp_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if form == "docs":
        rc = lib().docmask_gqa_attn_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(doc_ids),
            _ptr(cu_seqlens), n_docs, B, S, Skv, Hq, Hkv, D, cp_size, cp_rank,
            float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    else:
        fn = lib().docmask_gqa_attn_bwd_bounds if form == "bounds" else \
            lib().docmask_gqa_attn_bwd_plan
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                _ptr(bounds if form == "bounds" else plan), B, S, Skv, Hq, Hkv, D, cp_size,
                cp_rank, float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_attn_bwd")
    return dq, dk, dv


def docmask_gqa_check_docs(doc_ids, stream=None) -> int:
    """0 if every document id forms one contiguous run (synchronises)."""
    import torch
    _need(doc_ids, "doc_ids", torch.int32, 2)
    B, S = doc_ids.shape
    rc = lib().docmask_gqa_check_docs(_ptr(doc_ids), B, S, _stream(stream))
    if rc < 0:
        raise DocmaskGQAError(rc, "docmask_gqa_check_docs")
    return rc


def docmask_gqa_interval_bounds(lo, *, Skv: int, out=None, stream=None):
    """Bounds of the causal interval mask "query p attends to keys lo[b, p] .. p"
    (lo int32 [B, S], non-decreasing along p, 0 <= lo[p] <= p) for the
    attention calls' `bounds=` argument; same buffer as docmask_gqa_doc_bounds."""
    import torch
    _need(lo, "lo", torch.int32, 2)
    B, S = lo.shape
    need = docmask_gqa_doc_bounds_size(B, S, Skv)
    if out is None:
        out = torch.empty(max(need // 4, 1), dtype=torch.int32, device=lo.device)
    _need(out, "bounds", torch.int32, 1)
    rc = lib().docmask_gqa_interval_bounds(_ptr(lo), B, S, Skv, _ptr(out), out.numel() * 4,
                                           _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_interval_bounds")
    return out


def docmask_gqa_check_intervals(lo, stream=None) -> int:
    """0 if every row of lo [B, S] is non-decreasing with 0 <= lo[p] <= p
    (synchronises)."""
    import torch
    _need(lo, "lo", torch.int32, 2)
    B, S = lo.shape
    rc = lib().docmask_gqa_check_intervals(_ptr(lo), B, S, _stream(stream))
    if rc < 0:
        raise DocmaskGQAError(rc, "docmask_gqa_check_intervals")
    return rc


def docmask_gqa_attn_fwd_cross(q, k, v, lo, hi, *, softmax_scale: Optional[float] = None,
                               out=None, lse=None, workspace=None, stream=None):
    """Cross-attention forward: query token p of q [B,S,Hq,D] attends to keys
    lo[b,p] .. hi[b,p]-1 of k/v [B,Skv,Hkv,D] (lo, hi int32 [B,S],
    non-decreasing, 0 <= lo < hi <= Skv).  Returns out [B,S,Hq,D] bf16 and
    lse [B,S,Hq] fp32."""
    import torch
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(lo, "lo", torch.int32, 2)
    _need(hi, "hi", torch.int32, 2)
    B, S, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Skv, Hkv, D] matching q")
    if tuple(lo.shape) != (B, S) or tuple(hi.shape) != (B, S):
        raise ValueError("lo and hi must be [B, S]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, S, Hq, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    need = lib().docmask_gqa_fwd_cross_workspace_size(B, S, Skv, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib().docmask_gqa_attn_fwd_cross(
        _ptr(q), _ptr(k), _ptr(v), _ptr(lo), _ptr(hi), B, S, Skv, Hq, Hkv, D,
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_attn_fwd_cross")
    return out, lse


def docmask_gqa_attn_bwd_cross(q, k, v, out, dout, lse, lo, hi, *,
                               softmax_scale: Optional[float] = None, dq=None, dk=None,
                               dv=None, workspace=None, stream=None):
    """Cross-attention backward (same masking as docmask_gqa_attn_fwd_cross):
    dq [B,S,Hq,D] bf16, dk/dv [B,Skv,Hkv,D] fp32 from the forward's out and
    lse and the output gradient dout."""
    import torch
    for t, n in ((q, "q"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(lo, "lo", torch.int32, 2)
    _need(hi, "hi", torch.int32, 2)
    B, S, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must match q")
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Skv, Hkv, D] matching q")
    if tuple(lo.shape) != (B, S) or tuple(hi.shape) != (B, S):
        raise ValueError("lo and hi must be [B, S]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=k.device)
    if dv is None:
        dv = torch.empty(k.shape, dtype=torch.float32, device=k.device)
    _need(dq, "dq", torch.bfloat16, 4)
    _need(dk, "dk", torch.float32, 4)
    _need(dv, "dv", torch.float32, 4)
    need = lib().docmask_gqa_bwd_cross_workspace_size(B, S, Skv, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    rc = lib().docmask_gqa_attn_bwd_cross(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(lo), _ptr(hi), B, S,
        Skv, Hq, Hkv, D, float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != DMGQA_OK:
        raise DocmaskGQAError(rc, "docmask_gqa_attn_bwd_cross")
    return dq, dk, dv


def docmask_gqa_check_cross_intervals(lo, hi, Skv: int, stream=None) -> int:
    """0 if lo, hi [B, S] are non-decreasing with 0 <= lo < hi <= Skv
    (synchronises)."""
    import torch
    _need(lo, "lo", torch.int32, 2)
    _need(hi, "hi", torch.int32, 2)
    B, S = lo.shape
    rc = lib().docmask_gqa_check_cross_intervals(_ptr(lo), _ptr(hi), B, S, Skv, _stream(stream))
    if rc < 0:
        raise DocmaskGQAError(rc, "docmask_gqa_check_cross_intervals")
    return rc


def docmask_gqa_check_cu_seqlens(cu_seqlens, S: int, stream=None) -> int:
    """0 if cu_seqlens is a valid offset list ending at S (synchronises)."""
    import torch
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    rc = lib().docmask_gqa_check_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, S,
                                            _stream(stream))
    if rc < 0:
        raise DocmaskGQAError(rc, "docmask_gqa_check_cu_seqlens")
    return rc


def docmask_gqa_version() -> int:
    return int(lib().docmask_gqa_version())


def docmask_gqa_timing_enable(on: bool) -> None:
    lib().docmask_gqa_timing_enable(1 if on else 0)


def docmask_gqa_kernel_times() -> dict:
    """{kernel name: (total ms, launches)} recorded since timing was enabled
    (waits for the recorded events)."""
    l = lib()
    res = {}
    for i in range(l.docmask_gqa_kernel_count()):
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int(0)
        rc = l.docmask_gqa_timing_read(i, ctypes.byref(ms), ctypes.byref(n))
        if rc != DMGQA_OK:
            raise DocmaskGQAError(rc, "docmask_gqa_timing_read")
        res[l.docmask_gqa_kernel_name(i).decode()] = (ms.value, n.value)
    return res
