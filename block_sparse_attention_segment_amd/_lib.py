"""ctypes binding of libblockrank (the C ABI in include/blockrank.h).

Argument marshalling only: every step of the computation runs in the HIP library.  PyTorch
provides device memory (tensors) and the stream (torch.cuda.current_stream()).  If the built
library is missing, loading raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblockrank.so")

BR_OK, BR_ERR_INVALID_ARG, BR_ERR_UNSUPPORTED, BR_ERR_WORKSPACE, BR_ERR_HIP = range(5)

# Symbols the header declares; the CPU test checks the library exports each of them.
EXPORTED = ("br_attn_workspace_bytes", "br_attn_fwd", "br_attn_fwd_timed", "br_attn_fwd_noalloc", "br_attn_fwd_sink",
            "br_attn_fwd_rope_workspace_bytes", "br_attn_fwd_rope", "br_doc_scores_workspace_bytes", "br_doc_scores",
            "br_sort_docs", "br_rank_workspace_bytes", "br_rank_prompts", "br_rank_prompts_timed", "br_attn_plan_items", "br_attn_plan_schedule", "br_query_attn_workspace_bytes", "br_query_attn_fwd", "br_attn_routed_workspace_bytes", "br_attn_routed_fwd",
            "br_attn_bwd_workspace_bytes", "br_attn_bwd", "br_attn_bwd_plan_items",
            "br_infonce_workspace_bytes", "br_infonce", "br_doc_scores_bwd_workspace_bytes", "br_doc_scores_bwd",
            "br_ssmax_softmax_scale", "br_rope_workspace_bytes", "br_rope_fwd", "br_rope_signal_fwd", "br_rope_positions",
            "br_status_string", "br_last_error", "br_version")


class BrDims(ctypes.Structure):
    _fields_ = [("num_prompts", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64)]


class BlockRankError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status
        self.message = message


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def load_library() -> ctypes.CDLL:
    """Load libblockrank.so from the package directory (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_segment_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    dims_p = ctypes.POINTER(BrDims)
    sz_p = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "br_attn_workspace_bytes": [dims_p, _I32P, _I32P, sz_p],
        "br_attn_fwd": [dims_p, _P, _P, _P, _I32P, _I32P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t, _P],
        "br_attn_fwd_timed": [dims_p, _P, _P, _P, _I32P, _I32P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t, _P,
                              _P, _P],
        "br_attn_fwd_noalloc": [dims_p, _P, _P, _P, _I32P, _I32P, _P, _P, ctypes.c_float, _P],
        "br_attn_fwd_sink": [dims_p, _P, _P, _P, _I32P, _I32P, _P, _P, ctypes.c_float, ctypes.c_float, _P,
                             ctypes.c_size_t, _P],
        "br_attn_fwd_rope_workspace_bytes": [dims_p, _I32P, _I32P, ctypes.c_int32, ctypes.c_int32, sz_p],
        "br_attn_fwd_rope": [dims_p, _P, _P, _P, _I32P, _I32P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                             ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P],
        "br_doc_scores_workspace_bytes": [dims_p, ctypes.c_int32, _I32P, _I32P, sz_p],
        "br_doc_scores": [dims_p, _P, ctypes.c_int32, _P, _I32P, _I32P, _P, _P, ctypes.c_float, _P,
                          ctypes.c_size_t, _P],
        "br_sort_docs": [_P, _I32P, ctypes.c_int32, _P, _P],
        "br_rank_workspace_bytes": [dims_p, _I32P, _I32P, ctypes.c_int32, _I32P, _I32P, sz_p],
        "br_rank_prompts": [dims_p, _P, _P, _P, _P, ctypes.c_int32, _I32P, _I32P, _I32P, _I32P, _P, _P, _P, _P, _P,
                            ctypes.c_float, _P, ctypes.c_size_t, _P],
        "br_rank_prompts_timed": [dims_p, _P, _P, _P, _P, ctypes.c_int32, _I32P, _I32P, _I32P, _I32P, _P, _P, _P, _P,
                                  _P, ctypes.c_float, _P, ctypes.c_size_t, _P, _P, _P],
        "br_attn_plan_items": [dims_p, _I32P, _I32P, _I32P, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
                               ctypes.POINTER(ctypes.c_int32)],
        "br_attn_routed_workspace_bytes": [dims_p, _I32P, _I32P, _I32P, _I32P, ctypes.POINTER(ctypes.c_size_t)],
        "br_attn_routed_fwd": [dims_p, _P, _P, _P, _I32P, _I32P, _I32P, _I32P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t,
                               _P],
        "br_query_attn_workspace_bytes": [dims_p, ctypes.c_int32, _I32P, ctypes.POINTER(ctypes.c_size_t)],
        "br_query_attn_fwd": [dims_p, _P, _P, _P, ctypes.c_int32, _I32P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t, _P],
        "br_attn_bwd_workspace_bytes": [dims_p, _I32P, _I32P, sz_p],
        "br_attn_bwd": [dims_p, _P, _P, _P, _P, _P, _P, _I32P, _I32P, _P, _P, _P, ctypes.c_float, _P, ctypes.c_size_t,
                        _P],
        "br_attn_bwd_plan_items": [dims_p, _I32P, _I32P, _I32P, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
                                   ctypes.POINTER(ctypes.c_int32)],
        "br_infonce_workspace_bytes": [ctypes.c_int32, sz_p],
        "br_infonce": [_P, _I32P, ctypes.c_int32, _I32P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P],
        "br_doc_scores_bwd_workspace_bytes": [dims_p, ctypes.c_int32, _I32P, _I32P, sz_p],
        "br_doc_scores_bwd": [dims_p, _P, ctypes.c_int32, _P, _I32P, _I32P, _P, _P, _P, ctypes.c_int32, ctypes.c_float,
                              _P, ctypes.c_size_t, _P],
        "br_ssmax_softmax_scale": [ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_float)],
        "br_rope_workspace_bytes": [dims_p, _I32P, sz_p],
        "br_rope_fwd": [dims_p, _P, _P, _P, _P, _I32P, _I32P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                        ctypes.c_int32, _P, ctypes.c_size_t, _P],
        "br_rope_signal_fwd": [dims_p, _P, _P, ctypes.c_int32, _I32P, _I32P, ctypes.c_float, ctypes.c_int32,
                               ctypes.c_int32, _P, ctypes.c_size_t, _P],
        "br_rope_positions": [dims_p, _I32P, _I32P, ctypes.c_int32, ctypes.c_int32, _I32P, ctypes.c_int64],
        "br_attn_plan_schedule": [dims_p, _I32P, _I32P, ctypes.c_int32, _I32P, ctypes.c_int64, _I32P, ctypes.c_int64,
                                  ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.br_status_string.argtypes = [ctypes.c_int]
    lib.br_status_string.restype = ctypes.c_char_p
    lib.br_last_error.argtypes = []
    lib.br_last_error.restype = ctypes.c_char_p
    lib.br_version.argtypes = []
    lib.br_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load_library().br_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another failure
        return f"status {status}"


def _check(status: int) -> None:
    if status != BR_OK:
        raise BlockRankError(status, load_library().br_last_error().decode())


def _host_i32(a) -> np.ndarray:
    arr = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    return arr


def _ptr_i32(arr: np.ndarray):
    return arr.ctypes.data_as(_I32P)


def make_dims(num_prompts: int, num_q_heads: int, num_kv_heads: int, head_dim: int, total_tokens: int) -> BrDims:
    return BrDims(int(num_prompts), int(num_q_heads), int(num_kv_heads), int(head_dim), int(total_tokens))


def _dev_ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on_stream(fn):
    """Run ``fn`` with its ``stream`` argument (when given) as torch's current stream, so that the
    outputs, workspaces and zero fills it allocates belong to, and are ordered on, the stream its
    kernels run on: torch's caching allocator then reuses a freed workspace only for later work on
    that same stream."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        import torch
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    wrapper.runs_on_its_stream = True
    return wrapper


def attn_workspace_bytes(dims: BrDims, segment_offsets, seg_ptr) -> int:
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_attn_workspace_bytes(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), ctypes.byref(out)))
    return int(out.value)


def attn_plan_items(dims: BrDims, segment_offsets, seg_ptr) -> Tuple[np.ndarray, int]:
    """Host-only: the attention work list, [n, 8] int32, and the token rows per tile."""
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    n = ctypes.c_int64(0)
    tm = ctypes.c_int32(0)
    _check(lib.br_attn_plan_items(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), None, 0, ctypes.byref(n),
                                  ctypes.byref(tm)))
    items = np.zeros((max(int(n.value), 1), 8), dtype=np.int32)
    _check(lib.br_attn_plan_items(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), _ptr_i32(items), int(n.value),
                                  ctypes.byref(n), ctypes.byref(tm)))
    return items[:int(n.value)], int(tm.value)


def attn_plan_schedule(dims: BrDims, segment_offsets, seg_ptr, workgroups: int) -> Tuple[np.ndarray, np.ndarray]:
    """Host-only: the persistent schedule for `workgroups` slots: items [n, 8] int32 in run
    order and ranges [wg_per_head + 1] (workgroup w of a KV head runs items ranges[w]..ranges[w+1])."""
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    n, wph = ctypes.c_int64(0), ctypes.c_int32(0)
    _check(lib.br_attn_plan_schedule(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), int(workgroups), None, 0, None, 0,
                                     ctypes.byref(n), ctypes.byref(wph)))
    items = np.zeros((max(int(n.value), 1), 8), dtype=np.int32)
    ranges = np.zeros(int(wph.value) + 1, dtype=np.int32)
    _check(lib.br_attn_plan_schedule(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), int(workgroups), _ptr_i32(items),
                                     int(n.value), _ptr_i32(ranges), ranges.size, ctypes.byref(n), ctypes.byref(wph)))
    return items[:int(n.value)], ranges


@_on_stream
def attn_fwd(Q, K, V, segment_offsets, seg_ptr, out=None, lse=None, softmax_scale: float = 0.0,
             workspace=None, stream=None, kernel_events=None):
    """Block-sparse prefill attention.  Q [T,Hq,d], K/V [T,Hkv,d] bf16 CUDA tensors.

    Returns out (bf16 [T,Hq,d]); when ``lse`` is True a new fp32 [T,Hq] tensor is also
    returned (or pass a preallocated tensor).  ``kernel_events`` = (start, stop) raw hipEvent_t
    handles recorded around the attention kernel itself.
    """
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 CUDA tensor")
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape:
        raise ValueError("K and V must be [T, Hkv, d] matching Q")
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    if out is None:
        out = torch.empty_like(Q)
    want_lse = lse is True
    if want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=Q.device)
    elif lse is False:
        lse = None
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(attn_workspace_bytes(dims, so, sp), dtype=torch.uint8, device=Q.device)
    ev0, ev1 = kernel_events if kernel_events is not None else (None, None)
    _check(lib.br_attn_fwd_timed(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr_i32(so),
                                 _ptr_i32(sp), out.data_ptr(), _dev_ptr(lse), float(softmax_scale),
                                 workspace.data_ptr(), workspace.numel(), _stream_handle(stream), ev0, ev1))
    return (out, lse) if lse is not None else out


@_on_stream
def attn_fwd_sink(Q, K, V, segment_offsets, seg_ptr, sink: float, out=None, lse=None, softmax_scale: float = 0.0,
                  workspace=None, stream=None):
    """Block-sparse attention with the additive sink exp(sink) appended to every row's softmax
    denominator (output scaled by sigma(lse - sink)); arguments and results as for attn_fwd."""
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 CUDA tensor")
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape:
        raise ValueError("K and V must be [T, Hkv, d] matching Q")
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    out = torch.empty_like(Q) if out is None else out
    if lse is True:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=Q.device)
    elif lse is False:
        lse = None
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(dims, so, sp), dtype=torch.uint8, device=Q.device)
    _check(lib.br_attn_fwd_sink(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr_i32(so),
                                _ptr_i32(sp), out.data_ptr(), _dev_ptr(lse), float(softmax_scale), float(sink),
                                workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return (out, lse) if lse is not None else out


def attn_fwd_rope_workspace_bytes(dims: BrDims, segment_offsets, seg_ptr, query_pos0: int = 8192,
                                  docs_after_instruction: bool = True) -> int:
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_attn_fwd_rope_workspace_bytes(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), int(query_pos0),
                                                int(bool(docs_after_instruction)), ctypes.byref(out)))
    return out.value


@_on_stream
def attn_fwd_rope(Q, K, V, segment_offsets, seg_ptr, rope_theta: float = 10000.0, query_pos0: int = 8192,
                  docs_after_instruction: bool = True, interleaved: bool = False, out=None, lse=None,
                  softmax_scale: float = 0.0, workspace=None, stream=None):
    """Attention with Q rotated inside the kernel (K already rotated, e.g. rope(None, K, ...));
    results equal rope on Q followed by attn_fwd."""
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(name, t, 3)
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape:
        raise ValueError("K and V must be [T, Hkv, d] matching Q")
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    out = torch.empty_like(Q) if out is None else out
    if lse is True:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=Q.device)
    elif lse is False:
        lse = None
    if workspace is None:
        workspace = torch.empty(attn_fwd_rope_workspace_bytes(dims, so, sp, query_pos0, docs_after_instruction),
                                dtype=torch.uint8, device=Q.device)
    _check(lib.br_attn_fwd_rope(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr_i32(so),
                                _ptr_i32(sp), out.data_ptr(), _dev_ptr(lse), float(softmax_scale), float(rope_theta),
                                int(query_pos0), int(bool(docs_after_instruction)), int(bool(interleaved)),
                                workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return (out, lse) if lse is not None else out


NOALLOC_SCRATCH_BYTES = 32 << 20  # BR_NOALLOC_SCRATCH_BYTES in include/blockrank.h


@_on_stream
def attn_fwd_noalloc(Q, K, V, segment_offsets, seg_ptr, out, lse=None, softmax_scale: float = 0.0, stream=None):
    """br_attn_fwd_noalloc: the attention with the library's own per-GPU workspace; the caller
    passes every output (``out`` bf16 [T,Hq,d], optional ``lse`` fp32 [T,Hq]) and this wrapper
    allocates nothing.  Calls that overlap on one GPU race (one shared workspace)."""
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V), ("out", out)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 CUDA tensor")
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape or out.shape != Q.shape:
        raise ValueError("K and V must be [T, Hkv, d] and out [T, Hq, d], matching Q")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous()
                            or tuple(lse.shape) != (T, Hq)):
        raise ValueError("lse must be a contiguous float32 CUDA tensor [T, Hq]")
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    _check(lib.br_attn_fwd_noalloc(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr_i32(so),
                                   _ptr_i32(sp), out.data_ptr(), _dev_ptr(lse), float(softmax_scale),
                                   _stream_handle(stream)))
    return out


def attn_routed_workspace_bytes(dims: BrDims, segment_offsets, seg_ptr, keep_ptr, keep) -> int:
    lib = load_library()
    so, sp, kp, kk = _host_i32(segment_offsets), _host_i32(seg_ptr), _host_i32(keep_ptr), _host_i32(keep)
    out = ctypes.c_size_t(0)
    _check(lib.br_attn_routed_workspace_bytes(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), _ptr_i32(kp),
                                              _ptr_i32(kk), ctypes.byref(out)))
    return int(out.value)


@_on_stream
def attn_routed(Q, K, V, segment_offsets, seg_ptr, keep_ptr, keep, out=None, lse=None, softmax_scale: float = 0.0,
                workspace=None, stream=None):
    """Top-B routed attention: prompt b keeps documents keep[keep_ptr[b]:keep_ptr[b+1]] (local
    indices); dropped documents' rows are not computed (out rows left as they were) and the final
    query reads only the instruction and the kept documents.  Shapes as attn_fwd."""
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 CUDA tensor")
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape:
        raise ValueError("K and V must be [T, Hkv, d] matching Q")
    so, sp, kp, kk = _host_i32(segment_offsets), _host_i32(seg_ptr), _host_i32(keep_ptr), _host_i32(keep)
    if kk.size == 0:
        kk = np.zeros(1, dtype=np.int32)  # a valid pointer; keep_ptr says no document is kept
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    if out is None:
        out = torch.zeros_like(Q)
    if lse is True:
        lse = torch.zeros((T, Hq), dtype=torch.float32, device=Q.device)
    elif lse is False:
        lse = None
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(attn_routed_workspace_bytes(dims, so, sp, kp, kk), dtype=torch.uint8, device=Q.device)
    _check(lib.br_attn_routed_fwd(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr_i32(so),
                                  _ptr_i32(sp), _ptr_i32(kp), _ptr_i32(kk), out.data_ptr(), _dev_ptr(lse),
                                  float(softmax_scale), workspace.data_ptr(), workspace.numel(),
                                  _stream_handle(stream)))
    return (out, lse) if lse is not None else out


def attn_bwd_workspace_bytes(dims: BrDims, segment_offsets, seg_ptr) -> int:
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_attn_bwd_workspace_bytes(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), ctypes.byref(out)))
    return int(out.value)


def attn_bwd_plan_items(dims: BrDims, segment_offsets, seg_ptr):
    """Host-only: the backward's key-major items ([n, 8] int32) and the number of partial slots."""
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    n, slots = ctypes.c_int64(0), ctypes.c_int32(0)
    _check(lib.br_attn_bwd_plan_items(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), None, 0, ctypes.byref(n),
                                      ctypes.byref(slots)))
    items = np.zeros((max(1, n.value), 8), dtype=np.int32)
    _check(lib.br_attn_bwd_plan_items(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), _ptr_i32(items), n.value,
                                      ctypes.byref(n), ctypes.byref(slots)))
    return items[:n.value], int(slots.value)


@_on_stream
def attn_bwd(Q, K, V, O, dO, lse, segment_offsets, seg_ptr, softmax_scale: float = 0.0, dQ=None, dK=None, dV=None,
             workspace=None, stream=None):
    """Gradients (dQ [T,Hq,d], dK, dV [T,Hkv,d], fp32) of the block-sparse attention for the upstream
    gradient dO, given the forward's output O and log-sum-exp lse [T,Hq] (same softmax_scale)."""
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O), ("dO", dO)):
        _check_bf16(name, t, 3)
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape or O.shape != Q.shape or dO.shape != Q.shape:
        raise ValueError("shapes: Q, O, dO [T, Hq, d]; K, V [T, Hkv, d]")
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() or tuple(lse.shape) != (T, Hq):
        raise ValueError("lse must be a contiguous float32 CUDA tensor [T, Hq]")
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    f32 = dict(dtype=torch.float32, device=Q.device)
    dQ = torch.empty((T, Hq, d), **f32) if dQ is None else dQ
    dK = torch.empty((T, Hkv, d), **f32) if dK is None else dK
    dV = torch.empty((T, Hkv, d), **f32) if dV is None else dV
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(attn_bwd_workspace_bytes(dims, so, sp), dtype=torch.uint8, device=Q.device)
    _check(lib.br_attn_bwd(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), dO.data_ptr(),
                           lse.data_ptr(), _ptr_i32(so), _ptr_i32(sp), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(),
                           float(softmax_scale), workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return dQ, dK, dV


@_on_stream
def infonce(scores, doc_ptr, gold, tau: float = 0.05, loss=None, dscores=None, workspace=None, stream=None):
    """Per-prompt InfoNCE loss [B] and its gradient with respect to the scores [sum N_b] (fp32)."""
    import torch
    lib = load_library()
    if scores.dtype != torch.float32 or not scores.is_cuda or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 CUDA tensor")
    dp, gd = _host_i32(doc_ptr), _host_i32(gold)
    B = len(dp) - 1
    if len(gd) != B:
        raise ValueError("gold must have one entry per prompt")
    loss = torch.empty(B, dtype=torch.float32, device=scores.device) if loss is None else loss
    dscores = torch.empty_like(scores) if dscores is None else dscores
    if workspace is None:  # a caller's workspace is checked by the library
        out = ctypes.c_size_t(0)
        _check(lib.br_infonce_workspace_bytes(B, ctypes.byref(out)))
        workspace = torch.empty(out.value, dtype=torch.uint8, device=scores.device)
    _check(lib.br_infonce(scores.data_ptr(), _ptr_i32(dp), B, _ptr_i32(gd), float(tau), loss.data_ptr(),
                          dscores.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return loss, dscores


def doc_scores_bwd_workspace_bytes(dims: BrDims, n_signal: int, doc_offsets, doc_ptr) -> int:
    lib = load_library()
    do, dp = _host_i32(doc_offsets), _host_i32(doc_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_doc_scores_bwd_workspace_bytes(ctypes.byref(dims), int(n_signal), _ptr_i32(do), _ptr_i32(dp),
                                                 ctypes.byref(out)))
    return int(out.value)


@_on_stream
def doc_scores_bwd(Q_S, K, doc_offsets, doc_ptr, dscores, softmax_scale: float = 0.0, dQ_S=None, dK=None,
                   accumulate: bool = False, workspace=None, stream=None):
    """Gradient of sum_k dscores_k s_k through the readout: dQ_S [B,S,Hq,d] and dK [T,Hkv,d] (fp32).
    dK rows of document tokens are written (or added to with accumulate=True); a new dK is zeroed."""
    import torch
    lib = load_library()
    _check_bf16("Q_S", Q_S, 4)
    _check_bf16("K", K, 3)
    if dscores.dtype != torch.float32 or not dscores.is_cuda or not dscores.is_contiguous():
        raise ValueError("dscores must be a contiguous float32 CUDA tensor")
    B, S, Hq, d = Q_S.shape
    T, Hkv, _ = K.shape
    do, dp = _host_i32(doc_offsets), _host_i32(doc_ptr)
    dims = make_dims(B, Hq, Hkv, d, T)
    dQ_S = torch.empty((B, S, Hq, d), dtype=torch.float32, device=K.device) if dQ_S is None else dQ_S
    dK = torch.zeros((T, Hkv, d), dtype=torch.float32, device=K.device) if dK is None else dK
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(doc_scores_bwd_workspace_bytes(dims, S, do, dp), dtype=torch.uint8, device=K.device)
    _check(lib.br_doc_scores_bwd(ctypes.byref(dims), Q_S.data_ptr(), int(S), K.data_ptr(), _ptr_i32(do), _ptr_i32(dp),
                                 dscores.data_ptr(), dQ_S.data_ptr(), dK.data_ptr(), int(bool(accumulate)),
                                 float(softmax_scale), workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return dQ_S, dK


def ssmax_scale(s: float, n_docs: int, head_dim: int) -> float:
    """SSMax softmax_scale for a prompt of n_docs documents: s * ln(n_docs) / sqrt(head_dim)."""
    lib = load_library()
    out = ctypes.c_float(0.0)
    _check(lib.br_ssmax_softmax_scale(float(s), int(n_docs), int(head_dim), ctypes.byref(out)))
    return float(out.value)


def rope_workspace_bytes(dims: BrDims, seg_ptr) -> int:
    lib = load_library()
    sp = _host_i32(seg_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_rope_workspace_bytes(ctypes.byref(dims), _ptr_i32(sp), ctypes.byref(out)))
    return int(out.value)


def rope_positions(dims: BrDims, segment_offsets, seg_ptr, query_pos0: int = 8192,
                   docs_after_instruction: bool = True) -> np.ndarray:
    """Host-side position ids of every token (int32 [total_tokens])."""
    lib = load_library()
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    pos = np.zeros(int(dims.total_tokens), dtype=np.int32)
    _check(lib.br_rope_positions(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), int(query_pos0),
                                 int(bool(docs_after_instruction)), _ptr_i32(pos), pos.size))
    return pos


def _check_bf16(name, t, ndim):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != ndim:
        raise ValueError(f"{name} must be a contiguous {ndim}-D bfloat16 CUDA tensor")


@_on_stream
def rope(Q, K, segment_offsets, seg_ptr, rope_theta: float = 10000.0, query_pos0: int = 8192,
         docs_after_instruction: bool = True, interleaved: bool = False, Q_out=None, K_out=None,
         inplace: bool = False, workspace=None, stream=None):
    """Rotary embedding of Q [T, Hq, d] and K [T, Hkv, d] (either may be None) at the prompts'
    permutation-invariant positions.  Returns (Q_out, K_out); in place when inplace=True."""
    import torch
    lib = load_library()
    if Q is None and K is None:
        raise ValueError("nothing to rotate")
    if Q is not None:
        _check_bf16("Q", Q, 3)
    if K is not None:
        _check_bf16("K", K, 3)
    ref = Q if Q is not None else K
    T, d = ref.shape[0], ref.shape[2]
    Hq = Q.shape[1] if Q is not None else K.shape[1]
    Hkv = K.shape[1] if K is not None else Hq
    if Q is not None and K is not None and (K.shape[0] != T or K.shape[2] != d):
        raise ValueError("Q and K must share T and d")
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    dims = make_dims(len(sp) - 1, Hq, Hkv, d, T)
    if Q is not None and Q_out is None:
        Q_out = Q if inplace else torch.empty_like(Q)
    if K is not None and K_out is None:
        K_out = K if inplace else torch.empty_like(K)
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(rope_workspace_bytes(dims, sp), dtype=torch.uint8, device=ref.device)
    _check(lib.br_rope_fwd(ctypes.byref(dims), _dev_ptr(Q), _dev_ptr(K), _dev_ptr(Q_out), _dev_ptr(K_out),
                           _ptr_i32(so), _ptr_i32(sp), float(rope_theta), int(query_pos0),
                           int(bool(docs_after_instruction)), int(bool(interleaved)), workspace.data_ptr(),
                           workspace.numel(), _stream_handle(stream)))
    return Q_out, K_out


@_on_stream
def rope_signal(Q_S, segment_offsets, seg_ptr, rope_theta: float = 10000.0, query_pos0: int = 8192,
                interleaved: bool = False, out=None, inplace: bool = False, num_kv_heads: Optional[int] = None,
                workspace=None, stream=None):
    """Rotary embedding of the signal rows Q_S [B, S, Hq, d] at the positions of each prompt's last
    S query tokens."""
    import torch
    lib = load_library()
    _check_bf16("Q_S", Q_S, 4)
    B, S, Hq, d = Q_S.shape
    so, sp = _host_i32(segment_offsets), _host_i32(seg_ptr)
    if len(sp) != B + 1:
        raise ValueError("seg_ptr must have B + 1 entries")
    dims = make_dims(B, Hq, num_kv_heads or Hq, d, int(so[sp[-1] - 1]))
    if out is None:
        out = Q_S if inplace else torch.empty_like(Q_S)
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(rope_workspace_bytes(dims, sp), dtype=torch.uint8, device=Q_S.device)
    _check(lib.br_rope_signal_fwd(ctypes.byref(dims), Q_S.data_ptr(), out.data_ptr(), int(S), _ptr_i32(so),
                                  _ptr_i32(sp), float(rope_theta), int(query_pos0), int(bool(interleaved)),
                                  workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return out


def query_attn_workspace_bytes(dims: BrDims, corpus_len: int, query_offsets) -> int:
    lib = load_library()
    qo = _host_i32(query_offsets)
    out = ctypes.c_size_t(0)
    _check(lib.br_query_attn_workspace_bytes(ctypes.byref(dims), int(corpus_len), _ptr_i32(qo), ctypes.byref(out)))
    return int(out.value)


@_on_stream
def query_attn(Q, K, V, corpus_len: int, query_offsets, out=None, lse=None, softmax_scale: float = 0.0,
               workspace=None, stream=None):
    """Query-only attention over a cached corpus.  K/V [T,Hkv,d] hold the corpus [0, corpus_len)
    then the queries' own tokens; Q and out are [T - corpus_len, Hq, d] (query rows only).
    Query b owns tokens query_offsets[b] .. query_offsets[b+1] and reads the whole corpus plus
    its own tokens causally.  ``lse`` as in attn_fwd."""
    import torch
    lib = load_library()
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 CUDA tensor")
    Tq, Hq, d = Q.shape
    T, Hkv = K.shape[0], K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape or Tq != T - int(corpus_len):
        raise ValueError("K and V must be [T, Hkv, d] and Q [T - corpus_len, Hq, d]")
    qo = _host_i32(query_offsets)
    dims = make_dims(len(qo) - 1, Hq, Hkv, d, T)
    if out is None:
        out = torch.empty_like(Q)
    if lse is True:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=Q.device)
    elif lse is False:
        lse = None
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(query_attn_workspace_bytes(dims, corpus_len, qo), dtype=torch.uint8, device=Q.device)
    _check(lib.br_query_attn_fwd(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), int(corpus_len),
                                 _ptr_i32(qo), out.data_ptr(), _dev_ptr(lse), float(softmax_scale),
                                 workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return (out, lse) if lse is not None else out


def doc_scores_workspace_bytes(dims: BrDims, n_signal: int, doc_offsets, doc_ptr) -> int:
    lib = load_library()
    do, dp = _host_i32(doc_offsets), _host_i32(doc_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_doc_scores_workspace_bytes(ctypes.byref(dims), int(n_signal), _ptr_i32(do), _ptr_i32(dp),
                                             ctypes.byref(out)))
    return int(out.value)


@_on_stream
def doc_scores(Q_S, K, doc_offsets, doc_ptr, head_scores: bool = False, softmax_scale: float = 0.0,
               scores=None, workspace=None, stream=None):
    """Attention-mass scores.  Q_S [B,S,Hq,d], K [T,Hkv,d] bf16 CUDA tensors.

    Returns scores fp32 [sum N_b] (and head_scores [Hq, sum N_b] if requested)."""
    import torch
    lib = load_library()
    for name, t in (("Q_S", Q_S), ("K", K)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    if Q_S.dim() != 4 or K.dim() != 3 or Q_S.shape[3] != K.shape[2]:
        raise ValueError("Q_S must be [B, S, Hq, d] and K [T, Hkv, d]")
    B, S, Hq, d = Q_S.shape
    T, Hkv, _ = K.shape
    do, dp = _host_i32(doc_offsets), _host_i32(doc_ptr)
    if len(dp) != B + 1:
        raise ValueError("doc_ptr must have B + 1 entries")
    dims = make_dims(B, Hq, Hkv, d, T)
    n_docs = int(dp[-1]) - B
    if scores is None:
        scores = torch.empty(n_docs, dtype=torch.float32, device=K.device)
    hs = torch.empty((Hq, n_docs), dtype=torch.float32, device=K.device) if head_scores else None
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(doc_scores_workspace_bytes(dims, S, do, dp), dtype=torch.uint8, device=K.device)
    _check(lib.br_doc_scores(ctypes.byref(dims), Q_S.data_ptr(), int(S), K.data_ptr(), _ptr_i32(do), _ptr_i32(dp),
                             scores.data_ptr(), _dev_ptr(hs), float(softmax_scale), workspace.data_ptr(),
                             workspace.numel(), _stream_handle(stream)))
    return (scores, hs) if head_scores else scores


@_on_stream
def sort_docs(scores, doc_ptr, order=None, stream=None):
    """Per-prompt local document indices by descending score (ties: lower index)."""
    import torch
    lib = load_library()
    if scores.dtype != torch.float32 or not scores.is_cuda or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous float32 CUDA tensor")
    dp = _host_i32(doc_ptr)
    if order is None:
        order = torch.empty(scores.numel(), dtype=torch.int32, device=scores.device)
    _check(lib.br_sort_docs(scores.data_ptr(), _ptr_i32(dp), len(dp) - 1, order.data_ptr(),
                            _stream_handle(stream)))
    return order


def rank_workspace_bytes(dims: BrDims, segment_offsets, seg_ptr, n_signal: int, doc_offsets, doc_ptr) -> int:
    lib = load_library()
    so, sp, do, dp = _host_i32(segment_offsets), _host_i32(seg_ptr), _host_i32(doc_offsets), _host_i32(doc_ptr)
    out = ctypes.c_size_t(0)
    _check(lib.br_rank_workspace_bytes(ctypes.byref(dims), _ptr_i32(so), _ptr_i32(sp), int(n_signal), _ptr_i32(do),
                                       _ptr_i32(dp), ctypes.byref(out)))
    return int(out.value)


@_on_stream
def rank_step(Q, K, V, Q_S, segment_offsets, seg_ptr, doc_offsets, doc_ptr, softmax_scale: float = 0.0, out=None,
              lse=None, scores=None, head_scores=None, order=None, workspace=None, stream=None, kernel_events=None):
    """The whole hot path in one library call (br_rank_prompts): attention output, document scores
    and per-prompt order, bit-identical to attn_fwd + doc_scores + sort_docs."""
    import torch
    lib = load_library()
    for name, t, nd in (("Q", Q, 3), ("K", K, 3), ("V", V, 3), ("Q_S", Q_S, 4)):
        _check_bf16(name, t, nd)
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (T, Hkv, d) or V.shape != K.shape or Q_S.shape[2:] != (Hq, d):
        raise ValueError("shapes: Q [T,Hq,d], K/V [T,Hkv,d], Q_S [B,S,Hq,d]")
    so, sp, do, dp = _host_i32(segment_offsets), _host_i32(seg_ptr), _host_i32(doc_offsets), _host_i32(doc_ptr)
    B, S = Q_S.shape[0], Q_S.shape[1]
    dims = make_dims(B, Hq, Hkv, d, T)
    n_docs = int(dp[-1]) - B
    out = torch.empty_like(Q) if out is None else out
    if lse is True:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=Q.device)
    elif lse is False:
        lse = None
    scores = torch.empty(n_docs, dtype=torch.float32, device=Q.device) if scores is None else scores
    order = torch.empty(n_docs, dtype=torch.int32, device=Q.device) if order is None else order
    if workspace is None:  # a caller's workspace is checked by the library
        workspace = torch.empty(rank_workspace_bytes(dims, so, sp, S, do, dp), dtype=torch.uint8, device=Q.device)
    ev0, ev1 = kernel_events if kernel_events is not None else (None, None)
    _check(lib.br_rank_prompts_timed(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), Q_S.data_ptr(), int(S),
                                     _ptr_i32(so), _ptr_i32(sp), _ptr_i32(do), _ptr_i32(dp), out.data_ptr(),
                                     _dev_ptr(lse), scores.data_ptr(), _dev_ptr(head_scores), order.data_ptr(),
                                     float(softmax_scale), workspace.data_ptr(), workspace.numel(),
                                     _stream_handle(stream), ev0, ev1))
    return out, scores, order


def version() -> str:
    return load_library().br_version().decode()
