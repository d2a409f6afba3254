"""Thin ctypes binding of libsinkattn (include/sinkattn.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their ``data_ptr()`` and torch's current HIP stream are passed to
the C entry points, and a non-OK status raises ``SinkAttnError``.  All
attention arithmetic runs in the library's HIP kernels; there is no fallback
path.  torch supplies device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

HEAD_DIM = 64
PAGE_SIZE = 16
MAX_SPLITS = 256
MAX_DECODE_ROWS = 8
MAX_EXPERTS = 512
MAX_TOP_K = 8
MAX_BALANCED_BATCH = 256
NOALLOC_SCRATCH_BYTES = 8 << 20
EXPORTED = (
    "sinkattn_prefill",
    "sinkattn_decode_paged",
    "sinkattn_decode_paged_noalloc",
    "sinkattn_decode_paged_balanced",
    "sinkattn_decode_paged_balanced_pieces",
    "sinkattn_merge_balanced",
    "sinkattn_decode_balanced_workspace_bytes",
    "sinkattn_pick_num_segments",
    "sinkattn_balanced_segments",
    "sinkattn_decode_paged_multi",
    "sinkattn_append_paged_kv_rope",
    "sinkattn_moe_topk_softmax",
    "sinkattn_merge",
    "sinkattn_split_bounds",
    "sinkattn_pick_num_splits",
    "sinkattn_pick_num_splits_multi",
    "sinkattn_validate_kv_host",
    "sinkattn_status_string",
    "sinkattn_last_error",
    "sinkattn_last_hip_error",
    "sinkattn_abi_version",
)


class SinkAttnError(RuntimeError):
    """A libsinkattn call returned a non-OK status (or the library is missing)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libsinkattn status {status}: {message}")
        self.status = status


class _KV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("paged", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("kv_indptr", ctypes.c_void_p),
        ("page_indices", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("kv_len_host", ctypes.c_void_p),
    ]


def library_path() -> str:
    return os.environ.get("SINKATTN_LIB", os.path.join(_HERE, "libsinkattn.so"))


def load_library():
    """Load libsinkattn.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise SinkAttnError(-1, f"{path} is missing: build it with "
                                "`python -m gqa_attention_sinks_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.sinkattn_prefill.argtypes = [vp, vp, ctypes.POINTER(_KV), vp, vp, vp, i32, i32, i32, i32, i32,
                                     f32, i32, vp, vp]
    lib.sinkattn_prefill.restype = i32
    lib.sinkattn_decode_paged.argtypes = [vp, ctypes.POINTER(_KV), vp, i32, vp, vp, vp, vp, i32, i32,
                                          i32, i32, f32, i32, vp]
    lib.sinkattn_decode_paged.restype = i32
    lib.sinkattn_decode_paged_noalloc.argtypes = [vp, ctypes.POINTER(_KV), vp, i32, vp, vp, i32, i32, i32, i32,
                                                  f32, i32, vp]
    lib.sinkattn_decode_paged_noalloc.restype = i32
    lib.sinkattn_decode_paged_balanced.argtypes = [vp, ctypes.POINTER(_KV), vp, i32, vp, ctypes.c_int64, vp, vp,
                                                   i32, i32, i32, i32, f32, i32, vp]
    lib.sinkattn_decode_paged_balanced.restype = i32
    lib.sinkattn_decode_paged_balanced_pieces.argtypes = lib.sinkattn_decode_paged_balanced.argtypes
    lib.sinkattn_decode_paged_balanced_pieces.restype = i32
    lib.sinkattn_merge_balanced.argtypes = [vp, i32, vp, ctypes.c_int64, vp, vp, i32, i32, i32, vp]
    lib.sinkattn_merge_balanced.restype = i32
    lib.sinkattn_decode_balanced_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sinkattn_decode_balanced_workspace_bytes.restype = ctypes.c_int64
    lib.sinkattn_pick_num_segments.argtypes = [i32]
    lib.sinkattn_pick_num_segments.restype = i32
    lib.sinkattn_balanced_segments.argtypes = [vp, i32, i32, i32, vp]
    lib.sinkattn_balanced_segments.restype = i32
    lib.sinkattn_decode_paged_multi.argtypes = [vp, vp, vp, vp, ctypes.POINTER(_KV), vp, i32, vp, vp, vp,
                                                vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.sinkattn_decode_paged_multi.restype = i32
    lib.sinkattn_append_paged_kv_rope.argtypes = [vp, vp, vp, vp, ctypes.POINTER(_KV), vp, i32, i32, vp, i32,
                                                  i32, i32, i32, i32, vp]
    lib.sinkattn_append_paged_kv_rope.restype = i32
    lib.sinkattn_moe_topk_softmax.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.sinkattn_moe_topk_softmax.restype = i32
    lib.sinkattn_merge.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.sinkattn_merge.restype = i32
    lib.sinkattn_split_bounds.argtypes = [vp, i32, i32, i32, vp]
    lib.sinkattn_split_bounds.restype = i32
    lib.sinkattn_pick_num_splits.argtypes = [vp, i32, i32]
    lib.sinkattn_pick_num_splits.restype = i32
    lib.sinkattn_pick_num_splits_multi.argtypes = [vp, i32, i32, i32, i32, i32]
    lib.sinkattn_pick_num_splits_multi.restype = i32
    lib.sinkattn_validate_kv_host.argtypes = [ctypes.POINTER(_KV), vp, vp, vp, i32]
    lib.sinkattn_validate_kv_host.restype = i32
    lib.sinkattn_status_string.argtypes = [i32]
    lib.sinkattn_status_string.restype = ctypes.c_char_p
    lib.sinkattn_last_error.argtypes = []
    lib.sinkattn_last_error.restype = ctypes.c_char_p
    lib.sinkattn_last_hip_error.argtypes = []
    lib.sinkattn_last_hip_error.restype = ctypes.c_char_p
    lib.sinkattn_abi_version.argtypes = []
    lib.sinkattn_abi_version.restype = i32
    _LIB = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise SinkAttnError(status, lib.sinkattn_last_error().decode())


def abi_version() -> int:
    return load_library().sinkattn_abi_version()


# --------------------------------------------------------------------------
# tensor checks
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev(t, name, dtype, shape=None):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _kv_struct(k, v, kv_indptr, page_indices=None, kv_len=None, kv_len_host=None):
    torch = _torch()
    paged = page_indices is not None
    _dev(k, "k", torch.bfloat16)
    _dev(v, "v", torch.bfloat16)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    _dev(kv_indptr, "kv_indptr", torch.int32)
    if paged:
        if k.dim() != 4 or k.shape[2] != PAGE_SIZE or k.shape[3] != HEAD_DIM:
            raise ValueError("paged k/v must be [num_pages, Hkv, 16, 64]")
        _dev(page_indices, "page_indices", torch.int32)
        _dev(kv_len, "kv_len", torch.int32)
    elif k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("contiguous k/v must be [total_kv, Hkv, 64]")
    host = None
    if kv_len_host is not None:
        host = np.ascontiguousarray(kv_len_host, dtype=np.int32)
        if host.shape != (kv_indptr.numel() - 1,):
            raise ValueError("kv_len_host must have one entry per request")
    kvs = _KV(k.data_ptr(), v.data_ptr(), int(paged), PAGE_SIZE, kv_indptr.data_ptr(),
              page_indices.data_ptr() if paged else None, kv_len.data_ptr() if paged else None,
              int(k.shape[0]), None if host is None else host.ctypes.data)
    kvs._kv_len_host = host   # the struct points into it
    return kvs


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def prefill(q, qo_indptr, k, v, kv_indptr, sinks, sm_scale: float, window: int = 0,
            page_indices=None, kv_len=None, out=None, lse=None, return_lse: bool = False,
            qo_indptr_host=None, kv_len_host=None, stream=None):
    """Causal / sliding-window prefill (``sinkattn_prefill``).

    ``q`` [total_q, Hq, 64] bf16; ``qo_indptr`` [B+1] int32.  Contiguous KV:
    ``k``/``v`` [total_kv, Hkv, 64] with ``kv_indptr`` row offsets.  Paged KV:
    ``k``/``v`` [num_pages, Hkv, 16, 64] with ``kv_indptr`` page offsets,
    ``page_indices`` and ``kv_len``.  ``sinks`` [Hq] fp32 or None.
    ``qo_indptr_host``: optional host copy of ``qo_indptr`` (numpy/list) that
    lets the library size the launch exactly.  ``kv_len_host``: optional host
    copy of ``kv_len`` (paged) that orders the one-row requests' work on the
    host; it never changes the results.
    Returns ``out`` (and ``lse`` [total_q, Hq] fp32 when asked).
    """
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [total_q, Hq, 64]")
    total_q, hq, _ = q.shape
    _dev(qo_indptr, "qo_indptr", torch.int32)
    batch = qo_indptr.numel() - 1
    kvs = _kv_struct(k, v, kv_indptr, page_indices, kv_len, kv_len_host)
    hkv = k.shape[1]
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32, (hq,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (total_q, hq))
    host = None
    if qo_indptr_host is not None:
        host = np.ascontiguousarray(qo_indptr_host, dtype=np.int32)
        if host.shape != (batch + 1,):
            raise ValueError("qo_indptr_host must have batch + 1 entries")
    lib = load_library()
    _check(lib.sinkattn_prefill(_ptr(q), _ptr(qo_indptr), ctypes.byref(kvs), _ptr(sinks), _ptr(out),
                                _ptr(lse), batch, total_q, hq, hkv, HEAD_DIM, float(sm_scale),
                                int(window),
                                None if host is None else host.ctypes.data_as(ctypes.c_void_p),
                                _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_paged(q, k_pool, v_pool, page_indptr, page_indices, kv_len, sinks, sm_scale: float,
                 num_splits: int = 1, window: int = 0, out=None, o_part=None, lse_part=None,
                 lse=None, return_lse: bool = False, merge: bool = True, kv_len_host=None,
                 stream=None):
    """One query token per request over a paged cache (``sinkattn_decode_paged``).

    With ``num_splits`` > 1 the per-chunk partials ``o_part`` [B, Hq, S, 64]
    and ``lse_part`` [B, Hq, S] (allocated if not given) are written; with
    ``merge`` they are also merged into ``out`` in the same call.  Returns
    ``out`` (and ``lse``), or ``(o_part, lse_part)`` when ``merge`` is False.
    ``kv_len_host``: optional host copy of ``kv_len`` with which the library
    orders the work units (longest request first) on the host instead of in
    every workgroup; it never changes the results.
    """
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, Hq, 64]")
    batch, hq, _ = q.shape
    kvs = _kv_struct(k_pool, v_pool, page_indptr, page_indices, kv_len, kv_len_host)
    hkv = k_pool.shape[1]
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32, (hq,))
    s = int(num_splits)
    if s > 1:
        if o_part is None:
            o_part = torch.empty((batch, hq, s, HEAD_DIM), dtype=torch.float32, device=q.device)
        if lse_part is None:
            lse_part = torch.empty((batch, hq, s), dtype=torch.float32, device=q.device)
        _dev(o_part, "o_part", torch.float32, (batch, hq, s, HEAD_DIM))
        _dev(lse_part, "lse_part", torch.float32, (batch, hq, s))
    else:
        o_part = lse_part = None
    want_out = s == 1 or merge
    if want_out and out is None:
        out = torch.empty_like(q)
    if out is not None:
        _dev(out, "out", torch.bfloat16, q.shape)
    if want_out and return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, hq))
    lib = load_library()
    _check(lib.sinkattn_decode_paged(_ptr(q), ctypes.byref(kvs), _ptr(sinks), s,
                                     _ptr(out if want_out else None), _ptr(o_part), _ptr(lse_part),
                                     _ptr(lse if want_out else None), batch, hq, hkv, HEAD_DIM,
                                     float(sm_scale), int(window), _stream(stream)))
    if not want_out:
        return o_part, lse_part
    return (out, lse) if (return_lse or lse is not None) else out


def decode_paged_noalloc(q, k_pool, v_pool, page_indptr, page_indices, kv_len, sinks, sm_scale: float,
                         num_splits: int = 1, window: int = 0, out=None, lse=None, return_lse: bool = False,
                         kv_len_host=None, stream=None):
    """``sinkattn_decode_paged_noalloc``: like :func:`decode_paged` with the
    merge, the split partials in the library's own device array (nothing is
    allocated by the library; ``out`` and ``lse`` are allocated here when not
    given).  Returns ``out`` (and ``lse``)."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, Hq, 64]")
    batch, hq, _ = q.shape
    kvs = _kv_struct(k_pool, v_pool, page_indptr, page_indices, kv_len, kv_len_host)
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32, (hq,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, hq))
    lib = load_library()
    _check(lib.sinkattn_decode_paged_noalloc(_ptr(q), ctypes.byref(kvs), _ptr(sinks), int(num_splits), _ptr(out),
                                             _ptr(lse), batch, hq, k_pool.shape[1], HEAD_DIM, float(sm_scale),
                                             int(window), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_balanced_workspace_bytes(batch: int, num_qo_heads: int, num_segments: int) -> int:
    """Bytes of workspace :func:`decode_paged_balanced` needs."""
    n = int(load_library().sinkattn_decode_balanced_workspace_bytes(batch, num_qo_heads, num_segments))
    if n < 0:
        raise ValueError("batch, num_qo_heads and num_segments must be >= 1")
    return n


def pick_num_segments(num_kv_heads: int) -> int:
    """Host-only segment count that fills the current GPU in one launch round."""
    return int(load_library().sinkattn_pick_num_segments(int(num_kv_heads)))


def balanced_segments(kv_len_host, num_segments: int, window: int = 0) -> np.ndarray:
    """Host-only segment rule of the balanced decode: int32 [B, 2] first and
    last segment of each request (-1 for a request without keys)."""
    lens = np.ascontiguousarray(kv_len_host, dtype=np.int32)
    out = np.zeros((len(lens), 2), dtype=np.int32)
    _check(load_library().sinkattn_balanced_segments(lens.ctypes.data_as(ctypes.c_void_p), len(lens), int(window),
                                                     int(num_segments), out.ctypes.data_as(ctypes.c_void_p)))
    return out


def decode_paged_balanced(q, k_pool, v_pool, page_indptr, page_indices, kv_len, sinks, sm_scale: float,
                          num_segments: int = 0, window: int = 0, out=None, lse=None, workspace=None,
                          return_lse: bool = False, stream=None):
    """``sinkattn_decode_paged_balanced``: one query token per request, the
    batch's live pages cut into ``num_segments`` equal segments (0: the
    library's pick).  ``workspace`` (uint8 device tensor) is allocated here
    when not given.  Returns ``out`` (and ``lse``)."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, Hq, 64]")
    batch, hq, _ = q.shape
    kvs = _kv_struct(k_pool, v_pool, page_indptr, page_indices, kv_len)
    hkv = k_pool.shape[1]
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32, (hq,))
    n_seg = int(num_segments) if num_segments else pick_num_segments(hkv)
    need = decode_balanced_workspace_bytes(batch, hq, n_seg)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16, q.shape)
    if return_lse and lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (batch, hq))
    lib = load_library()
    _check(lib.sinkattn_decode_paged_balanced(_ptr(q), ctypes.byref(kvs), _ptr(sinks), n_seg, _ptr(workspace),
                                              workspace.numel(), _ptr(out), _ptr(lse), batch, hq, hkv, HEAD_DIM,
                                              float(sm_scale), int(window), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def balanced_workspace_views(workspace, batch: int, num_qo_heads: int, num_segments: int):
    """The documented parts of a balanced-decode workspace: (plan int32
    [B+1], lse fp32 [slots, Hq], o fp32 [slots, Hq, 64]), slots =
    num_segments + batch; the segment table int32 [B, 2] follows the plan
    (``balanced_workspace_segments``)."""
    slots = num_segments + batch
    plan_bytes = ((3 * batch + 1) * 4 + 255) // 256 * 256
    lse_bytes = (slots * num_qo_heads * 4 + 255) // 256 * 256
    plan = workspace[:(batch + 1) * 4].view(_torch().int32)
    lse = workspace[plan_bytes:plan_bytes + slots * num_qo_heads * 4].view(_torch().float32)
    o = workspace[plan_bytes + lse_bytes:plan_bytes + lse_bytes + slots * num_qo_heads * HEAD_DIM * 4]
    return plan, lse.view(slots, num_qo_heads), o.view(_torch().float32).view(slots, num_qo_heads, HEAD_DIM)


def balanced_workspace_segments(workspace, batch: int):
    """The segment table of a balanced-decode workspace: int32 [B, 2], each
    request's first and last segment (-1 for a request without keys)."""
    return workspace[(batch + 1) * 4:(3 * batch + 1) * 4].view(_torch().int32).view(batch, 2)


def decode_paged_multi(q, qo_indptr, k_pool, v_pool, page_indptr, page_indices, kv_len, sinks,
                       sm_scale: float, max_qo_len: int, num_splits: int = 1, window: int = 0,
                       out=None, o_part=None, lse_part=None, lse=None, return_lse: bool = False,
                       merge: bool = True, custom_mask=None, mask_indptr=None, kv_len_host=None,
                       stream=None):
    """Several query rows per request over a paged cache
    (``sinkattn_decode_paged_multi``); ``q`` is [total_q, Hq, 64] and
    ``qo_indptr`` [B+1] int32 with 1 .. ``max_qo_len`` rows per request.
    ``custom_mask`` (uint8 bit-packed, with int32 byte offsets
    ``mask_indptr`` [B+1]) replaces the causal rule.  Partials are per query
    row: ``o_part`` [total_q, Hq, S, 64], ``lse_part``
    [total_q, Hq, S].  ``kv_len_host`` as in :func:`decode_paged`.  Returns
    like :func:`decode_paged`."""
    torch = _torch()
    _dev(q, "q", torch.bfloat16)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [total_q, Hq, 64]")
    total_q, hq, _ = q.shape
    _dev(qo_indptr, "qo_indptr", torch.int32)
    batch = qo_indptr.numel() - 1
    if custom_mask is not None:
        _dev(custom_mask, "custom_mask", torch.uint8)
        _dev(mask_indptr, "mask_indptr", torch.int32, (batch + 1,))
    kvs = _kv_struct(k_pool, v_pool, page_indptr, page_indices, kv_len, kv_len_host)
    hkv = k_pool.shape[1]
    if sinks is not None:
        _dev(sinks, "sinks", torch.float32, (hq,))
    s = int(num_splits)
    if s > 1:
        if o_part is None:
            o_part = torch.empty((total_q, hq, s, HEAD_DIM), dtype=torch.float32, device=q.device)
        if lse_part is None:
            lse_part = torch.empty((total_q, hq, s), dtype=torch.float32, device=q.device)
        _dev(o_part, "o_part", torch.float32, (total_q, hq, s, HEAD_DIM))
        _dev(lse_part, "lse_part", torch.float32, (total_q, hq, s))
    else:
        o_part = lse_part = None
    want_out = s == 1 or merge
    if want_out and out is None:
        out = torch.empty_like(q)
    if out is not None:
        _dev(out, "out", torch.bfloat16, q.shape)
    if want_out and return_lse and lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (total_q, hq))
    lib = load_library()
    _check(lib.sinkattn_decode_paged_multi(_ptr(q), _ptr(qo_indptr), _ptr(custom_mask),
                                           _ptr(mask_indptr if custom_mask is not None else None),
                                           ctypes.byref(kvs), _ptr(sinks), s,
                                           _ptr(out if want_out else None), _ptr(o_part), _ptr(lse_part),
                                           _ptr(lse if want_out else None), batch, total_q,
                                           int(max_qo_len), hq, hkv, HEAD_DIM, float(sm_scale),
                                           int(window), _stream(stream)))
    if not want_out:
        return o_part, lse_part
    return (out, lse) if (return_lse or lse is not None) else out


def append_paged_kv_rope(k_new, v_new, append_indptr, k_pool, v_pool, page_indptr, page_indices, kv_len,
                         cos_sin, interleaved: bool = False, q=None, q_out=None, stream=None):
    """Append the new tokens' keys/values to the paged pools with rotary
    embedding of the keys and, when ``q`` is given, of the queries
    (``sinkattn_append_paged_kv_rope``).  ``cos_sin`` is [max_pos, 64] fp32;
    returns ``q_out`` (allocated if not given; may be ``q`` itself) or None."""
    torch = _torch()
    _dev(k_new, "k_new", torch.bfloat16)
    if k_new.dim() != 3 or k_new.shape[2] != HEAD_DIM:
        raise ValueError("k_new must be [total_new, Hkv, 64]")
    total_new, hkv, _ = k_new.shape
    _dev(v_new, "v_new", torch.bfloat16, k_new.shape)
    _dev(append_indptr, "append_indptr", torch.int32)
    batch = append_indptr.numel() - 1
    _dev(cos_sin, "cos_sin", torch.float32)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != HEAD_DIM:
        raise ValueError("cos_sin must be [max_pos, 64]")
    kvs = _kv_struct(k_pool, v_pool, page_indptr, page_indices, kv_len)
    if k_pool.shape[1] != hkv:
        raise ValueError("k_new and the pools disagree on the KV head count")
    hq = hkv
    if q is not None:
        _dev(q, "q", torch.bfloat16)
        if q.dim() != 3 or q.shape[0] != total_new or q.shape[2] != HEAD_DIM:
            raise ValueError("q must be [total_new, Hq, 64]")
        hq = q.shape[1]
        if q_out is None:
            q_out = torch.empty_like(q)
        _dev(q_out, "q_out", torch.bfloat16, q.shape)
    lib = load_library()
    _check(lib.sinkattn_append_paged_kv_rope(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(append_indptr),
                                             ctypes.byref(kvs), _ptr(cos_sin), cos_sin.shape[0],
                                             int(bool(interleaved)), _ptr(q_out if q is not None else None),
                                             batch, total_new, hq, hkv, HEAD_DIM, _stream(stream)))
    return q_out


def moe_topk_softmax(logits, top_k: int, topk_idx=None, topk_w=None, stream=None):
    """Top-K experts per token and the softmax over their logits alone
    (``sinkattn_moe_topk_softmax``): ``logits`` [T, E] bf16 -> (``topk_idx``
    [T, K] int32, ``topk_w`` [T, K] bf16)."""
    torch = _torch()
    _dev(logits, "logits", torch.bfloat16)
    if logits.dim() != 2:
        raise ValueError("logits must be [num_tokens, num_experts]")
    t, e = logits.shape
    k = int(top_k)
    if topk_idx is None:
        topk_idx = torch.empty((t, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((t, k), dtype=torch.bfloat16, device=logits.device)
    _dev(topk_idx, "topk_idx", torch.int32, (t, k))
    _dev(topk_w, "topk_w", torch.bfloat16, (t, k))
    lib = load_library()
    _check(lib.sinkattn_moe_topk_softmax(_ptr(logits), t, e, k, _ptr(topk_idx), _ptr(topk_w), _stream(stream)))
    return topk_idx, topk_w


def merge(o_part, lse_part, out=None, lse=None, return_lse: bool = False, stream=None):
    """LSE merge of split partials (``sinkattn_merge``): ``o_part`` [R, H, S, 64]
    fp32 and ``lse_part`` [R, H, S] fp32 -> ``out`` [R, H, 64] bf16."""
    torch = _torch()
    _dev(o_part, "o_part", torch.float32)
    if o_part.dim() != 4 or o_part.shape[3] != HEAD_DIM:
        raise ValueError("o_part must be [rows, heads, splits, 64]")
    rows, heads, s, _ = o_part.shape
    _dev(lse_part, "lse_part", torch.float32, (rows, heads, s))
    if out is None:
        out = torch.empty((rows, heads, HEAD_DIM), dtype=torch.bfloat16, device=o_part.device)
    _dev(out, "out", torch.bfloat16, (rows, heads, HEAD_DIM))
    if return_lse and lse is None:
        lse = torch.empty((rows, heads), dtype=torch.float32, device=o_part.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, (rows, heads))
    lib = load_library()
    _check(lib.sinkattn_merge(_ptr(o_part), _ptr(lse_part), rows, heads, s, HEAD_DIM, _ptr(out),
                              _ptr(lse), _stream(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def split_bounds(kv_len_host, num_splits: int, page_size: int = PAGE_SIZE) -> np.ndarray:
    """Host-only chunk rule of the split decode: int32 [B, S, 2] token ranges."""
    lens = np.ascontiguousarray(kv_len_host, dtype=np.int32)
    out = np.zeros((len(lens), num_splits, 2), dtype=np.int32)
    lib = load_library()
    _check(lib.sinkattn_split_bounds(lens.ctypes.data_as(ctypes.c_void_p), len(lens), page_size,
                                     num_splits, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def pick_num_splits(kv_len_host, num_kv_heads: int) -> int:
    """Host-only split count suggested for a decode batch."""
    lens = np.ascontiguousarray(kv_len_host, dtype=np.int32)
    return int(load_library().sinkattn_pick_num_splits(lens.ctypes.data_as(ctypes.c_void_p), len(lens),
                                                       num_kv_heads))


def pick_num_splits_multi(kv_len_host, num_qo_heads: int, num_kv_heads: int, max_qo_len: int,
                          with_mask: bool = False) -> int:
    """Host-only split count suggested for a several-row (verify) batch."""
    lens = np.ascontiguousarray(kv_len_host, dtype=np.int32)
    return int(load_library().sinkattn_pick_num_splits_multi(lens.ctypes.data_as(ctypes.c_void_p), len(lens),
                                                             num_qo_heads, num_kv_heads, max_qo_len,
                                                             int(bool(with_mask))))


def validate_kv_host(kv_indptr, num_pages: int, page_indices=None, kv_len=None):
    """Host-only check of a batch's KV metadata (``sinkattn_validate_kv_host``)
    before it is copied to the GPU: ``kv_indptr`` [B+1], and for a paged cache
    ``page_indices`` and ``kv_len`` [B] (host arrays); ``num_pages`` is the
    pool's page count (paged) or the rows of k and v (contiguous).  Raises
    ``SinkAttnError`` naming the first bad entry."""
    indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    paged = page_indices is not None
    pages = np.ascontiguousarray(page_indices if paged else np.zeros(1), dtype=np.int32)
    lens = np.ascontiguousarray(kv_len if paged else np.zeros(1), dtype=np.int32)
    if indptr.ndim != 1 or indptr.size < 1:
        raise ValueError("kv_indptr must be a 1-D array of batch + 1 offsets")
    if paged and lens.shape != (indptr.size - 1,):
        raise ValueError("kv_len must have one entry per request")
    if paged and not (0 <= int(indptr[-1]) <= pages.size):
        raise ValueError("page_indices must hold kv_indptr[-1] entries")
    kv = _KV(None, None, int(paged), PAGE_SIZE, None, None, None, int(num_pages), None)
    vp = ctypes.c_void_p
    _check(load_library().sinkattn_validate_kv_host(ctypes.byref(kv), indptr.ctypes.data_as(vp),
                                                    pages.ctypes.data_as(vp) if paged else None,
                                                    lens.ctypes.data_as(vp) if paged else None,
                                                    indptr.size - 1))


def raw_library():
    """The ctypes handle, for callers that drive the C ABI directly."""
    return load_library()


def kv_descriptor(k, v, kv_indptr, page_indices=None, kv_len=None, kv_len_host=None) -> _KV:
    """Build the ``sinkattn_kv`` struct for direct C-ABI calls (it keeps the
    int32 copy of ``kv_len_host`` it points to alive)."""
    return _kv_struct(k, v, kv_indptr, page_indices, kv_len, kv_len_host)
