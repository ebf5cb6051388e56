"""ctypes binding of libpsattn.so (C ABI in include/psattn.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of the shared library.  PyTorch supplies device memory and the
current HIP stream.  There is no fallback: if the library is missing or a call
fails, an exception is raised.

The C entry points are exposed under their own names (``psattn_fwd``,
``psattn_fwd_noalloc``, ``psattn_workspace_size``, ``psattn_bwd``,
``psattn_bwd_workspace_size``, ``psattn_mla_fwd``, ``psattn_mla_dense_fwd``,
``psattn_plan_dump``, ``psattn_plan_host``, ``psattn_status_string``,
``psattn_last_error``) taking raw integers / pointers, plus tensor-level
helpers (``fwd_flat``, ``fwd_paged``, ``bwd_flat``, ``fwd_mla``,
``fwd_mla_dense``).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpsattn.so")

F32, BF16, FP8 = 0, 1, 2
MODE_FLAT, MODE_PAGED = 0, 1
OK, E_INVAL, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, 1, 2, 3, 4
ITEM_FIELDS = 10


class PsattnDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("prefix_len", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("seg_offsets", ctypes.c_void_p),
        ("max_seg_len", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("draft_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("prefix_lens", ctypes.c_void_p),
        ("kv_indptr", ctypes.c_void_p),
        ("kv_indices", ctypes.c_void_p),
        ("max_prefix_len", ctypes.c_int32),
        ("k_ext", ctypes.c_void_p),
        ("v_ext", ctypes.c_void_p),
        ("draft_mask", ctypes.c_void_p),
        ("qo_indptr", ctypes.c_void_p),
        ("seg_parent", ctypes.c_void_p),
    ]


class PsattnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_items", ctypes.c_int64),
        ("tile_tokens", ctypes.c_int32),
        ("rows_per_tile", ctypes.c_int32),
        ("n_splits", ctypes.c_int32),
        ("split_len", ctypes.c_int32),
        ("kv_tile", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class PsattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"psattn status {status}: {msg}")
        self.status = status


_lib = None


def load(path: Optional[str] = None):
    """Load libpsattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it first (python -m prefix_shared_block_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    dp = ctypes.POINTER(PsattnDesc)
    ip = ctypes.POINTER(PsattnPlanInfo)
    lib.psattn_fwd.argtypes = [vp, vp, vp, vp, vp, dp, i32, i32, i32, f32, i32, i32, f32, f32, vp, sz, vp]
    lib.psattn_fwd.restype = i32
    lib.psattn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, dp, i32, i32, i32, f32, i32, i32, f32, f32, vp]
    lib.psattn_fwd_noalloc.restype = i32
    lib.psattn_workspace_size.argtypes = [dp, i32, i32, i32, i32, i32]
    lib.psattn_workspace_size.restype = sz
    lib.psattn_plan_dump.argtypes = [dp, i32, i32, i32, i32, i32, vp, i64, ip, vp]
    lib.psattn_plan_dump.restype = i32
    lib.psattn_plan_host.argtypes = [dp, i32, i32, i32, i32, i32, vp, i64, ip]
    lib.psattn_plan_host.restype = i32
    lib.psattn_bwd_workspace_size.argtypes = [dp, i32, i32, i32, i32]
    lib.psattn_bwd_workspace_size.restype = sz
    lib.psattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, dp, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.psattn_bwd.restype = i32
    lib.psattn_mla_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, i32, f32, i32, vp]
    lib.psattn_mla_fwd.restype = i32
    lib.psattn_mla_dense_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, f32, i32, vp]
    lib.psattn_mla_dense_fwd.restype = i32
    lib.psattn_status_string.argtypes = [i32]
    lib.psattn_status_string.restype = ctypes.c_char_p
    lib.psattn_last_error.argtypes = []
    lib.psattn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ------------------------------------------------------------------ raw C ABI
def _ref(desc):
    return None if desc is None else ctypes.byref(desc)


def psattn_status_string(status: int) -> str:
    return load().psattn_status_string(status).decode()


def psattn_last_error() -> str:
    return load().psattn_last_error().decode()


def psattn_workspace_size(desc: PsattnDesc, hq: int, hkv: int, d: int, q_dtype: int, kv_dtype: int) -> int:
    return int(load().psattn_workspace_size(_ref(desc), hq, hkv, d, q_dtype, kv_dtype))


def psattn_fwd(q: int, k: int, v: int, o: int, lse: int, desc: PsattnDesc, hq: int, hkv: int, d: int,
               sm_scale: float, q_dtype: int, kv_dtype: int, k_scale: float, v_scale: float,
               workspace: int, workspace_bytes: int, stream: int) -> int:
    return int(load().psattn_fwd(q, k, v, o, lse, _ref(desc), hq, hkv, d, sm_scale, q_dtype,
                                 kv_dtype, k_scale, v_scale, workspace, workspace_bytes, stream))


def psattn_fwd_noalloc(q: int, k: int, v: int, o: int, lse: int, desc: PsattnDesc, hq: int, hkv: int, d: int,
                       sm_scale: float, q_dtype: int, kv_dtype: int, k_scale: float, v_scale: float,
                       stream: int) -> int:
    return int(load().psattn_fwd_noalloc(q, k, v, o, lse, _ref(desc), hq, hkv, d, sm_scale, q_dtype, kv_dtype,
                                         k_scale, v_scale, stream))


def psattn_bwd_workspace_size(desc: PsattnDesc, hq: int, hkv: int, d: int, dtype: int) -> int:
    return int(load().psattn_bwd_workspace_size(_ref(desc), hq, hkv, d, dtype))


def psattn_bwd(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int,
               desc: PsattnDesc, hq: int, hkv: int, d: int, sm_scale: float, dtype: int, workspace: int,
               workspace_bytes: int, stream: int) -> int:
    return int(load().psattn_bwd(q, k, v, o, lse, dout, dq, dk, dv, _ref(desc), hq, hkv, d, sm_scale, dtype,
                                 workspace, workspace_bytes, stream))


def psattn_mla_fwd(q: int, ckv: int, indices: int, sink: int, o: int, lse: int, num_tokens: int, num_heads: int,
                   dim: int, num_kv: int, kv_stride: int, topk: int, sm_scale: float, dtype: int, stream: int) -> int:
    return int(load().psattn_mla_fwd(q, ckv, indices, sink, o, lse, num_tokens, num_heads, dim, num_kv, kv_stride,
                                     topk, sm_scale, dtype, stream))


def psattn_mla_dense_fwd(q: int, ckv: int, sink: int, o: int, lse: int, num_tokens: int, num_heads: int,
                         dim: int, num_kv: int, kv_stride: int, sm_scale: float, dtype: int, stream: int) -> int:
    return int(load().psattn_mla_dense_fwd(q, ckv, sink, o, lse, num_tokens, num_heads, dim, num_kv, kv_stride,
                                           sm_scale, dtype, stream))


def psattn_plan_dump(desc: PsattnDesc, hq: int, hkv: int, d: int, q_dtype: int, kv_dtype: int,
                     items_dev: int, capacity: int, info: PsattnPlanInfo, stream: int) -> int:
    return int(load().psattn_plan_dump(_ref(desc), hq, hkv, d, q_dtype, kv_dtype, items_dev,
                                       capacity, ctypes.byref(info), stream))


def psattn_plan_host(desc: PsattnDesc, hq: int, hkv: int, d: int, q_dtype: int, kv_dtype: int,
                     items_host: int, capacity: int, info: PsattnPlanInfo) -> int:
    return int(load().psattn_plan_host(_ref(desc), hq, hkv, d, q_dtype, kv_dtype, items_host,
                                       capacity, ctypes.byref(info)))


def check(status: int):
    if status != OK:
        raise PsattnError(status, f"{psattn_status_string(status)}: {psattn_last_error()}")


# ------------------------------------------------------------------ descriptors
def flat_desc(total_tokens: int, prefix_len: int, num_segments: int, seg_offsets_ptr: int,
              max_seg_len: int, seg_parent_ptr: int = 0) -> PsattnDesc:
    d = PsattnDesc()
    d.mode = MODE_FLAT
    d.total_tokens = int(total_tokens)
    d.prefix_len = int(prefix_len)
    d.num_segments = int(num_segments)
    d.seg_offsets = seg_offsets_ptr or None
    d.max_seg_len = int(max_seg_len)
    d.seg_parent = seg_parent_ptr or None
    return d


def paged_desc(batch: int, draft_len: int, page_size: int, num_pages: int, prefix_lens_ptr: int,
               kv_indptr_ptr: int, kv_indices_ptr: int, max_prefix_len: int, k_ext_ptr: int,
               v_ext_ptr: int, draft_mask_ptr: int = 0, qo_indptr_ptr: int = 0) -> PsattnDesc:
    d = PsattnDesc()
    d.mode = MODE_PAGED
    d.batch = int(batch)
    d.draft_len = int(draft_len)
    d.page_size = int(page_size)
    d.num_pages = int(num_pages)
    d.prefix_lens = prefix_lens_ptr or None
    d.kv_indptr = kv_indptr_ptr or None
    d.kv_indices = kv_indices_ptr or None
    d.max_prefix_len = int(max_prefix_len)
    d.k_ext = k_ext_ptr or None
    d.v_ext = v_ext_ptr or None
    d.draft_mask = draft_mask_ptr or None
    d.qo_indptr = qo_indptr_ptr or None
    return d


# ------------------------------------------------------------------ tensor helpers
def _dtype_code(t, explicit: Optional[int] = None) -> int:
    import torch

    if explicit is not None:
        return explicit
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _stream_handle(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def fwd_flat(q, k, v, prefix_len: int, seg_offsets, max_seg_len: int, sm_scale: Optional[float] = None,
             out=None, lse=None, seg_parent=None):
    """Flat-packed [P | S1 .. SN] forward.  q [T,Hq,D], k/v [T,Hkv,D] contiguous
    on one GPU; seg_offsets: int32 device tensor with N+1 entries; max_seg_len:
    host upper bound of the segment lengths; seg_parent: optional int32
    device tensor of N parent segments (-1: the prefix) for multi-level
    sharing.  Returns (o, lse)."""
    import torch

    t_n, hq, d = q.shape
    hkv = k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((t_n, hq), dtype=torch.float32, device=q.device)
    n = int(seg_offsets.numel()) - 1 if seg_offsets is not None else 0
    if seg_parent is not None and int(seg_parent.numel()) != n:
        raise ValueError(f"seg_parent has {int(seg_parent.numel())} entries, {n} segments")
    desc = flat_desc(t_n, prefix_len, n, _ptr(seg_offsets), max_seg_len, _ptr(seg_parent))
    qdt = _dtype_code(q)
    st = psattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), desc, hq, hkv, d, float(sm_scale),
                    qdt, _dtype_code(k), 1.0, 1.0, 0, 0, _stream_handle(q.device))
    check(st)
    return out, lse


def bwd_flat(q, k, v, o, lse, dout, prefix_len: int, seg_offsets, max_seg_len: int,
             sm_scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None, seg_parent=None):
    """Gradients of the flat forward for the upstream gradient dout.  o and
    lse are the forward's outputs; shapes and the descriptor (seg_parent
    included) as in fwd_flat.  Returns (dq, dk, dv)."""
    import torch

    t_n, hq, d = q.shape
    hkv = k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    n = int(seg_offsets.numel()) - 1 if seg_offsets is not None else 0
    if seg_parent is not None and int(seg_parent.numel()) != n:
        raise ValueError(f"seg_parent has {int(seg_parent.numel())} entries, {n} segments")
    desc = flat_desc(t_n, prefix_len, n, _ptr(seg_offsets), max_seg_len, _ptr(seg_parent))
    dt = _dtype_code(q)
    ws_bytes = psattn_bwd_workspace_size(desc, hq, hkv, d, dt)
    if ws_bytes == 0 and t_n > 0:
        raise PsattnError(2, psattn_last_error())
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = psattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), desc,
                    hq, hkv, d, float(sm_scale), dt, _ptr(workspace), wsz, _stream_handle(q.device))
    check(st)
    return dq, dk, dv


def fwd_mla(q, ckv, indices, sm_scale: Optional[float] = None, sink=None, out=None, lse=None):
    """Sparse shared-latent MLA forward.  q [T, H, 512] bf16; ckv [S, stride]
    bf16 latent rows (the first 512 used); indices int32 [T, topk] (-1 or any
    entry outside [0, S) skipped); sink: optional fp32 [H].  Returns (o, lse)."""
    import torch

    t_n, hq, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if ckv.dim() != 2 or ckv.stride(1) != 1:
        raise ValueError("ckv must be [S, stride] with unit column stride")
    if indices.dim() != 2 or indices.shape[0] != t_n or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous [T, topk] tensor")
    if indices.dtype != torch.int32:
        raise TypeError(f"indices must be int32, not {indices.dtype}")
    if not q.is_contiguous():
        raise ValueError("q must be a contiguous [T, H, D] tensor")
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() != hq or not sink.is_contiguous()):
        raise ValueError("sink must be a contiguous float32 tensor of H entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((t_n, hq), dtype=torch.float32, device=q.device)
    st = psattn_mla_fwd(_ptr(q), _ptr(ckv), _ptr(indices), _ptr(sink), _ptr(out), _ptr(lse), t_n, hq, d,
                        int(ckv.shape[0]), int(ckv.stride(0)), int(indices.shape[1]), float(sm_scale),
                        _dtype_code(q), _stream_handle(q.device))
    check(st)
    return out, lse


def fwd_mla_dense(q, ckv, sm_scale: Optional[float] = None, sink=None, out=None, lse=None):
    """Dense causal shared-latent MLA prefill.  q [T, H, 512] bf16 are the
    last T rows of the cache ckv [S, stride] bf16 (S >= T); token t attends
    to rows 0 .. S - T + t.  sink: optional fp32 [H].  Returns (o, lse)."""
    import torch

    t_n, hq, d = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if ckv.dim() != 2 or ckv.stride(1) != 1:
        raise ValueError("ckv must be [S, stride] with unit column stride")
    if not q.is_contiguous():
        raise ValueError("q must be a contiguous [T, H, D] tensor")
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() != hq or not sink.is_contiguous()):
        raise ValueError("sink must be a contiguous float32 tensor of H entries")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((t_n, hq), dtype=torch.float32, device=q.device)
    st = psattn_mla_dense_fwd(_ptr(q), _ptr(ckv), _ptr(sink), _ptr(out), _ptr(lse), t_n, hq, d, int(ckv.shape[0]),
                              int(ckv.stride(0)), float(sm_scale), _dtype_code(q), _stream_handle(q.device))
    check(st)
    return out, lse


def fwd_paged(q, k_pool, v_pool, kv_indptr, kv_indices, prefix_lens, k_ext, v_ext, draft_len: int,
              max_prefix_len: int, sm_scale: Optional[float] = None, k_scale: float = 1.0,
              v_scale: float = 1.0, kv_dtype: Optional[int] = None, out=None, lse=None, workspace=None,
              draft_mask=None, qo_indptr=None, noalloc: bool = False):
    """Speculative-verify forward over a paged prefix.  q [B*Lx,Hq,D];
    pools [num_pages, page_size, Hkv, D]; k_ext/v_ext [B*Lx, Hkv, D]; index
    arrays int32 on the device; draft_mask: optional uint8 [B, Lx, Lx] draft
    tree on the device (None: the causal chain); qo_indptr: optional int32
    [B+1] ragged draft rows on the device, draft_len then being their upper
    bound (q holds qo_indptr[B] rows).  noalloc=True calls
    psattn_fwd_noalloc (split scratch in the library's device array; no
    workspace is allocated here).  Returns (o, lse)."""
    import torch

    rows, hq, d = q.shape
    num_pages, page_size, hkv, _ = k_pool.shape
    batch = int(prefix_lens.numel())
    if qo_indptr is None and rows != batch * draft_len:
        raise ValueError("q must hold batch * draft_len rows (or pass qo_indptr)")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    kvdt = _dtype_code(k_pool, kv_dtype)
    qdt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((rows, hq), dtype=torch.float32, device=q.device)
    desc = paged_desc(batch, draft_len, page_size, num_pages, _ptr(prefix_lens), _ptr(kv_indptr),
                      _ptr(kv_indices), max_prefix_len, _ptr(k_ext), _ptr(v_ext), _ptr(draft_mask),
                      _ptr(qo_indptr))
    if noalloc:
        check(psattn_fwd_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), desc, hq, hkv, d,
                                 float(sm_scale), qdt, kvdt, float(k_scale), float(v_scale),
                                 _stream_handle(q.device)))
        return out, lse
    ws_bytes = psattn_workspace_size(desc, hq, hkv, d, qdt, kvdt)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = psattn_fwd(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), desc, hq, hkv, d,
                    float(sm_scale), qdt, kvdt, float(k_scale), float(v_scale), _ptr(workspace), wsz,
                    _stream_handle(q.device))
    check(st)
    return out, lse


def plan_info(desc: PsattnDesc, hq: int, hkv: int, d: int, q_dtype: int, kv_dtype: int) -> PsattnPlanInfo:
    info = PsattnPlanInfo()
    check(psattn_plan_host(desc, hq, hkv, d, q_dtype, kv_dtype, 0, 0, info))
    return info
