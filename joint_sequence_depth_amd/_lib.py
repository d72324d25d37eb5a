"""ctypes binding of libmoda_attn.so (argument marshalling only).

Every step of the computation runs in the HIP library. torch supplies device
memory and the current stream. There is no fallback: without the built library
(or without a GPU) the calls raise.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoda_attn.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

STATUS_NAMES = {
    0: "MODA_OK",
    1: "MODA_ERR_NULL",
    2: "MODA_ERR_SHAPE",
    3: "MODA_ERR_DTYPE",
    4: "MODA_ERR_ALIGN",
    5: "MODA_ERR_UNSUPPORTED",
    6: "MODA_ERR_HIP",
    7: "MODA_ERR_VALUE",
}

# every symbol include/moda_attn.h declares
EXPORTS = ("moda_attn_fwd", "moda_attn_fwd_varlen", "moda_attn_fwd_phases", "moda_attn_fwd_varlen_phases",
           "moda_attn_fwd_topk", "moda_attn_fwd_varlen_topk", "moda_attn_fwd_topk_workspace_size",
           "moda_attn_decode", "moda_attn_decode_noalloc", "moda_attn_decode_workspace_size",
           "moda_attn_bwd", "moda_attn_bwd_varlen", "moda_attn_bwd_workspace_size", "moda_depth_kv_write",
           "moda_depth_kv_project",
           "moda_last_error", "moda_abi_version")

_lib = None


class ModaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the shared library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route this module's calls to another build of the library (the
    poisoned-LDS debug build) inside the block."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m joint_sequence_depth_amd.build` "
            "(there is no non-HIP fallback)"
        )
    L = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.moda_attn_fwd.argtypes = [vp] * 7 + [i32, i32, i64, i64, i32, i32, i32, i32, i32, i32, f32, vp]
    L.moda_attn_fwd.restype = ctypes.c_int
    L.moda_attn_fwd_varlen.argtypes = [vp] * 7 + [i32, i32, vp, i32, i64, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    L.moda_attn_fwd_varlen.restype = ctypes.c_int
    L.moda_attn_fwd_phases.argtypes = L.moda_attn_fwd.argtypes[:-1] + [i32, vp]
    L.moda_attn_fwd_phases.restype = ctypes.c_int
    L.moda_attn_fwd_varlen_phases.argtypes = L.moda_attn_fwd_varlen.argtypes[:-1] + [i32, vp]
    L.moda_attn_fwd_varlen_phases.restype = ctypes.c_int
    L.moda_attn_fwd_topk.argtypes = L.moda_attn_fwd.argtypes[:16] + [i32, i32] + L.moda_attn_fwd.argtypes[16:18] + [
        vp, i64, vp]
    L.moda_attn_fwd_topk.restype = ctypes.c_int
    L.moda_attn_fwd_varlen_topk.argtypes = L.moda_attn_fwd_varlen.argtypes[:18] + [i32, i32] + \
        L.moda_attn_fwd_varlen.argtypes[18:20] + [vp, i64, vp]
    L.moda_attn_fwd_varlen_topk.restype = ctypes.c_int
    L.moda_attn_fwd_topk_workspace_size.argtypes = [i64, i32]
    L.moda_attn_fwd_topk_workspace_size.restype = ctypes.c_int64
    L.moda_attn_decode.argtypes = [vp] * 7 + [i32, i32, vp, i64, i32, i32, i32, i32, i32, i32, f32, vp, i64, vp]
    L.moda_attn_decode.restype = ctypes.c_int
    L.moda_attn_decode_noalloc.argtypes = [vp] * 7 + [i32, i32, vp, i64, i32, i32, i32, i32, i32, i32, f32, vp]
    L.moda_attn_decode_noalloc.restype = ctypes.c_int
    L.moda_attn_decode_workspace_size.argtypes = [i64, i32, i32, i32, i32]
    L.moda_attn_decode_workspace_size.restype = ctypes.c_int64
    L.moda_attn_bwd.argtypes = [vp] * 13 + [i32, i32, i64, i64, i32, i32, i32, i32, i32, i32, f32, vp, i64, vp]
    L.moda_attn_bwd.restype = ctypes.c_int
    L.moda_attn_bwd_varlen.argtypes = [vp] * 13 + [i32, i32, vp, i32, i64, i32, i32, i32, i32, i32, i32, i32, f32,
                                                    vp, i64, vp]
    L.moda_attn_bwd_varlen.restype = ctypes.c_int
    L.moda_attn_bwd_workspace_size.argtypes = [i64, i32, i32, i32]
    L.moda_attn_bwd_workspace_size.restype = ctypes.c_int64
    L.moda_depth_kv_write.argtypes = [vp] * 4 + [i32, i64, i32, i32, i32, i32, vp]
    L.moda_depth_kv_write.restype = ctypes.c_int
    L.moda_depth_kv_project.argtypes = [vp] * 4 + [i32, i64, i32, i32, i32, i32, i32, vp]
    L.moda_depth_kv_project.restype = ctypes.c_int
    L.moda_last_error.argtypes = []
    L.moda_last_error.restype = ctypes.c_char_p
    L.moda_abi_version.argtypes = []
    L.moda_abi_version.restype = ctypes.c_int32
    return L


def _check(status: int):
    if status != 0:
        raise ModaError(status, lib().moda_last_error().decode(errors="replace"))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _window(k_depth, v_depth, slot_offset: int, n_depth: int, s_cap: int, row_elems: int):
    """Depth base pointers of the slot window [slot_offset, slot_offset + n_depth)."""
    if k_depth is None:
        if slot_offset:
            raise ValueError("slot_offset needs depth tensors")
        return None, None
    if slot_offset < 0 or n_depth < 0 or slot_offset + n_depth > s_cap:
        raise ValueError(f"slot window [{slot_offset}, {slot_offset + n_depth}) exceeds S_cap = {s_cap}")
    off = slot_offset * row_elems * k_depth.element_size()
    return k_depth.data_ptr() + off, v_depth.data_ptr() + off


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def attn_fwd(
    q,
    k,
    v,
    k_depth=None,
    v_depth=None,
    n_depth: Optional[int] = None,
    causal: bool = True,
    scale: Optional[float] = None,
    cu_seqlens=None,
    max_seqlen: Optional[int] = None,
    out=None,
    lse=None,
    stream=None,
    out_dtype=None,
    return_lse: bool = True,
    slot_offset: int = 0,
    phase: int = 3,
    depth_topk: Optional[int] = None,
    depth_recent: int = 0,
    workspace=None,
):
    """MoDA joint sequence/depth attention forward through the C ABI.

    Batch layout: q [B,T,Hq,d], k/v [B,T,Hkv,d], k_depth/v_depth [B,T,S_cap,Hkv,d].
    Packed layout (cu_seqlens, int32 [n_seqs+1] on the device): q [N,Hq,d], k/v
    [N,Hkv,d], depth [N,S_cap,Hkv,d]. Returns (out, lse) with out like q and lse
    float32 [B,Hq,T] or [Hq,N]. ``n_depth`` defaults to the slot capacity (0 without
    depth tensors); ``scale`` to 1/sqrt(d). ``out_dtype`` (torch.float32 is allowed
    for bfloat16 inputs) defaults to q's dtype, or to ``out``'s when it is given.
    With ``return_lse=False`` no lse is written (NULL at the C ABI) and None is returned.
    ``slot_offset`` reads the window of slots [slot_offset, slot_offset + n_depth)
    (the depth base pointers move by that many slots; the slot stride stays S_cap).
    ``phase`` 1 or 2 computes the sequence part or the depth part alone (each its
    own softmax, for measurement and for the merge check); 3, the default, is the
    operator. Packed calls need ``max_seqlen`` (the longest sequence): the binding
    never reads ``cu_seqlens`` back from the device.
    ``depth_topk`` (with ``depth_recent``) makes each row read only some of its
    depth slots: the last ``depth_recent`` and the ``depth_topk`` others with the
    largest depth logits (top-S, sliding window or hybrid buffer; n_depth <= 64).
    ``workspace`` (uint8 device tensor of ``topk_workspace_size`` bytes) holds the
    per-row slot masks; allocated here when not given.
    """
    import torch

    varlen = cu_seqlens is not None
    lead = 1 if varlen else 2
    if q.dim() != lead + 2 or k.dim() != lead + 2 or v.dim() != lead + 2:
        raise ValueError("q, k, v must be [B,T,H,d] (or [N,H,d] with cu_seqlens)")
    for t in (q, k, v, k_depth, v_depth, out, lse, cu_seqlens):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if t is not None and t.device.type != "cuda":
            raise ValueError("all tensors must be on the GPU")
    d = q.shape[-1]
    Hq, Hkv = q.shape[-2], k.shape[-2]
    if k.shape != v.shape or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if k_depth is not None:
        if v_depth is None or k_depth.shape != v_depth.shape:
            raise ValueError("k_depth and v_depth must both be given with one shape")
        if k_depth.dim() != lead + 3 or k_depth.shape[:lead] != q.shape[:lead] or k_depth.shape[-2:] != (Hkv, d):
            raise ValueError(f"depth tensors must be [..., S_cap, Hkv, d], got {tuple(k_depth.shape)}")
        if k_depth.dtype != q.dtype or v_depth.dtype != q.dtype:
            raise TypeError("depth tensors must share q's dtype")
        s_cap = k_depth.shape[lead]
    else:
        s_cap = 0
    if n_depth is None:
        n_depth = s_cap - slot_offset
    kd_ptr, vd_ptr = _window(k_depth, v_depth, slot_offset, n_depth, s_cap, Hkv * d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must have q's shape and out_dtype")
    if varlen:
        N = q.shape[0]
        lse_shape = (Hq, N)
    else:
        B, T = q.shape[0], q.shape[1]
        lse_shape = (B, Hq, T)
    if not return_lse:
        lse = None
    elif lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    elif tuple(lse.shape) != lse_shape or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 {lse_shape}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    code = _dtype_code(q)
    out_code = _dtype_code(out)
    L = lib()
    if depth_topk is not None:
        if phase != 3:
            raise ValueError("bounded depth reads run the whole operator (phase 3)")
        n_tok = q.shape[0] if varlen else q.shape[0] * q.shape[1]
        if workspace is None:
            workspace = torch.empty(max(topk_workspace_size(n_tok, Hq), 16), dtype=torch.uint8, device=q.device)
        elif not workspace.is_contiguous() or workspace.device.type != "cuda":
            raise ValueError("workspace must be a contiguous GPU tensor")
        sel = (int(depth_topk), int(depth_recent))
        ws = (_ptr(workspace), workspace.numel() * workspace.element_size())
    if varlen:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
        n_seqs = cu_seqlens.numel() - 1
        if max_seqlen is None:
            raise ValueError("packed calls need max_seqlen (the longest sequence); cu_seqlens stays on the device")
        args = (_ptr(q), _ptr(k), _ptr(v), kd_ptr, vd_ptr, _ptr(out), _ptr(lse), code, out_code, _ptr(cu_seqlens),
                n_seqs, q.shape[0], int(max_seqlen), Hq, Hkv, d, s_cap, int(n_depth), int(bool(causal)), float(scale))
        if depth_topk is not None:
            status = L.moda_attn_fwd_varlen_topk(*args[:18], *sel, *args[18:], *ws, stream)
        elif phase == 3:
            status = L.moda_attn_fwd_varlen(*args, stream)
        else:
            status = L.moda_attn_fwd_varlen_phases(*args, int(phase), stream)
    else:
        args = (_ptr(q), _ptr(k), _ptr(v), kd_ptr, vd_ptr, _ptr(out), _ptr(lse), code, out_code, q.shape[0],
                q.shape[1], Hq, Hkv, d, s_cap, int(n_depth), int(bool(causal)), float(scale))
        if depth_topk is not None:
            status = L.moda_attn_fwd_topk(*args[:16], *sel, *args[16:], *ws, stream)
        elif phase == 3:
            status = L.moda_attn_fwd(*args, stream)
        else:
            status = L.moda_attn_fwd_phases(*args, int(phase), stream)
    _check(status)
    return out, lse


def topk_workspace_size(total_tokens: int, n_heads_q: int) -> int:
    """Bytes of device workspace a bounded-depth-read forward over N tokens needs."""
    n = lib().moda_attn_fwd_topk_workspace_size(total_tokens, n_heads_q)
    if n < 0:
        raise ValueError("invalid sizes")
    return int(n)


def decode_workspace_size(batch: int, n_heads_q: int, n_heads_kv: int, head_dim: int, max_cache_len: int) -> int:
    """Bytes of device workspace one decode call with these sizes needs."""
    n = lib().moda_attn_decode_workspace_size(batch, n_heads_q, n_heads_kv, head_dim, max_cache_len)
    if n < 0:
        raise ValueError("invalid decode sizes")
    return int(n)


def attn_decode(
    q,
    k_cache,
    v_cache,
    cache_seqlens,
    k_depth=None,
    v_depth=None,
    n_depth: Optional[int] = None,
    scale: Optional[float] = None,
    out=None,
    lse=None,
    workspace=None,
    stream=None,
    out_dtype=None,
    return_lse: bool = True,
):
    """One decode step through the C ABI: q [B,Hq,d] (one new token per sequence),
    k_cache/v_cache [B,T_max,Hkv,d] with cache_seqlens (int32 [B] on the device)
    valid rows each (the last being the new token's own), k_depth/v_depth
    [B,S_cap,Hkv,d] the new token's depth slots. Returns (out [B,Hq,d], lse
    float32 [B,Hq]). ``workspace`` (a uint8 device tensor) is allocated here when
    not given; pass one to keep the call allocation-free."""
    import torch

    for t in (q, k_cache, v_cache, cache_seqlens, k_depth, v_depth, out, lse, workspace):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if t is not None and t.device.type != "cuda":
            raise ValueError("all tensors must be on the GPU")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B,Hq,d] and the caches [B,T_max,Hkv,d]")
    B, Hq, d = q.shape
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} cache{tuple(k_cache.shape)}")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("cache_seqlens must be int32 [B] on the device")
    if k_depth is not None:
        if v_depth is None or k_depth.shape != v_depth.shape or k_depth.dim() != 4:
            raise ValueError("k_depth and v_depth must both be [B,S_cap,Hkv,d]")
        if k_depth.shape[0] != B or k_depth.shape[2:] != (Hkv, d):
            raise ValueError(f"depth tensors must be [B,S_cap,Hkv,d], got {tuple(k_depth.shape)}")
        if k_depth.dtype != q.dtype or v_depth.dtype != q.dtype:
            raise TypeError("depth tensors must share q's dtype")
        s_cap = k_depth.shape[1]
    else:
        s_cap = 0
    if n_depth is None:
        n_depth = s_cap
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype:
        raise ValueError("out must have q's shape and out_dtype")
    if not return_lse:
        lse = None
    elif lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif tuple(lse.shape) != (B, Hq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq]")
    if workspace is None:
        n = decode_workspace_size(B, Hq, Hkv, d, T_max) if B > 0 else 0
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = lib().moda_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_depth), _ptr(v_depth), _ptr(out), _ptr(lse),
        _dtype_code(q), _dtype_code(out), _ptr(cache_seqlens), B, T_max, Hq, Hkv, d, s_cap, int(n_depth),
        float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), stream,
    )
    _check(status)
    return out, lse


DECODE_SCRATCH_BYTES = 16 << 20  # MODA_DECODE_SCRATCH_BYTES


def attn_decode_noalloc(q, k_cache, v_cache, cache_seqlens, out, k_depth=None, v_depth=None,
                        n_depth: Optional[int] = None, scale: Optional[float] = None, lse=None, stream=None):
    """One decode step through ``moda_attn_decode_noalloc``: as ``attn_decode``, but
    the partial states go through the library's own per-GPU scratch array, so
    neither the library nor this binding allocates anything: ``out`` (and ``lse``,
    if wanted; None = not written) are the caller's. Steps needing more than
    DECODE_SCRATCH_BYTES of scratch are rejected. Calls that overlap on one GPU
    share the scratch and race. Returns (out, lse)."""
    import torch

    for t in (q, k_cache, v_cache, cache_seqlens, k_depth, v_depth, out, lse):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if t is not None and t.device.type != "cuda":
            raise ValueError("all tensors must be on the GPU")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B,Hq,d] and the caches [B,T_max,Hkv,d]")
    B, Hq, d = q.shape
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d or out.shape != q.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} cache{tuple(k_cache.shape)} out{tuple(out.shape)}")
    if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("cache_seqlens must be int32 [B] on the device")
    if lse is not None and (tuple(lse.shape) != (B, Hq) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, Hq]")
    s_cap = 0
    if k_depth is not None:
        if v_depth is None or k_depth.shape != v_depth.shape or k_depth.dim() != 4:
            raise ValueError("k_depth and v_depth must both be [B,S_cap,Hkv,d]")
        s_cap = k_depth.shape[1]
    if n_depth is None:
        n_depth = s_cap
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = lib().moda_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_depth), _ptr(v_depth), _ptr(out), _ptr(lse),
        _dtype_code(q), _dtype_code(out), _ptr(cache_seqlens), B, T_max, Hq, Hkv, d, s_cap, int(n_depth),
        float(scale), stream,
    )
    _check(status)
    return out, lse


def bwd_workspace_size(total_tokens: int, n_heads_q: int, head_dim: int, n_depth: int) -> int:
    """Bytes of device workspace one backward call with these sizes needs."""
    n = lib().moda_attn_bwd_workspace_size(total_tokens, n_heads_q, head_dim, n_depth)
    if n < 0:
        raise ValueError("invalid backward sizes")
    return int(n)


def attn_bwd(
    q,
    k,
    v,
    k_depth,
    v_depth,
    out,
    dout,
    lse,
    n_depth: Optional[int] = None,
    causal: bool = True,
    scale: Optional[float] = None,
    cu_seqlens=None,
    max_seqlen: Optional[int] = None,
    grads=None,
    workspace=None,
    stream=None,
):
    """Backward of ``attn_fwd`` through the C ABI. ``out`` and ``lse`` are the
    forward's results, ``dout`` the gradient of ``out`` (same dtype as out: the
    gradient dtype). Returns (dq, dk, dv, dk_depth, dv_depth) in that dtype, laid
    out like q, k, v, k_depth, v_depth (dk_depth/dv_depth None without depth
    tensors). Slots [n_depth, S_cap) of the depth gradients are zero when this
    function allocates them, and left untouched in a caller's ``grads``, a
    tuple of five preallocated tensors, and ``workspace`` (a uint8 device tensor of
    ``bwd_workspace_size`` bytes) make the call allocation-free. Packed calls need
    ``max_seqlen``."""
    import torch

    varlen = cu_seqlens is not None
    lead = 1 if varlen else 2
    ts = (q, k, v, k_depth, v_depth, out, dout, lse, cu_seqlens, workspace) + tuple(grads or ())
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if t is not None and t.device.type != "cuda":
            raise ValueError("all tensors must be on the GPU")
    if q.dim() != lead + 2 or k.shape != v.shape or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != q.shape[-1]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out.shape != q.shape or dout.shape != q.shape or out.dtype != dout.dtype:
        raise ValueError("out and dout must have q's shape and one dtype")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    d, Hq, Hkv = q.shape[-1], q.shape[-2], k.shape[-2]
    if k_depth is not None:
        if v_depth is None or k_depth.shape != v_depth.shape or k_depth.dim() != lead + 3:
            raise ValueError("k_depth and v_depth must both be [..., S_cap, Hkv, d]")
        if k_depth.shape[:lead] != q.shape[:lead] or k_depth.shape[-2:] != (Hkv, d):
            raise ValueError(f"depth tensors must be [..., S_cap, Hkv, d], got {tuple(k_depth.shape)}")
        if k_depth.dtype != q.dtype or v_depth.dtype != q.dtype:
            raise TypeError("depth tensors must share q's dtype")
        s_cap = k_depth.shape[lead]
    else:
        s_cap = 0
    if n_depth is None:
        n_depth = s_cap
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    N = q.shape[0] if varlen else q.shape[0] * q.shape[1]
    lse_shape = (Hq, N) if varlen else (q.shape[0], Hq, q.shape[1])
    if lse is None or tuple(lse.shape) != lse_shape or lse.dtype != torch.float32:
        raise ValueError(f"lse must be the forward's float32 {lse_shape}")
    gdt = out.dtype
    if grads is None:
        # the library never writes slots [n_depth, S_cap): their gradient is zero
        grads = (torch.empty_like(q, dtype=gdt), torch.empty_like(k, dtype=gdt), torch.empty_like(v, dtype=gdt),
                 None if k_depth is None else torch.zeros_like(k_depth, dtype=gdt),
                 None if v_depth is None else torch.zeros_like(v_depth, dtype=gdt))
    dq, dk, dv, dkd, dvd = grads
    for g, ref in zip(grads, (q, k, v, k_depth, v_depth)):
        if (g is None) != (ref is None) or (g is not None and (g.shape != ref.shape or g.dtype != gdt)):
            raise ValueError("grads must match q, k, v, k_depth, v_depth in shape, in out's dtype")
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_size(N, Hq, d, int(n_depth)), 256), dtype=torch.uint8,
                                device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    code, gcode = _dtype_code(q), _dtype_code(out)
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(k_depth), _ptr(v_depth), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dkd), _ptr(dvd))
    wsb = workspace.numel() * workspace.element_size()
    L = lib()
    if varlen:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 device tensor")
        n_seqs = cu_seqlens.numel() - 1
        if max_seqlen is None:
            raise ValueError("packed calls need max_seqlen (the longest sequence); cu_seqlens stays on the device")
        status = L.moda_attn_bwd_varlen(*ptrs, code, gcode, _ptr(cu_seqlens), n_seqs, N, int(max_seqlen), Hq, Hkv, d,
                                        s_cap, int(n_depth), int(bool(causal)), float(scale), _ptr(workspace), wsb,
                                        stream)
    else:
        status = L.moda_attn_bwd(*ptrs, code, gcode, q.shape[0], q.shape[1], Hq, Hkv, d, s_cap, int(n_depth),
                                 int(bool(causal)), float(scale), _ptr(workspace), wsb, stream)
    _check(status)
    return dq, dk, dv, dkd, dvd


def depth_kv_write(k_src, v_src, k_depth, v_depth, slot: int, stream=None):
    """Store k_src/v_src ([B,T,Hkv,d] or [N,Hkv,d]) into slot ``slot`` of the depth
    cache k_depth/v_depth ([B,T,S_cap,Hkv,d] or [N,S_cap,Hkv,d]) in place. For a
    bounded slot buffer pass slot = w % S_cap for the w-th entry written."""
    import torch

    for t in (k_src, v_src, k_depth, v_depth):
        if not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("all tensors must be contiguous GPU tensors")
    if k_src.shape != v_src.shape or k_depth.shape != v_depth.shape:
        raise ValueError("k and v tensors must match in shape")
    lead = k_src.dim() - 2
    if k_depth.dim() != lead + 3 or k_depth.shape[:lead] != k_src.shape[:lead] or k_depth.shape[-2:] != k_src.shape[-2:]:
        raise ValueError(f"depth cache must be [..., S_cap, Hkv, d] for sources {tuple(k_src.shape)}")
    if len({t.dtype for t in (k_src, v_src, k_depth, v_depth)}) != 1:
        raise TypeError("all tensors must share one dtype")
    n = 1
    for x in k_src.shape[:lead]:
        n *= x
    if stream is None:
        stream = torch.cuda.current_stream(k_src.device).cuda_stream
    _check(lib().moda_depth_kv_write(_ptr(k_src), _ptr(v_src), _ptr(k_depth), _ptr(v_depth), _dtype_code(k_src), n,
                                     k_src.shape[-2], k_src.shape[-1], k_depth.shape[lead], int(slot), stream))
    return k_depth, v_depth


def depth_kv_project(x, w_kv, k_depth, v_depth, slot: int, stream=None):
    """Project the FFN input into one depth slot in place: x [N, D_model] (or
    [B, T, D_model]), w_kv [2*Hkv*d, D_model] (key rows, then value rows: the
    [out, in] layout of a linear layer), k_depth/v_depth [N, S_cap, Hkv, d] (or
    [B, T, S_cap, Hkv, d]); slot ``slot`` of every token receives x W_k^T and x W_v^T."""
    import torch

    for t in (x, w_kv, k_depth, v_depth):
        if not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("all tensors must be contiguous GPU tensors")
    if k_depth.shape != v_depth.shape:
        raise ValueError("k_depth and v_depth must match in shape")
    lead = x.dim() - 1
    if k_depth.dim() != lead + 3 or k_depth.shape[:lead] != x.shape[:lead]:
        raise ValueError(f"depth cache must be [..., S_cap, Hkv, d] for x {tuple(x.shape)}")
    s_cap, hkv, d = k_depth.shape[lead:]
    if w_kv.dim() != 2 or tuple(w_kv.shape) != (2 * hkv * d, x.shape[-1]):
        raise ValueError(f"w_kv must be [2*Hkv*d, D_model] = {(2 * hkv * d, x.shape[-1])}")
    if len({t.dtype for t in (x, w_kv, k_depth, v_depth)}) != 1:
        raise TypeError("all tensors must share one dtype")
    n = 1
    for s in x.shape[:lead]:
        n *= s
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(lib().moda_depth_kv_project(_ptr(x), _ptr(w_kv), _ptr(k_depth), _ptr(v_depth), _dtype_code(x), n,
                                       x.shape[-1], hkv, d, s_cap, int(slot), stream))
    return k_depth, v_depth
