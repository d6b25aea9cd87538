"""ncattn: QK-norm + RoPE + causal sliding-window GQA attention for MI355X (gfx950).

Thin Python binding over the C-ABI library ``libncattn.so`` (declared in
``include/ncattn.h``).  This module only marshals arguments: it checks tensor
dtypes/devices/shapes, allocates outputs and workspace with torch, and passes
raw device pointers plus torch's current HIP stream to the library.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is missing or cannot be loaded every call raises.

Functions (names follow the C ABI):
    qknorm_rope_(q, k, pos_offset=None, rope_base=1e5, eps=1e-6, qk_gain=1.0)
    fwd(q, k, v, window=(-1, 0), softmax_scale=None) -> (o, lse)
    bwd(q, k, v, o, lse, do, window=(-1, 0), softmax_scale=None) -> (dq, dk, dv)
    decode(q, k_new, v_new, k_cache, v_cache, cache_seqlens, window=-1,
           softmax_scale=None, return_lse=False) -> o  (or (o, lse))
    decode_noalloc(q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse=None,
                   window=-1, softmax_scale=None)  (no workspace; outputs given)
    window_sizes(pattern, n_layer, short_window, long_window=-1) -> [(left, 0), ...]
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["qknorm_rope_", "qknorm_rope_rstd_", "rstd_like", "qknorm_rope_bwd_", "fwd", "fwd_qknorm_rope_", "bwd", "bwd_qknorm_rope", "decode", "decode_noalloc", "prefill",
           "cache_replicate",
           "window_sizes", "lib", "NcattnError", "LIB_PATH",
           "BF16", "F32", "STATUS", "bwd_workspace", "decode_workspace", "BWD_STAGES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libncattn.so")
BF16, F32 = 0, 1
STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}

_lib = None


class NcattnError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with {STATUS.get(code, code)}: {msg}")
        self.code = code


def lib():
    """The loaded ctypes handle of libncattn.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"ncattn: {LIB_PATH} is not built; run "
                          f"`python -m transformer_attention_qknorm_amd._build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.ncattn_qknorm_rope.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, f32, f32, f32, i32, vp]
    L.ncattn_qknorm_rope_bwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, f32, f32, f32, i32, vp]
    L.ncattn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.ncattn_qknorm_rope_rstd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, f32, f32, f32, i32, vp]
    L.ncattn_fwd_fp8.argtypes = [vp, vp, vp, f32, f32, f32, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
    L.ncattn_fwd_qknorm_rope.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, f32, f32, f32, i32, i32,
                                         f32, i32, vp]
    L.ncattn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.ncattn_bwd_workspace_bytes.restype = sz
    L.ncattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                             vp, sz, vp]
    for fn in ("ncattn_bwd_preprocess", "ncattn_bwd_dkdv", "ncattn_bwd_dq"):
        getattr(L, fn).argtypes = L.ncattn_bwd.argtypes
        getattr(L, fn).restype = i32
    L.ncattn_bwd_qknorm_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, f32, vp, vp, vp, i32, i32, i32, i32,
                                         i32, i32, i32, f32, i32, vp, sz, vp]
    L.ncattn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.ncattn_decode_workspace_bytes.restype = sz
    L.ncattn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    L.ncattn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.ncattn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    L.ncattn_cache_replicate.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.ncattn_last_error.restype = ctypes.c_char_p
    L.ncattn_version.restype = ctypes.c_char_p
    for fn in ("ncattn_qknorm_rope", "ncattn_qknorm_rope_bwd", "ncattn_fwd", "ncattn_fwd_qknorm_rope", "ncattn_bwd",
               "ncattn_bwd_qknorm_rope", "ncattn_qknorm_rope_rstd", "ncattn_fwd_fp8",
               "ncattn_decode", "ncattn_decode_noalloc",
               "ncattn_prefill", "ncattn_cache_replicate"):
        getattr(L, fn).restype = i32
    _lib = L
    return L


def _check(fn, rc):
    if rc != 0:
        raise NcattnError(fn, rc, lib().ncattn_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"ncattn: unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("ncattn: tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("ncattn: tensors must be contiguous")
    dev = ts[0].device
    if any(t.device != dev for t in ts):
        raise ValueError("ncattn: tensors must share one device")
    return dev


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _window(window):
    if isinstance(window, int):
        return window, 0
    wl, wr = window
    return int(wl), int(wr)


def _scale(softmax_scale):
    return 0.0 if softmax_scale is None else float(softmax_scale)


def _qk_shapes(fn, q, k, pos_offset):
    dev = _dev(q, k)
    if q.dtype != k.dtype or q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"ncattn.{fn}: q and k must be 4-D tensors of one dtype")
    B, T, H, D = q.shape
    if k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError(f"ncattn.{fn}: k must be [B][T][n_kv_head][D] matching q")
    if pos_offset is not None:
        _dev(pos_offset)
        if pos_offset.dtype != torch.int32 or pos_offset.numel() != B:
            raise ValueError(f"ncattn.{fn}: pos_offset must be int32 [B]")
    return dev, B, T, H, k.shape[2], D


def rstd_like(q, k):
    """An fp32 [B][T][n_head + n_kv_head] tensor for the rows' 1/r."""
    return torch.empty((q.shape[0], q.shape[1], q.shape[2] + k.shape[2]), dtype=torch.float32, device=q.device)


def _check_rstd(fn, rstd, q, k):
    _dev(rstd)
    if rstd.dtype != torch.float32 or tuple(rstd.shape) != (q.shape[0], q.shape[1], q.shape[2] + k.shape[2]) \
            or not rstd.is_contiguous():
        raise ValueError(f"ncattn.{fn}: rstd must be contiguous fp32 [B][T][n_head + n_kv_head]")


def qknorm_rope_(q, k, pos_offset=None, rope_base=100000.0, eps=1e-6, qk_gain=1.0):
    """In-place QK-norm + RoPE of q [B][T][H][D] and k [B][T][KV][D]; returns (q, k)."""
    dev, B, T, H, KV, D = _qk_shapes("qknorm_rope_", q, k, pos_offset)
    with torch.cuda.device(dev):
        rc = lib().ncattn_qknorm_rope(_ptr(q), _ptr(k), B, T, H, KV, D, _ptr(pos_offset),
                                      float(rope_base), float(eps), float(qk_gain), _dtype_code(q), _stream(dev))
    _check("ncattn_qknorm_rope", rc)
    return q, k


def qknorm_rope_rstd_(q, k, pos_offset=None, rope_base=100000.0, eps=1e-6, qk_gain=1.0, rstd=None):
    """qknorm_rope_ that also returns each row's 1/r (fp32 [B][T][H + KV], q rows
    first), what bwd_qknorm_rope needs instead of the raw rows; returns (q, k, rstd)."""
    dev, B, T, H, KV, D = _qk_shapes("qknorm_rope_rstd_", q, k, pos_offset)
    rstd = rstd_like(q, k) if rstd is None else rstd
    _check_rstd("qknorm_rope_rstd_", rstd, q, k)
    with torch.cuda.device(dev):
        rc = lib().ncattn_qknorm_rope_rstd(_ptr(q), _ptr(k), _ptr(rstd), B, T, H, KV, D, _ptr(pos_offset),
                                           float(rope_base), float(eps), float(qk_gain), _dtype_code(q), _stream(dev))
    _check("ncattn_qknorm_rope_rstd", rc)
    return q, k, rstd


def qknorm_rope_bwd_(dq, dk, q, k, pos_offset=None, rope_base=100000.0, eps=1e-6, qk_gain=1.0):
    """Backward of qknorm_rope_, in place: dq, dk hold the gradients of its outputs
    on entry and those of its inputs on return; q, k are its inputs (before
    normalisation, untouched).  Returns (dq, dk)."""
    dev = _dev(dq, dk, q, k)
    if q.dim() != 4 or k.dim() != 4 or dq.shape != q.shape or dk.shape != k.shape \
            or len({dq.dtype, dk.dtype, q.dtype, k.dtype}) != 1:
        raise ValueError("ncattn.qknorm_rope_bwd_: dq, dk must match q, k (4-D, one dtype)")
    B, T, H, D = q.shape
    if k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError("ncattn.qknorm_rope_bwd_: k must be [B][T][n_kv_head][D] matching q")
    if pos_offset is not None:
        _dev(pos_offset)
        if pos_offset.dtype != torch.int32 or pos_offset.numel() != B:
            raise ValueError("ncattn.qknorm_rope_bwd_: pos_offset must be int32 [B]")
    with torch.cuda.device(dev):
        rc = lib().ncattn_qknorm_rope_bwd(_ptr(dq), _ptr(dk), _ptr(q), _ptr(k), B, T, H, k.shape[2], D,
                                          _ptr(pos_offset), float(rope_base), float(eps), float(qk_gain),
                                          _dtype_code(q), _stream(dev))
    _check("ncattn_qknorm_rope_bwd", rc)
    return dq, dk


def fwd(q, k, v, window=(-1, 0), softmax_scale=None, out=None):
    """Attention forward: returns (o [B][T][H][D], lse [B][H][T] fp32).
    ``out=(o, lse)`` reuses preallocated outputs."""
    dev = _dev(q, k, v)
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D or q.dtype != k.dtype \
            or q.dtype != v.dtype:
        raise ValueError("ncattn.fwd: k, v must be [B][T][n_kv_head][D] of q's dtype")
    wl, wr = _window(window)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    else:
        o, lse = out
        _dev(o, lse)
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H, T) or lse.dtype != torch.float32:
            raise ValueError("ncattn.fwd: out must be (o like q, lse fp32 [B][H][T])")
    with torch.cuda.device(dev):
        rc = lib().ncattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, H, k.shape[2], D, wl, wr,
                              _scale(softmax_scale), _dtype_code(q), _stream(dev))
    _check("ncattn_fwd", rc)
    return o, lse


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, window=(-1, 0), softmax_scale=None, out=None):
    """Attention forward on fp8 inputs: q [B][T][H][128], k, v [B][T][KV][128] as
    torch.float8_e4m3fn (OCP e4m3), each standing for its values times a per-tensor
    descale (positive floats).  Returns (o bf16 [B][T][H][128], lse fp32
    [B][H][T]); ``out=(o, lse)`` reuses preallocated outputs."""
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or q.dtype != torch.float8_e4m3fn or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("ncattn.fwd_fp8: q, k, v must be 4-D torch.float8_e4m3fn")
    B, T, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError("ncattn.fwd_fp8: k, v must be [B][T][n_kv_head][D] matching q")
    wl, wr = _window(window)
    if out is None:
        o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    else:
        o, lse = out
        _dev(o, lse)
        if o.shape != q.shape or o.dtype != torch.bfloat16 or lse.shape != (B, H, T) or lse.dtype != torch.float32:
            raise ValueError("ncattn.fwd_fp8: out must be (o bf16 shaped like q, lse fp32 [B][H][T])")
    with torch.cuda.device(dev):
        rc = lib().ncattn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), float(q_descale), float(k_descale), float(v_descale),
                                  _ptr(o), _ptr(lse), B, T, H, k.shape[2], D, wl, wr, _scale(softmax_scale),
                                  _stream(dev))
    _check("ncattn_fwd_fp8", rc)
    return o, lse


def fwd_qknorm_rope_(q, k, v, pos_offset=None, rope_base=100000.0, eps=1e-6, qk_gain=1.0, window=(-1, 0),
                     softmax_scale=None, out=None, rstd=None):
    """QK-norm + RoPE of q and k, in place, fused with the attention forward:
    the same as qknorm_rope_(q, k, ...) then fwd(q, k, v, ...).  Returns (o, lse).
    ``rstd`` (fp32 [B][T][H + KV], see rstd_like) also receives each row's 1/r."""
    dev = _dev(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or len({q.dtype, k.dtype, v.dtype}) != 1:
        raise ValueError("ncattn.fwd_qknorm_rope_: q, k, v must be 4-D of one dtype, k and v alike")
    B, T, H, D = q.shape
    if k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError("ncattn.fwd_qknorm_rope_: k, v must be [B][T][n_kv_head][D] matching q")
    if pos_offset is not None:
        _dev(pos_offset)
        if pos_offset.dtype != torch.int32 or pos_offset.numel() != B:
            raise ValueError("ncattn.fwd_qknorm_rope_: pos_offset must be int32 [B]")
    wl, wr = _window(window)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    else:
        o, lse = out
        _dev(o, lse)
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H, T) or lse.dtype != torch.float32:
            raise ValueError("ncattn.fwd_qknorm_rope_: out must be (o like q, lse fp32 [B][H][T])")
    if rstd is not None:
        _check_rstd("fwd_qknorm_rope_", rstd, q, k)
    with torch.cuda.device(dev):
        rc = lib().ncattn_fwd_qknorm_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(rstd), B, T, H,
                                          k.shape[2], D,
                                          _ptr(pos_offset), float(rope_base), float(eps), float(qk_gain), wl, wr,
                                          _scale(softmax_scale), _dtype_code(q), _stream(dev))
    _check("ncattn_fwd_qknorm_rope", rc)
    return o, lse


BWD_STAGES = {None: "ncattn_bwd", "preprocess": "ncattn_bwd_preprocess", "dkdv": "ncattn_bwd_dkdv",
              "dq": "ncattn_bwd_dq"}


def bwd_workspace(q, k, window=(-1, 0)):
    """A workspace tensor large enough for bwd() on these shapes and window."""
    B, T, H, D = q.shape
    n = lib().ncattn_bwd_workspace_bytes(B, T, H, k.shape[2], D, _window(window)[0], _dtype_code(q))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def bwd(q, k, v, o, lse, do, window=(-1, 0), softmax_scale=None, out=None, workspace=None, stage=None):
    """Attention backward: returns (dq, dk, dv).

    ``out=(dq, dk, dv)`` and ``workspace`` reuse preallocated buffers; ``stage``
    ("preprocess", "dkdv" or "dq") enqueues only that stage of the backward (the
    three in that order, with one workspace, equal the full call)."""
    dev = _dev(q, k, v, o, lse, do)
    B, T, H, D = q.shape
    KV = k.shape[2]
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, H, T) or lse.dtype != torch.float32:
        raise ValueError("ncattn.bwd: o, do must match q and lse must be fp32 [B][H][T]")
    if k.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype or q.dtype != o.dtype or q.dtype != do.dtype:
        raise ValueError("ncattn.bwd: inconsistent shapes or dtypes")
    if stage not in BWD_STAGES:
        raise ValueError(f"ncattn.bwd: unknown stage {stage!r}")
    wl, wr = _window(window)
    dt = _dtype_code(q)
    ws = bwd_workspace(q, k, (wl, wr)) if workspace is None else workspace
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _dev(dq, dk, dv, ws)
        if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
            raise ValueError("ncattn.bwd: out must be (dq like q, dk like k, dv like v)")
    fn = getattr(lib(), BWD_STAGES[stage])
    with torch.cuda.device(dev):
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                B, T, H, KV, D, wl, wr, _scale(softmax_scale), dt, _ptr(ws), ws.numel(), _stream(dev))
    _check(BWD_STAGES[stage], rc)
    return dq, dk, dv


def bwd_qknorm_rope(q, k, v, o, lse, do, rstd, pos_offset=None, rope_base=100000.0, qk_gain=1.0, window=(-1, 0),
                    softmax_scale=None, out=None, workspace=None):
    """The backward of QK-norm + RoPE followed by attention, in one call: returns
    (dq, dk, dv) with dq, dk the gradients of the raw (pre-norm) rows.  q, k are
    the post-norm rows the forward attended with and rstd their 1/r as
    qknorm_rope_rstd_ or fwd_qknorm_rope_ stored it.  ``out`` and ``workspace``
    reuse preallocated buffers."""
    dev = _dev(q, k, v, o, lse, do)
    B, T, H, D = q.shape
    KV = k.shape[2]
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, H, T) or lse.dtype != torch.float32:
        raise ValueError("ncattn.bwd_qknorm_rope: o, do must match q and lse must be fp32 [B][H][T]")
    if k.shape != v.shape or len({q.dtype, k.dtype, v.dtype, o.dtype, do.dtype}) != 1:
        raise ValueError("ncattn.bwd_qknorm_rope: inconsistent shapes or dtypes")
    _check_rstd("bwd_qknorm_rope", rstd, q, k)
    if pos_offset is not None:
        _dev(pos_offset)
        if pos_offset.dtype != torch.int32 or pos_offset.numel() != B:
            raise ValueError("ncattn.bwd_qknorm_rope: pos_offset must be int32 [B]")
    wl, wr = _window(window)
    ws = bwd_workspace(q, k, (wl, wr)) if workspace is None else workspace
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _dev(dq, dk, dv, ws)
        if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
            raise ValueError("ncattn.bwd_qknorm_rope: out must be (dq like q, dk like k, dv like v)")
    with torch.cuda.device(dev):
        rc = lib().ncattn_bwd_qknorm_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(rstd),
                                          _ptr(pos_offset), float(rope_base), float(qk_gain), _ptr(dq), _ptr(dk),
                                          _ptr(dv), B, T, H, KV, D, wl, wr, _scale(softmax_scale), _dtype_code(q),
                                          _ptr(ws), ws.numel(), _stream(dev))
    _check("ncattn_bwd_qknorm_rope", rc)
    return dq, dk, dv


def decode_workspace(q, k_cache, window=-1):
    """A workspace tensor large enough for decode() on these shapes and window."""
    B, _, H, D = q.shape
    wl = window if isinstance(window, int) else _window(window)[0]
    n = lib().ncattn_decode_workspace_bytes(B, k_cache.shape[1], H, k_cache.shape[2], D, wl)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def decode(q, k_new, v_new, k_cache, v_cache, cache_seqlens, window=-1, softmax_scale=None, return_lse=False,
           out=None, workspace=None):
    """Single-token decode; writes k_new/v_new into cache slot cache_seqlens[b] in place.

    q [B][1][H][D], k_new/v_new [B][1][KV][D], caches [B][T_max][KV][D] (bf16),
    cache_seqlens int32 [B] (not advanced).  Returns o [B][1][H][D] (and lse [B][H]).
    """
    dev = _dev(q, k_new, v_new, k_cache, v_cache, cache_seqlens)
    B, one, H, D = q.shape
    T_max, KV = k_cache.shape[1], k_cache.shape[2]
    if one != 1 or k_new.shape != (B, 1, KV, D) or v_new.shape != (B, 1, KV, D) \
            or k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("ncattn.decode: inconsistent shapes")
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.numel() != B:
        raise ValueError("ncattn.decode: cache_seqlens must be int32 [B]")
    wl = window if isinstance(window, int) else _window(window)[0]
    dt = _dtype_code(q)
    L = lib()
    ws = decode_workspace(q, k_cache, wl) if workspace is None else workspace
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev) if return_lse else None
    else:
        o, lse = out if isinstance(out, tuple) else (out, None)
        _dev(o)
        if o.shape != q.shape or o.dtype != q.dtype:
            raise ValueError("ncattn.decode: out must be like q")
    with torch.cuda.device(dev):
        rc = L.ncattn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                             _ptr(o), _ptr(lse), B, T_max, H, KV, D, wl, _scale(softmax_scale), dt, _ptr(ws),
                             ws.numel(), _stream(dev))
    _check("ncattn_decode", rc)
    return (o, lse) if return_lse else o


DECODE_SCRATCH_BYTES = 32 << 20  # NCATTN_DECODE_SCRATCH_BYTES


def decode_noalloc(q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse=None, window=-1, softmax_scale=None):
    """decode() through ncattn_decode_noalloc: no workspace, the split-KV partials
    go to the library's per-device scratch (at most DECODE_SCRATCH_BYTES); the
    outputs o [B][1][H][D] (and optionally lse fp32 [B][H]) are given by the
    caller, so nothing is allocated.  Calls on one device must not overlap."""
    dev = _dev(q, k_new, v_new, k_cache, v_cache, cache_seqlens, o)
    B, one, H, D = q.shape
    T_max, KV = k_cache.shape[1], k_cache.shape[2]
    if one != 1 or k_new.shape != (B, 1, KV, D) or v_new.shape != (B, 1, KV, D) \
            or k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("ncattn.decode_noalloc: inconsistent shapes")
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.numel() != B:
        raise ValueError("ncattn.decode_noalloc: cache_seqlens must be int32 [B]")
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("ncattn.decode_noalloc: o must be like q")
    if lse is not None:
        _dev(lse)
        if lse.shape != (B, H) or lse.dtype != torch.float32:
            raise ValueError("ncattn.decode_noalloc: lse must be fp32 [B][H]")
    wl = window if isinstance(window, int) else _window(window)[0]
    with torch.cuda.device(dev):
        rc = lib().ncattn_decode_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(cache_seqlens), _ptr(o), _ptr(lse), B, T_max, H, KV, D, wl,
                                         _scale(softmax_scale), _dtype_code(q), _stream(dev))
    _check("ncattn_decode_noalloc", rc)
    return o


def prefill(q, k_new, v_new, k_cache, v_cache, cache_seqlens, window=-1, softmax_scale=None, return_lse=False,
            out=None):
    """Chunked prefill: writes the chunk k_new/v_new [B][Tn][KV][D] into cache rows
    cache_seqlens[b].. in place, then attends q [B][Tn][H][D] (positions
    cache_seqlens[b] + i) over the cache.  caches [B][T_max][KV][D] (bf16),
    cache_seqlens int32 [B] (not advanced).  Returns o [B][Tn][H][D] (and lse
    [B][H][Tn])."""
    dev = _dev(q, k_new, v_new, k_cache, v_cache, cache_seqlens)
    B, Tn, H, D = q.shape
    T_max, KV = k_cache.shape[1], k_cache.shape[2]
    if k_new.shape != (B, Tn, KV, D) or v_new.shape != (B, Tn, KV, D) or k_cache.shape != v_cache.shape \
            or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("ncattn.prefill: inconsistent shapes")
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.numel() != B:
        raise ValueError("ncattn.prefill: cache_seqlens must be int32 [B]")
    wl = window if isinstance(window, int) else _window(window)[0]
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Tn), dtype=torch.float32, device=dev) if return_lse else None
    else:
        o, lse = out if isinstance(out, tuple) else (out, None)
        _dev(o)
        if o.shape != q.shape or o.dtype != q.dtype:
            raise ValueError("ncattn.prefill: out must be like q")
    with torch.cuda.device(dev):
        rc = lib().ncattn_prefill(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(cache_seqlens), _ptr(o), _ptr(lse), B, Tn, T_max, H, KV, D, wl,
                                  _scale(softmax_scale), _dtype_code(q), _stream(dev))
    _check("ncattn_prefill", rc)
    return (o, lse) if return_lse else o


def cache_replicate(k_src, v_src, src_seqlen, k_dst, v_dst, dst_seqlens):
    """Copies the first src_seqlen[0] rows of a batch-1 cache k_src, v_src
    [1][T_src][KV][D] into every row of k_dst, v_dst [N][T_max][KV][D] and sets
    dst_seqlens [N] (int32) to that length, in place ("nanochat Admin & Developer
    Guide", section 7: prefill once, then copy the cache to the samples).  A
    length outside [0, T_src] copies nothing and sets dst_seqlens to -1."""
    dev = _dev(k_src, v_src, src_seqlen, k_dst, v_dst, dst_seqlens)
    if k_src.dim() != 4 or k_src.shape[0] != 1 or v_src.shape != k_src.shape:
        raise ValueError("ncattn.cache_replicate: sources must be [1][T_src][KV][D]")
    _, T_src, KV, D = k_src.shape
    if k_dst.dim() != 4 or v_dst.shape != k_dst.shape or k_dst.shape[2:] != (KV, D):
        raise ValueError("ncattn.cache_replicate: destinations must be [N][T_max][KV][D] like the sources")
    if k_dst.dtype != k_src.dtype or v_dst.dtype != k_src.dtype or v_src.dtype != k_src.dtype:
        raise ValueError("ncattn.cache_replicate: sources and destinations must share a dtype")
    N, T_max = k_dst.shape[0], k_dst.shape[1]
    if src_seqlen.dtype != torch.int32 or src_seqlen.numel() != 1:
        raise ValueError("ncattn.cache_replicate: src_seqlen must be int32 [1]")
    if dst_seqlens.dtype != torch.int32 or dst_seqlens.numel() != N:
        raise ValueError("ncattn.cache_replicate: dst_seqlens must be int32 [N]")
    with torch.cuda.device(dev):
        rc = lib().ncattn_cache_replicate(_ptr(k_src), _ptr(v_src), _ptr(src_seqlen), _ptr(k_dst), _ptr(v_dst),
                                          _ptr(dst_seqlens), N, T_src, T_max, KV, D, _dtype_code(k_src),
                                          _stream(dev))
    _check("ncattn_cache_replicate", rc)


def window_sizes(pattern, n_layer, short_window, long_window=-1):
    """Per-layer (left, right) windows from a pattern of 'S'/'L' tiled over the
    layers, the final layer always 'L' ("nanochat Admin & Developer Guide",
    section 3, "Sliding-window attention"); -1 means unbounded."""
    p = str(pattern).upper()
    if not p or set(p) - {"S", "L"}:
        raise ValueError("window pattern must be a non-empty string over {'S', 'L'}")
    sizes = [short_window if p[i % len(p)] == "S" else long_window for i in range(n_layer)]
    if n_layer:
        sizes[-1] = long_window
    return [(w, 0) for w in sizes]
