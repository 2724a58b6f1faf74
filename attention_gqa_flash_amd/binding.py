"""ctypes binding of libsinkattn.so (argument marshalling only).

Every step of the computation runs in the HIP library; this module checks
tensor dtypes/devices/shapes, allocates outputs with torch, and passes raw
device pointers and the current HIP stream across the C ABI declared in
include/sinkattn.h.  If the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsinkattn.so")
_lib = None

_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("sinkattn %s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


def library() -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SinkAttnError(-1, "%s is missing: build it with `python -m attention_gqa_flash_amd.build`"
                            % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.sinkattn_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                            vp, vp, vp]
    lib.sinkattn_prefill_varlen.restype = ctypes.c_int
    lib.sinkattn_prefill_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                            f32, vp, vp, vp]
    lib.sinkattn_prefill_append.restype = ctypes.c_int
    lib.sinkattn_prefill_append_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                                    i32, f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_prefill_append_splitkv.restype = ctypes.c_int
    lib.sinkattn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.sinkattn_decode_workspace_bytes.restype = sz
    lib.sinkattn_decode_splitkv.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, f32, i32,
                                            vp, sz, vp, vp, vp]
    lib.sinkattn_decode_splitkv.restype = ctypes.c_int
    lib.sinkattn_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, f32, i32, vp, vp,
                                                    vp]
    lib.sinkattn_decode_splitkv_noalloc.restype = ctypes.c_int
    lib.sinkattn_decode_splitkv_fp8.argtypes = [vp, vp, vp, f32, f32, vp, i32, i32, vp, i32, i32, i32, i32, f32,
                                                i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_splitkv_fp8.restype = ctypes.c_int
    lib.sinkattn_decode_splitkv_multi.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32, i32, i32,
                                                  f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_splitkv_multi.restype = ctypes.c_int
    lib.sinkattn_decode_paged.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, i32, i32, f32,
                                          i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_paged.restype = ctypes.c_int
    lib.sinkattn_decode_paged_fp8.argtypes = [vp, vp, vp, f32, f32, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32,
                                              i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_paged_fp8.restype = ctypes.c_int
    lib.sinkattn_prefill_append_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp,
                                                  i32, i32, i32, i32, f32, vp, vp, vp]
    lib.sinkattn_prefill_append_paged.restype = ctypes.c_int
    lib.sinkattn_prefill_append_paged_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                          vp, i32, i32, i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_prefill_append_paged_splitkv.restype = ctypes.c_int
    lib.sinkattn_decode_paged_multi.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, i32,
                                                i32, i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_paged_multi.restype = ctypes.c_int
    lib.sinkattn_decode_splitkv_multi_fp8.argtypes = [vp, vp, vp, f32, f32, vp, vp, i32, i32, i32, i32, vp, i32, i32,
                                                      i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_splitkv_multi_fp8.restype = ctypes.c_int
    lib.sinkattn_decode_paged_multi_fp8.argtypes = [vp, vp, vp, f32, f32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                    vp, i32, i32, i32, i32, f32, i32, vp, sz, vp, vp, vp]
    lib.sinkattn_decode_paged_multi_fp8.restype = ctypes.c_int
    f64 = ctypes.c_double
    lib.sinkattn_rope_qkv_append.argtypes = [vp, vp, vp, i32, i32, i32, i32, f64, f64, i32, f64, f64, i32, vp, vp, vp, i32,
                                             vp]
    lib.sinkattn_rope_qkv_append.restype = ctypes.c_int
    lib.sinkattn_oproj_bias.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.sinkattn_oproj_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sinkattn_oproj_workspace_bytes.restype = sz
    lib.sinkattn_oproj_bias.restype = ctypes.c_int
    lib.sinkattn_merge_lse.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.sinkattn_merge_lse.restype = ctypes.c_int
    lib.sinkattn_last_error.argtypes = []
    lib.sinkattn_last_error.restype = ctypes.c_char_p
    lib.sinkattn_version.argtypes = []
    lib.sinkattn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = library().sinkattn_last_error().decode()
        raise SinkAttnError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions (got %d)" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: Optional[torch.Tensor],
                   cu_seqlens: torch.Tensor, max_seqlen: int, window: int = 0, softmax_scale: float = 0.125,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   return_lse: bool = False):
    """Varlen prefill.  q [T, Hq, 64] bf16, k/v [T, Hkv, 64] bf16, sinks [Hq]
    fp32 or None, cu_seqlens [B+1] int32 (device).  Returns o (and lse)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    t, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (t, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out must match q")
    if return_lse and lse is None:
        lse = torch.empty((t, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
        if lse.shape != (t, hq):
            raise ValueError("lse must be [T, Hq]")
    _check(library().sinkattn_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens), cu_seqlens.shape[0] - 1,
        int(max_seqlen), t, hq, hkv, d, int(window), float(softmax_scale), _ptr(out), _ptr(lse),
        _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def prefill_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: Optional[torch.Tensor],
                   cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                   window: int = 0, softmax_scale: float = 0.125, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = False, num_splits: int = 1,
                   workspace: Optional[torch.Tensor] = None):
    """Append prefill / multi-token-query decode: q [Tq, Hq, 64] bf16 packed
    by cu_seqlens_q, k/v [Tk, Hkv, 64] bf16 packed by cu_seqlens_k (both
    [B+1] int32, device); each sequence's queries are its last tokens
    (bottom-right causal).  num_splits > 1 splits each query tile's keys
    (sinkattn_prefill_append_splitkv); ``workspace`` (uint8, device) is then
    allocated here when not given.  Returns o (and lse)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    if k.shape[2] != d or v.shape != k.shape:
        raise ValueError("k and v must be [Tk, Hkv, D] matching q")
    if cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3)
        if out.shape != q.shape:
            raise ValueError("out must match q")
    if return_lse and lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
        if lse.shape != (tq, hq):
            raise ValueError("lse must be [Tq, Hq]")
    if int(num_splits) > 1:
        need = decode_workspace_bytes(tq, hq, d, int(num_splits))
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(library().sinkattn_prefill_append_splitkv(
            _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            cu_seqlens_q.shape[0] - 1, int(max_seqlen_q), int(max_seqlen_k), tq, tk, hq, hkv, d, int(window),
            float(softmax_scale), int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
            _stream(q.device)))
    else:
        _check(library().sinkattn_prefill_append(
            _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            cu_seqlens_q.shape[0] - 1, int(max_seqlen_q), int(max_seqlen_k), tq, tk, hq, hkv, d, int(window),
            float(softmax_scale), _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(library().sinkattn_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits))


def decode_splitkv(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   cu_seqlens_k: torch.Tensor, max_seqlen_k: int, sinks: Optional[torch.Tensor],
                   window: int = 0, softmax_scale: float = 0.125, num_splits: int = 1,
                   workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Split-KV decode.  q [B, Hq, 64] bf16, k/v cache [Tk, Hkv, 64] bf16
    packed by cu_seqlens_k [B+1] int32.  ``workspace`` (uint8, device) is
    allocated here when needed and not given."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    bsz, hq, d = q.shape
    hkv = k_cache.shape[1]
    if v_cache.shape != k_cache.shape or k_cache.shape[2] != d:
        raise ValueError("k_cache and v_cache must be [Tk, Hkv, D] matching q")
    if cu_seqlens_k.shape[0] != bsz + 1:
        raise ValueError("cu_seqlens_k must have batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    need = decode_workspace_bytes(bsz, hq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    _check(library().sinkattn_decode_splitkv(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_k), bsz, int(max_seqlen_k), _ptr(sinks),
        hq, hkv, d, int(window), float(softmax_scale), int(num_splits), _ptr(workspace), ws_bytes,
        _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


NOALLOC_SCRATCH_BYTES = 32 << 20  # the static scratch of decode_splitkv_noalloc


def decode_splitkv_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           cu_seqlens_k: torch.Tensor, max_seqlen_k: int, sinks: Optional[torch.Tensor],
                           window: int = 0, softmax_scale: float = 0.125, num_splits: int = 1,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           return_lse: bool = False):
    """decode_splitkv without a workspace: the library's static per-device
    scratch holds the split partials (at most NOALLOC_SCRATCH_BYTES).  The
    call allocates nothing when ``out`` (and ``lse``, if wanted) are given."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    bsz, hq, d = q.shape
    hkv = k_cache.shape[1]
    if v_cache.shape != k_cache.shape or k_cache.shape[2] != d:
        raise ValueError("k_cache and v_cache must be [Tk, Hkv, D] matching q")
    if cu_seqlens_k.shape[0] != bsz + 1:
        raise ValueError("cu_seqlens_k must have batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    _check(library().sinkattn_decode_splitkv_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_k), bsz, int(max_seqlen_k), _ptr(sinks),
        hq, hkv, d, int(window), float(softmax_scale), int(num_splits), _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_splitkv_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float,
                       v_scale: float, cu_seqlens_k: torch.Tensor, max_seqlen_k: int, sinks: Optional[torch.Tensor],
                       window: int = 0, softmax_scale: float = 0.125, num_splits: int = 1,
                       workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Split-KV decode against an E4M3 cache.  q [B, Hq, 64] bf16; k/v cache
    [Tk, Hkv, 64] uint8 E4M3 codes (K = k_scale * e4m3(code), V likewise)
    packed by cu_seqlens_k [B+1] int32."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.uint8, 3)
    _need(v_cache, "v_cache", torch.uint8, 3)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    bsz, hq, d = q.shape
    hkv = k_cache.shape[1]
    if v_cache.shape != k_cache.shape or k_cache.shape[2] != d:
        raise ValueError("k_cache and v_cache must be [Tk, Hkv, D] matching q")
    if cu_seqlens_k.shape[0] != bsz + 1:
        raise ValueError("cu_seqlens_k must have batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    need = decode_workspace_bytes(bsz, hq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    _check(library().sinkattn_decode_splitkv_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale), _ptr(cu_seqlens_k), bsz,
        int(max_seqlen_k), _ptr(sinks), hq, hkv, d, int(window), float(softmax_scale), int(num_splits),
        _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_splitkv_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                         sinks: Optional[torch.Tensor], window: int = 0, softmax_scale: float = 0.125,
                         num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = False):
    """Multi-token-query split-KV decode: q [Tq, Hq, 64] bf16 packed by
    cu_seqlens_q, caches [Tk, Hkv, 64] bf16 packed by cu_seqlens_k; each
    sequence's queries are its newest tokens (bottom-right causal)."""
    return _decode_multi(q, k_cache, v_cache, None, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sinks,
                         window, softmax_scale, num_splits, workspace, out, lse, return_lse)


def decode_splitkv_multi_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float,
                             v_scale: float, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                             max_seqlen_k: int, sinks: Optional[torch.Tensor], window: int = 0,
                             softmax_scale: float = 0.125, num_splits: int = 1,
                             workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """decode_splitkv_multi against an E4M3 cache: k/v uint8 codes
    [Tk, Hkv, 64], K = k_scale * e4m3(code), V = v_scale * e4m3(code)."""
    return _decode_multi(q, k_cache, v_cache, (k_scale, v_scale), cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                         max_seqlen_k, sinks, window, softmax_scale, num_splits, workspace, out, lse, return_lse)


def _decode_multi(q, k_cache, v_cache, scales, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, sinks, window,
                  softmax_scale, num_splits, workspace, out, lse, return_lse):
    _need(q, "q", torch.bfloat16, 3)
    kv_dtype = torch.bfloat16 if scales is None else torch.uint8
    _need(k_cache, "k_cache", kv_dtype, 3)
    _need(v_cache, "v_cache", kv_dtype, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    tq, hq, d = q.shape
    hkv = k_cache.shape[1]
    if v_cache.shape != k_cache.shape or k_cache.shape[2] != d:
        raise ValueError("k_cache and v_cache must be [Tk, Hkv, D] matching q")
    if cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    need = decode_workspace_bytes(tq, hq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    tail = (_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.shape[0] - 1, int(max_seqlen_q), int(max_seqlen_k),
            tq, _ptr(sinks), hq, hkv, d, int(window), float(softmax_scale), int(num_splits), _ptr(workspace),
            ws_bytes, _ptr(out), _ptr(lse), _stream(q.device))
    if scales is None:
        _check(library().sinkattn_decode_splitkv_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), *tail))
    else:
        _check(library().sinkattn_decode_splitkv_multi_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(scales[0]),
                                                           float(scales[1]), *tail))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, max_seqlen_k: int, sinks: Optional[torch.Tensor], window: int = 0,
                 softmax_scale: float = 0.125, num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Split-KV decode against a paged cache: q [B, Hq, 64] bf16; k/v pages
    [P, page_size, Hkv, 64] bf16; block_table [B, max_pages] int32;
    seq_lens [B] int32 (all device)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    bsz, hq, d = q.shape
    num_pages, page_size, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if v_pages.shape != k_pages.shape or k_pages.shape[3] != d:
        raise ValueError("k_pages and v_pages must be [P, page_size, Hkv, D] matching q")
    if block_table.shape[0] != bsz or seq_lens.shape[0] != bsz:
        raise ValueError("block_table and seq_lens need one row / entry per sequence")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    need = decode_workspace_bytes(bsz, hq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    _check(library().sinkattn_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), bsz, block_table.shape[1],
        page_size, num_pages, int(max_seqlen_k), _ptr(sinks), hq, hkv, d, int(window), float(softmax_scale),
        int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_paged_fp8(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, k_scale: float, v_scale: float,
                     block_table: torch.Tensor, seq_lens: torch.Tensor, max_seqlen_k: int,
                     sinks: Optional[torch.Tensor], window: int = 0, softmax_scale: float = 0.125,
                     num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = False):
    """Split-KV decode against a paged FP8 cache: q [B, Hq, 64] bf16; k/v
    pages [P, page_size, Hkv, 64] uint8 E4M3 codes with host scales;
    block_table [B, max_pages] int32; seq_lens [B] int32 (all device)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.uint8, 4)
    _need(v_pages, "v_pages", torch.uint8, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    bsz, hq, d = q.shape
    num_pages, page_size, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if v_pages.shape != k_pages.shape or k_pages.shape[3] != d:
        raise ValueError("k_pages and v_pages must be [P, page_size, Hkv, D] matching q")
    if block_table.shape[0] != bsz or seq_lens.shape[0] != bsz:
        raise ValueError("block_table and seq_lens need one row / entry per sequence")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    need = decode_workspace_bytes(bsz, hq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    _check(library().sinkattn_decode_paged_fp8(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), float(k_scale), float(v_scale), _ptr(block_table), _ptr(seq_lens), bsz,
        block_table.shape[1], page_size, num_pages, int(max_seqlen_k), _ptr(sinks), hq, hkv, d, int(window),
        float(softmax_scale), int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def prefill_append_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                         seq_lens_k: torch.Tensor, cu_seqlens_q: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                         sinks: Optional[torch.Tensor], window: int = 0, softmax_scale: float = 0.125,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         return_lse: bool = False, num_splits: int = 1, workspace: Optional[torch.Tensor] = None):
    """Append (chunked) prefill against a paged cache: q [Tq, Hq, 64] bf16
    packed by cu_seqlens_q; k/v pages [P, page_size, Hkv, 64] bf16;
    block_table [B, max_pages] int32; seq_lens_k [B] int32 (all device).
    num_splits > 1 splits each query tile's keys
    (sinkattn_prefill_append_paged_splitkv; ``workspace`` allocated here when
    not given)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens_k, "seq_lens_k", torch.int32, 1)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    tq, hq, d = q.shape
    bsz = seq_lens_k.shape[0]
    num_pages, page_size, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if v_pages.shape != k_pages.shape or k_pages.shape[3] != d:
        raise ValueError("k_pages and v_pages must be [P, page_size, Hkv, D] matching q")
    if block_table.shape[0] != bsz or cu_seqlens_q.shape[0] != bsz + 1:
        raise ValueError("block_table needs one row per sequence and cu_seqlens_q batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    if int(num_splits) > 1:
        if workspace is None:
            workspace = torch.empty(decode_workspace_bytes(tq, hq, d, int(num_splits)), dtype=torch.uint8,
                                    device=q.device)
        _check(library().sinkattn_prefill_append_paged_splitkv(
            _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens_k), _ptr(cu_seqlens_q), bsz,
            block_table.shape[1], page_size, num_pages, int(max_seqlen_q), int(max_seqlen_k), tq, _ptr(sinks), hq,
            hkv, d, int(window), float(softmax_scale), int(num_splits), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(q.device)))
    else:
        _check(library().sinkattn_prefill_append_paged(
            _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens_k), _ptr(cu_seqlens_q), bsz,
            block_table.shape[1], page_size, num_pages, int(max_seqlen_q), int(max_seqlen_k), tq, _ptr(sinks), hq,
            hkv, d, int(window), float(softmax_scale), _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def decode_paged_multi(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                       seq_lens: torch.Tensor, cu_seqlens_q: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                       sinks: Optional[torch.Tensor], window: int = 0, softmax_scale: float = 0.125,
                       num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       return_lse: bool = False):
    """Multi-token-query decode against a paged cache: q [Tq, Hq, 64] bf16
    packed by cu_seqlens_q; k/v pages [P, page_size, Hkv, 64] bf16;
    block_table [B, max_pages] int32; seq_lens [B] int32 (all device)."""
    return _decode_paged_multi(q, k_pages, v_pages, None, block_table, seq_lens, cu_seqlens_q, max_seqlen_q,
                               max_seqlen_k, sinks, window, softmax_scale, num_splits, workspace, out, lse, return_lse)


def decode_paged_multi_fp8(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, k_scale: float,
                           v_scale: float, block_table: torch.Tensor, seq_lens: torch.Tensor,
                           cu_seqlens_q: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                           sinks: Optional[torch.Tensor], window: int = 0, softmax_scale: float = 0.125,
                           num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           return_lse: bool = False):
    """decode_paged_multi over pages of E4M3 codes (uint8 [P, page_size,
    Hkv, 64]) with per-tensor scales."""
    return _decode_paged_multi(q, k_pages, v_pages, (k_scale, v_scale), block_table, seq_lens, cu_seqlens_q,
                               max_seqlen_q, max_seqlen_k, sinks, window, softmax_scale, num_splits, workspace, out, lse,
                               return_lse)


def _decode_paged_multi(q, k_pages, v_pages, scales, block_table, seq_lens, cu_seqlens_q, max_seqlen_q, max_seqlen_k,
                        sinks, window, softmax_scale, num_splits, workspace, out, lse, return_lse):
    _need(q, "q", torch.bfloat16, 3)
    kv_dtype = torch.bfloat16 if scales is None else torch.uint8
    _need(k_pages, "k_pages", kv_dtype, 4)
    _need(v_pages, "v_pages", kv_dtype, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    tq, hq, d = q.shape
    bsz = seq_lens.shape[0]
    num_pages, page_size, hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if v_pages.shape != k_pages.shape or k_pages.shape[3] != d:
        raise ValueError("k_pages and v_pages must be [P, page_size, Hkv, D] matching q")
    if block_table.shape[0] != bsz or cu_seqlens_q.shape[0] != bsz + 1:
        raise ValueError("block_table needs one row per sequence and cu_seqlens_q batch + 1 entries")
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, 1)
        if sinks.shape[0] != hq:
            raise ValueError("sinks must have num_q_heads entries")
    need = decode_workspace_bytes(tq, hq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    tail = (_ptr(block_table), _ptr(seq_lens), _ptr(cu_seqlens_q), bsz, block_table.shape[1], page_size, num_pages,
            int(max_seqlen_q), int(max_seqlen_k), tq, _ptr(sinks), hq, hkv, d, int(window), float(softmax_scale),
            int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(q.device))
    if scales is None:
        _check(library().sinkattn_decode_paged_multi(_ptr(q), _ptr(k_pages), _ptr(v_pages), *tail))
    else:
        _check(library().sinkattn_decode_paged_multi_fp8(_ptr(q), _ptr(k_pages), _ptr(v_pages), float(scales[0]),
                                                         float(scales[1]), *tail))
    return (out, lse) if (return_lse or lse is not None) else out


def rope_qkv_append(qkv: torch.Tensor, positions: torch.Tensor, slot_mapping: torch.Tensor, num_q_heads: int,
                    num_kv_heads: int, k_cache: torch.Tensor, v_cache: torch.Tensor, rope_theta: float = 10000.0,
                    yarn_factor: float = 1.0, yarn_original_max_position: int = 4096, yarn_beta_fast: float = 32.0,
                    yarn_beta_slow: float = 1.0, yarn_truncate: bool = False,
                    q_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The fused rotary step: qkv [T, Hq + 2 Hkv, 64] bf16, positions and
    slot_mapping [T] int32; writes the rotated K and the V of token t into
    k_cache / v_cache [rows, Hkv, 64] row slot_mapping[t] (-1: none) and
    returns the rotated Q [T, Hq, 64]."""
    _need(qkv, "qkv", torch.bfloat16, 3)
    _need(positions, "positions", torch.int32, 1)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    t, heads, d = qkv.shape
    if heads != num_q_heads + 2 * num_kv_heads:
        raise ValueError("qkv must hold num_q_heads + 2 * num_kv_heads heads")
    if positions.shape[0] != t or slot_mapping.shape[0] != t:
        raise ValueError("positions and slot_mapping need one entry per token")
    if k_cache.shape != v_cache.shape or k_cache.shape[1:] != (num_kv_heads, d):
        raise ValueError("k_cache and v_cache must be [rows, num_kv_heads, head_dim]")
    if q_out is None:
        q_out = torch.empty((t, num_q_heads, d), dtype=torch.bfloat16, device=qkv.device)
    _check(library().sinkattn_rope_qkv_append(
        _ptr(qkv), _ptr(positions), _ptr(slot_mapping), t, int(num_q_heads), int(num_kv_heads), d,
        float(rope_theta), float(yarn_factor), int(yarn_original_max_position), float(yarn_beta_fast),
        float(yarn_beta_slow), int(bool(yarn_truncate)), _ptr(q_out), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
        _stream(qkv.device)))
    return q_out


def oproj_bias(o: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor],
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Output projection with bias: o [N, K] bf16 (or [N, Hq, D], viewed as
    [N, Hq * D]), w [E, K] bf16, bias [E] fp32 or None -> y [N, E] bf16."""
    if o.dim() == 3:
        o = o.reshape(o.shape[0], -1)
    _need(o, "o", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 2)
    n, k = o.shape
    e = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("w must be [out_features, in_features] matching o")
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
        if bias.shape[0] != e:
            raise ValueError("bias must have out_features entries")
    if out is None:
        out = torch.empty((n, e), dtype=torch.bfloat16, device=o.device)
    need = int(library().sinkattn_oproj_workspace_bytes(n, k, e))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=o.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().sinkattn_oproj_bias(_ptr(o), _ptr(w), _ptr(bias), n, k, e, _ptr(out), _ptr(workspace), ws_bytes,
                                         _stream(o.device)))
    return out


def merge_lse(o_parts: torch.Tensor, lse_parts: torch.Tensor, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, return_lse: bool = False):
    """Merge partials o_parts [S, N, H, 64] fp32 with lse_parts [S, N, H]."""
    _need(o_parts, "o_parts", torch.float32, 4)
    _need(lse_parts, "lse_parts", torch.float32, 3)
    s, n, h, d = o_parts.shape
    if lse_parts.shape != (s, n, h):
        raise ValueError("lse_parts must be [S, N, H]")
    if out is None:
        out = torch.empty((n, h, d), dtype=torch.bfloat16, device=o_parts.device)
    if return_lse and lse is None:
        lse = torch.empty((n, h), dtype=torch.float32, device=o_parts.device)
    _check(library().sinkattn_merge_lse(_ptr(o_parts), _ptr(lse_parts), s, n, h, d, _ptr(out), _ptr(lse),
                                        _stream(o_parts.device)))
    return (out, lse) if (return_lse or lse is not None) else out


def version() -> str:
    return library().sinkattn_version().decode()
