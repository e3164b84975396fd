"""Python binding of libgqa.so: GroupQueryAttention over a shared KV buffer.

Argument marshalling only. Every step of the op (rotary, eviction, append,
attention, split merge) runs in the HIP kernels behind the C ABI declared in
include/gqa.h; this module reads shapes off torch tensors, checks that they
agree, and passes raw device pointers and the current HIP stream. There is no
CPU or PyTorch fallback: if the library has not been built, importing this
package raises.

The functions carry the C entry points' names:
  gqa_append_kv, gqa_attention_prefill, gqa_attention_decode,
  gqa_attention_present, gqa_evict_window, gqa_workspace_bytes,
  gqa_attention_decode_noalloc.
The attention functions also take separate present_key/present_value
tensors (past and present in different buffers) and then call
gqa_attention_present.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa.so")

GQA_OK, GQA_ERR_NO_ROOM, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP = range(6)
GQA_FP32, GQA_FP16, GQA_BF16 = 0, 1, 2
STATUS_NAMES = {0: "ok", 1: "no_room", 2: "invalid_arg", 3: "unsupported", 4: "workspace", 5: "hip"}
EXPORTED = ("gqa_workspace_bytes", "gqa_append_kv", "gqa_attention_prefill", "gqa_attention_decode",
            "gqa_attention_present", "gqa_evict_window", "gqa_attention_decode_noalloc",
            "gqa_stream_read", "gqa_status_string", "gqa_last_error")
NOALLOC_SCRATCH_BYTES = 64 << 20     # GQA_NOALLOC_SCRATCH_BYTES


class GQAError(RuntimeError):
    """A non-OK status from the library; `.status` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("new_tokens", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("kv_num_heads", ctypes.c_int32),
                ("head_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("local_window_size", ctypes.c_int32),
                ("cos_cache", ctypes.c_void_p), ("sin_cache", ctypes.c_void_p),
                ("rotary_rows", ctypes.c_int32), ("rotary_interleaved", ctypes.c_int32),
                ("greedy_eviction", ctypes.c_int32),
                ("attention_bias", ctypes.c_void_p), ("bias_batch", ctypes.c_int32),
                ("bias_heads", ctypes.c_int32), ("bias_total", ctypes.c_int32),
                ("position_offset_host", ctypes.c_void_p), ("position_offset_dev", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python __graft_entry__.py build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32P, VP = ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p
    lib.gqa_workspace_bytes.argtypes = [P, ctypes.POINTER(Options)]
    lib.gqa_workspace_bytes.restype = ctypes.c_size_t
    lib.gqa_append_kv.argtypes = [P, ctypes.POINTER(Options), VP, VP, VP, VP, I32P, VP, VP]
    lib.gqa_append_kv.restype = ctypes.c_int
    for name in ("gqa_attention_prefill", "gqa_attention_decode"):
        f = getattr(lib, name)
        f.argtypes = [P, ctypes.POINTER(Options), VP, VP, VP, VP, VP, I32P, VP, VP, VP,
                      ctypes.c_size_t, VP]
        f.restype = ctypes.c_int
    lib.gqa_attention_present.argtypes = [P, ctypes.POINTER(Options), VP, VP, VP, VP, VP,
                                          ctypes.c_int32, VP, VP, I32P, VP, VP, VP,
                                          ctypes.c_size_t, VP]
    lib.gqa_attention_present.restype = ctypes.c_int
    lib.gqa_attention_decode_noalloc.argtypes = [P, ctypes.POINTER(Options), VP, VP, VP, VP, VP,
                                                 I32P, VP, VP, VP]
    lib.gqa_attention_decode_noalloc.restype = ctypes.c_int
    lib.gqa_evict_window.argtypes = [P, ctypes.c_int32, VP, VP, I32P, VP, I32P, VP, ctypes.c_size_t, VP]
    lib.gqa_evict_window.restype = ctypes.c_int
    lib.gqa_stream_read.argtypes = [VP, ctypes.c_size_t, VP]
    lib.gqa_stream_read.restype = ctypes.c_int
    lib.gqa_status_string.argtypes = [ctypes.c_int]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_last_error.argtypes = []
    lib.gqa_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status: int):
    if status != GQA_OK:
        msg = (lib.gqa_last_error() or b"").decode() or lib.gqa_status_string(status).decode()
        raise GQAError(status, msg)


def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: GQA_FP32, torch.float16: GQA_FP16, torch.bfloat16: GQA_BF16}
    if t.dtype not in m:
        raise GQAError(GQA_ERR_INVALID_ARG, f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _host_lengths(seqlens_k_host, B: int):
    a = np.ascontiguousarray(np.asarray(seqlens_k_host.cpu() if hasattr(seqlens_k_host, "cpu")
                                        else seqlens_k_host), dtype=np.int32)
    if a.shape != (B,):
        raise GQAError(GQA_ERR_INVALID_ARG, f"seqlens_k_host has shape {a.shape}, expected ({B},)")
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _cache_shape(k_cache, v_cache):
    if k_cache.dim() != 4 or tuple(k_cache.shape) != tuple(v_cache.shape):
        raise GQAError(GQA_ERR_INVALID_ARG, "k_cache / v_cache must both be [B, Hkv, M, D]")
    if k_cache.dtype != v_cache.dtype:
        raise GQAError(GQA_ERR_INVALID_ARG, "k_cache and v_cache dtypes differ")
    return tuple(int(x) for x in k_cache.shape)


def _same_buffer(past, present, what: str):
    # The op may bind one tensor to both past and present; we require it and
    # check the addresses at run time.
    if present is not None and present.data_ptr() != past.data_ptr():
        raise GQAError(GQA_ERR_INVALID_ARG, f"past_{what} and present_{what} must share one buffer")


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise GQAError(GQA_ERR_INVALID_ARG, "tensors must be contiguous")


def _check_aux(B, D, device, seqlens_k_dev, cos_cache, sin_cache, *tensors):
    """What the kernels read beyond the main tensors must have the layout
    they assume: int32 [B] device lengths, fp32 [P, D/2] rotary tables, and
    every tensor on one device."""
    torch = _torch()
    for t in tensors + (seqlens_k_dev, cos_cache, sin_cache):
        if t is not None and t.device != device:
            raise GQAError(GQA_ERR_INVALID_ARG, f"tensor on {t.device}, expected {device}")
    if seqlens_k_dev is not None and (seqlens_k_dev.dtype != torch.int32
                                      or seqlens_k_dev.numel() != B
                                      or not seqlens_k_dev.is_contiguous()):
        raise GQAError(GQA_ERR_INVALID_ARG, f"seqlens_k_dev must be a contiguous int32 tensor of {B}")
    if cos_cache is not None or sin_cache is not None:
        if cos_cache is None or sin_cache is None:
            raise GQAError(GQA_ERR_INVALID_ARG, "cos_cache and sin_cache must be given together")
        for t in (cos_cache, sin_cache):
            if (t.dtype != torch.float32 or t.dim() != 2 or int(t.shape[1]) != D // 2
                    or tuple(t.shape) != tuple(cos_cache.shape) or not t.is_contiguous()):
                raise GQAError(GQA_ERR_INVALID_ARG,
                               f"cos_cache / sin_cache must be contiguous float32 [P, {D // 2}]")


def make_shape(B, S, H, Hkv, D, M, dtype) -> Shape:
    return Shape(B, S, H, Hkv, D, M, dtype)


def make_options(scale=0.0, local_window_size=-1, cos_cache=None, sin_cache=None,
                 rotary_interleaved=False, greedy_eviction=False, attention_bias=None,
                 offsets=None) -> Options:
    """`offsets`: None, or the (host array, device tensor) pair that
    _position_offsets returns."""
    rows = int(cos_cache.shape[0]) if cos_cache is not None else 0
    bb = bh = bt = 0
    if attention_bias is not None:
        if attention_bias.dim() != 4:
            raise GQAError(GQA_ERR_INVALID_ARG, "attention_bias must be [B or 1, H or 1, S, T]")
        bb, bh, bt = (int(attention_bias.shape[i]) for i in (0, 1, 3))
    oh = od = None
    if offsets is not None:
        oh, od = offsets[0].ctypes.data, _ptr(offsets[1])
    return Options(float(scale), int(local_window_size), _ptr(cos_cache), _ptr(sin_cache), rows,
                   int(bool(rotary_interleaved)), int(bool(greedy_eviction)), _ptr(attention_bias),
                   bb, bh, bt, oh, od)


def _position_offsets(position_offset, position_offset_dev, B: int, device, allocate: bool = True):
    """Host int32 [B] copy (kept alive by the caller through the call) and
    the device tensor of the per-sequence position offsets, or None.

    `position_offset` is the host copy (array-like or CPU tensor); the device
    copy is `position_offset_dev` when given, else (allocate=True) a new
    tensor made from the host copy."""
    if position_offset is None:
        if position_offset_dev is not None:
            raise GQAError(GQA_ERR_INVALID_ARG, "position_offset_dev needs its host copy position_offset")
        return None
    host, _ = _host_lengths(position_offset, B)
    if position_offset_dev is None:
        if not allocate:
            raise GQAError(GQA_ERR_INVALID_ARG, "give position_offset_dev (this entry point allocates nothing)")
        position_offset_dev = _torch().from_numpy(host.copy()).to(device)
    torch = _torch()
    if (position_offset_dev.dtype != torch.int32 or position_offset_dev.numel() != B
            or not position_offset_dev.is_contiguous() or position_offset_dev.device != device):
        raise GQAError(GQA_ERR_INVALID_ARG,
                       f"position_offset_dev must be a contiguous int32 tensor of {B} on {device}")
    return host, position_offset_dev


_workspaces = {}


def gqa_workspace_bytes(B, S, H, Hkv, D, M, dtype: int, local_window_size: int = -1) -> int:
    opts = make_options(0.0, local_window_size)
    return int(lib.gqa_workspace_bytes(ctypes.byref(make_shape(B, S, H, Hkv, D, M, dtype)),
                                       ctypes.byref(opts)))


def workspace_for(shape: Shape, device, opts: Optional[Options] = None):
    """A zero-filled workspace for this shape and options, cached per device
    and size.

    Calls that share a cached workspace must not overlap in time (same stream
    or synchronised streams)."""
    n = int(lib.gqa_workspace_bytes(ctypes.byref(shape), ctypes.byref(opts) if opts else None))
    if n == 0:
        return None, 0
    key = (str(device), n)
    ws = _workspaces.get(key)
    if ws is None:
        ws = _torch().zeros(n, dtype=_torch().uint8, device=device)
        _workspaces[key] = ws
    return ws, n


def _kv_common(k_new, k_cache, v_cache, num_heads):
    B, S, hkvd = (int(x) for x in k_new.shape)
    Bc, Hkv, M, D = _cache_shape(k_cache, v_cache)
    if Bc != B or hkvd != Hkv * D:
        raise GQAError(GQA_ERR_INVALID_ARG, "k_new must be [B, S, Hkv*D] matching the cache")
    return B, S, Hkv, M, D


def gqa_append_kv(k_new, v_new, k_cache, v_cache, seqlens_k_host, seqlens_k_dev, *,
                  cos_cache=None, sin_cache=None, rotary_interleaved=False,
                  present_key=None, present_value=None, stream=None, position_offset=None,
                  position_offset_dev=None):
    """Append S new rows per sequence at seqlens_k (rotary on K if tables given)."""
    _same_buffer(k_cache, present_key, "key")
    _same_buffer(v_cache, present_value, "value")
    _contig(k_new, v_new, k_cache, v_cache, cos_cache, sin_cache)
    if tuple(k_new.shape) != tuple(v_new.shape) or k_new.dim() != 3:
        raise GQAError(GQA_ERR_INVALID_ARG, "k_new / v_new must both be [B, S, Hkv*D]")
    B, S, Hkv, M, D = _kv_common(k_new, k_cache, v_cache, None)
    _check_aux(B, D, k_cache.device, seqlens_k_dev, cos_cache, sin_cache, k_new, v_new, v_cache)
    shape = make_shape(B, S, Hkv, Hkv, D, M, dtype_code(k_cache))
    offs = _position_offsets(position_offset, position_offset_dev, B, k_cache.device)
    opts = make_options(0.0, -1, cos_cache, sin_cache, rotary_interleaved, offsets=offs)
    hl, hp = _host_lengths(seqlens_k_host, B)  # keep hl alive through the call
    _check(lib.gqa_append_kv(ctypes.byref(shape), ctypes.byref(opts), _ptr(k_new), _ptr(v_new),
                             _ptr(k_cache), _ptr(v_cache), hp, _ptr(seqlens_k_dev), _stream(stream)))


def _attention(fn, q, k_new, v_new, k_cache, v_cache, seqlens_k_host, seqlens_k_dev, out,
               scale, local_window_size, cos_cache, sin_cache, rotary_interleaved,
               present_key, present_value, workspace, stream, greedy_eviction=False,
               attention_bias=None, position_offset=None, position_offset_dev=None):
    past_k = past_v = None
    past_rows = 0
    if (present_key is None) != (present_value is None):
        raise GQAError(GQA_ERR_INVALID_ARG, "present_key and present_value go together")
    if present_key is not None and (present_key.data_ptr() != k_cache.data_ptr()
                                    or present_value.data_ptr() != v_cache.data_ptr()):
        # separate buffers: k_cache / v_cache are the past, the call fills present
        _contig(k_cache, v_cache)
        Bp, Hp, past_rows, Dp = _cache_shape(k_cache, v_cache)
        if ((Bp, Hp, Dp) != tuple(int(x) for x in present_key.shape[:2]) + (int(present_key.shape[3]),)
                or present_key.dtype != k_cache.dtype):
            raise GQAError(GQA_ERR_INVALID_ARG, "past and present must agree in B, Hkv, D and dtype")
        past_k, past_v = k_cache, v_cache
        k_cache, v_cache = present_key, present_value
    _contig(q, k_new, v_new, k_cache, v_cache, cos_cache, sin_cache)
    if q.dim() != 3 or tuple(k_new.shape) != tuple(v_new.shape) or k_new.dim() != 3:
        raise GQAError(GQA_ERR_INVALID_ARG, "q must be [B, S, H*D], k_new/v_new [B, S, Hkv*D]")
    B, S, Hkv, M, D = _kv_common(k_new, k_cache, v_cache, None)
    if int(q.shape[0]) != B or int(q.shape[1]) != S or int(q.shape[2]) % D:
        raise GQAError(GQA_ERR_INVALID_ARG, "q must be [B, S, H*D] with the cache's D")
    H = int(q.shape[2]) // D
    if q.dtype != k_cache.dtype or k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise GQAError(GQA_ERR_INVALID_ARG, "q, k_new, v_new and the caches must share a dtype")
    if out is None:
        out = _torch().empty_like(q)
    _contig(out)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise GQAError(GQA_ERR_INVALID_ARG, "out must match q")
    _check_aux(B, D, k_cache.device, seqlens_k_dev, cos_cache, sin_cache, q, k_new, v_new,
               v_cache, out, attention_bias, past_k, past_v)
    shape = make_shape(B, S, H, Hkv, D, M, dtype_code(q))
    if attention_bias is not None:
        _contig(attention_bias)
        if (attention_bias.dtype != q.dtype or attention_bias.dim() != 4
                or int(attention_bias.shape[2]) != S):
            raise GQAError(GQA_ERR_INVALID_ARG, "attention_bias must be [B or 1, H or 1, S, T] in q's dtype")
    offs = _position_offsets(position_offset, position_offset_dev, B, k_cache.device)
    opts = make_options(scale, local_window_size, cos_cache, sin_cache, rotary_interleaved,
                        greedy_eviction, attention_bias, offs)
    hl, hp = _host_lengths(seqlens_k_host, B)  # keep hl alive through the call
    if workspace is None:
        ws, nbytes = workspace_for(shape, q.device, opts)
    else:
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    if past_k is not None:
        if fn is lib.gqa_attention_decode and S != 1:
            raise GQAError(GQA_ERR_INVALID_ARG, "decode needs new_tokens == 1")
        _check(lib.gqa_attention_present(ctypes.byref(shape), ctypes.byref(opts), _ptr(q),
                                         _ptr(k_new), _ptr(v_new), _ptr(past_k), _ptr(past_v),
                                         int(past_rows), _ptr(k_cache), _ptr(v_cache), hp,
                                         _ptr(seqlens_k_dev), _ptr(out), _ptr(ws), nbytes,
                                         _stream(stream)))
        return out
    _check(fn(ctypes.byref(shape), ctypes.byref(opts), _ptr(q), _ptr(k_new), _ptr(v_new),
              _ptr(k_cache), _ptr(v_cache), hp, _ptr(seqlens_k_dev), _ptr(out), _ptr(ws),
              nbytes, _stream(stream)))
    return out


def gqa_attention_prefill(q, k_new, v_new, k_cache, v_cache, seqlens_k_host, seqlens_k_dev,
                          out=None, *, scale=0.0, local_window_size=-1, cos_cache=None,
                          sin_cache=None, rotary_interleaved=False, present_key=None,
                          present_value=None, workspace=None, stream=None, greedy_eviction=False,
                          attention_bias=None, position_offset=None,
                          position_offset_dev=None):
    """The whole op for S >= 1 new tokens; returns out [B, S, H*D].

    With present_key/present_value in buffers other than k_cache/v_cache,
    k_cache/v_cache are the past ([B, Hkv, past_rows, D], only read) and the
    present buffers receive past ++ new (gqa_attention_present)."""
    return _attention(lib.gqa_attention_prefill, q, k_new, v_new, k_cache, v_cache, seqlens_k_host,
                      seqlens_k_dev, out, scale, local_window_size, cos_cache, sin_cache,
                      rotary_interleaved, present_key, present_value, workspace, stream,
                      greedy_eviction, attention_bias, position_offset,
                      position_offset_dev)


def gqa_attention_decode(q, k_new, v_new, k_cache, v_cache, seqlens_k_host, seqlens_k_dev,
                         out=None, *, scale=0.0, local_window_size=-1, cos_cache=None,
                         sin_cache=None, rotary_interleaved=False, present_key=None,
                         present_value=None, workspace=None, stream=None, greedy_eviction=False,
                         attention_bias=None, position_offset=None,
                         position_offset_dev=None):
    """The whole op for one new token per sequence; returns out [B, 1, H*D]."""
    return _attention(lib.gqa_attention_decode, q, k_new, v_new, k_cache, v_cache, seqlens_k_host,
                      seqlens_k_dev, out, scale, local_window_size, cos_cache, sin_cache,
                      rotary_interleaved, present_key, present_value, workspace, stream,
                      greedy_eviction, attention_bias, position_offset,
                      position_offset_dev)


def gqa_attention_decode_noalloc(q, k_new, v_new, k_cache, v_cache, seqlens_k_host, seqlens_k_dev,
                                 out, *, scale=0.0, local_window_size=-1, cos_cache=None,
                                 sin_cache=None, rotary_interleaved=False, greedy_eviction=False,
                                 attention_bias=None, stream=None, position_offset=None,
                                 position_offset_dev=None):
    """gqa_attention_decode on the library's static device scratch: no
    workspace, and nothing is allocated, here or in the library (`out` must
    be given). Calls that overlap in time on one GPU race on the scratch."""
    if out is None:
        raise GQAError(GQA_ERR_INVALID_ARG, "out must be given (this entry point allocates nothing)")
    _contig(q, k_new, v_new, k_cache, v_cache, out, cos_cache, sin_cache, attention_bias)
    if q.dim() != 3 or tuple(k_new.shape) != tuple(v_new.shape) or k_new.dim() != 3:
        raise GQAError(GQA_ERR_INVALID_ARG, "q must be [B, 1, H*D], k_new/v_new [B, 1, Hkv*D]")
    B, S, Hkv, M, D = _kv_common(k_new, k_cache, v_cache, None)
    if int(q.shape[0]) != B or int(q.shape[1]) != S or int(q.shape[2]) % D:
        raise GQAError(GQA_ERR_INVALID_ARG, "q must be [B, S, H*D] with the cache's D")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise GQAError(GQA_ERR_INVALID_ARG, "out must match q")
    if q.dtype != k_cache.dtype or k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise GQAError(GQA_ERR_INVALID_ARG, "q, k_new, v_new and the caches must share a dtype")
    _check_aux(B, D, k_cache.device, seqlens_k_dev, cos_cache, sin_cache, q, k_new, v_new,
               v_cache, out, attention_bias)
    if attention_bias is not None and (attention_bias.dtype != q.dtype or attention_bias.dim() != 4
                                       or int(attention_bias.shape[2]) != S):
        raise GQAError(GQA_ERR_INVALID_ARG, "attention_bias must be [B or 1, H or 1, S, T] in q's dtype")
    shape = make_shape(B, S, int(q.shape[2]) // D, Hkv, D, M, dtype_code(q))
    offs = _position_offsets(position_offset, position_offset_dev, B, k_cache.device,
                             allocate=False)
    opts = make_options(scale, local_window_size, cos_cache, sin_cache, rotary_interleaved,
                        greedy_eviction, attention_bias, offs)
    hl, hp = _host_lengths(seqlens_k_host, B)  # keep hl alive through the call
    _check(lib.gqa_attention_decode_noalloc(ctypes.byref(shape), ctypes.byref(opts), _ptr(q),
                                            _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                            hp, _ptr(seqlens_k_dev), _ptr(out), _stream(stream)))
    return out


def gqa_stream_read(buf, *, stream=None):
    """Enqueue one plain streaming read of the whole (contiguous) device tensor
    `buf`: the yardstick for the memory-bound kernels, not part of the op."""
    _contig(buf)
    _check(lib.gqa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _stream(stream)))


def gqa_evict_window(k_cache, v_cache, seqlens_k_host, seqlens_k_dev, incoming: int, *,
                     workspace=None, stream=None):
    """Compact each sequence so `incoming` tokens fit; returns the new host lengths."""
    _contig(k_cache, v_cache)
    B, Hkv, M, D = _cache_shape(k_cache, v_cache)
    shape = make_shape(B, 0, Hkv, Hkv, D, M, dtype_code(k_cache))
    hl, hp = _host_lengths(seqlens_k_host, B)  # keep hl alive through the call
    after = np.zeros(B, np.int32)
    if workspace is None:
        ws, nbytes = workspace_for(shape, k_cache.device)
    else:
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    _check(lib.gqa_evict_window(ctypes.byref(shape), int(incoming), _ptr(k_cache), _ptr(v_cache), hp,
                                _ptr(seqlens_k_dev), after.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                _ptr(ws), nbytes, _stream(stream)))
    return after
