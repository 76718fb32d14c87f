"""Paged FP8 / INT8 (and KIVI-style INT4 / INT2) KV cache for MI355X.

Thin ctypes binding over ``libkvq.so`` (HIP kernels for gfx950, C ABI in
``include/kvq.h``).  Argument marshalling only: every step of the path runs in
the library's kernels on the caller's (torch's current) HIP stream.  PyTorch
provides device memory and streams.  The library must be built
(``python quantized_kv_cache_08_amd/build.py``); without it every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "KVQ_FP8_E4M3", "KVQ_INT8_ASYM", "KVQ_INT4_KIVI", "KVQ_FP8_E5M2", "KVQ_INT2_KIVI", "KIVI_DTYPES", "KVQ_ATTN_FP8_QK", "KVQ_ATTN_FP8_PV",
    "KVQ_SCALE_PER_TENSOR", "KVQ_SCALE_PER_HEAD", "KVQ_SCALE_PER_TOKEN_HEAD",
    "KVQ_OK", "KVQ_EINVAL", "KVQ_EUNSUPPORTED", "KVQ_EWORKSPACE", "KVQ_EHIP",
    "KvqError", "Cache", "lib", "record_bytes", "append", "kivi_append", "decode_workspace_bytes",
    "verify_workspace_bytes", "verify_attention", "verify_split", "verify_reduce",
    "decode_attention", "decode_attention_noalloc", "kivi_decode_attention", "decode_split", "decode_reduce", "status_string",
    "LIB_PATH",
]

KVQ_FP8_E4M3, KVQ_INT8_ASYM, KVQ_INT4_KIVI, KVQ_FP8_E5M2, KVQ_INT2_KIVI = 1, 2, 3, 4, 5
KIVI_DTYPES = (KVQ_INT4_KIVI, KVQ_INT2_KIVI)
KVQ_ATTN_FP8_QK = 1          # kvq_cache.attn_flags: FP8-domain QK (query quantized to E4M3)
KVQ_ATTN_FP8_PV = 2          # kvq_cache.attn_flags: FP8 score-V product (probabilities in E4M3)
KVQ_SCALE_PER_TENSOR, KVQ_SCALE_PER_HEAD, KVQ_SCALE_PER_TOKEN_HEAD = 0, 1, 2
KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_EWORKSPACE, KVQ_EHIP = 0, -1, -2, -3, -4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", _I32), ("scale_mode", _I32), ("num_pages", _I32), ("page_size", _I32),
        ("num_kv_heads", _I32), ("head_dim", _I32),
        ("k_pages", _P), ("v_pages", _P), ("static_scales", _P),
        ("k_window", _P), ("v_window", _P),
        ("max_seqs", _I32), ("window_tokens", _I32), ("residual", _I32), ("attn_flags", _I32),
    ]


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


_lib = None

_DECODE_ARGS = [ctypes.POINTER(CacheDesc), _P, _I32, _I32, _P, _I32, _P, _I32, ctypes.c_float, _I32,
                _P, ctypes.c_size_t, _P, _P, _P]


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvq.so not built ({LIB_PATH}); run quantized_kv_cache_08_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_record_bytes.restype = ctypes.c_size_t
        L.kvq_record_bytes.argtypes = [_I32] * 5
        L.kvq_append.restype = ctypes.c_int
        L.kvq_append.argtypes = [ctypes.POINTER(CacheDesc), _P, _P, _P, _I32, _P]
        L.kvq_kivi_append.restype = ctypes.c_int
        L.kvq_kivi_append.argtypes = [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]
        L.kvq_decode_workspace_bytes.restype = ctypes.c_int
        L.kvq_decode_workspace_bytes.argtypes = [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, _I32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
        for fn in ("kvq_decode_attention", "kvq_kivi_decode_attention", "kvq_decode_split"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = _DECODE_ARGS
        L.kvq_decode_attention_noalloc.restype = ctypes.c_int
        L.kvq_decode_attention_noalloc.argtypes = _DECODE_ARGS[:10] + [_P, _P, _P]
        L.kvq_decode_reduce.restype = ctypes.c_int
        L.kvq_decode_reduce.argtypes = [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, _I32, _P,
                                        ctypes.c_size_t, _P, _P, _P]
        L.kvq_verify_workspace_bytes.restype = ctypes.c_int
        L.kvq_verify_workspace_bytes.argtypes = [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, _I32, _I32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
        for fn in ("kvq_verify_attention", "kvq_verify_split"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = [ctypes.POINTER(CacheDesc), _P, _I32, _I32] + _DECODE_ARGS[3:]
        L.kvq_verify_reduce.restype = ctypes.c_int
        L.kvq_verify_reduce.argtypes = [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, _I32, _I32, _P,
                                        ctypes.c_size_t, _P, _P, _P]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvqError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape=None, optional: bool = False,
          min_numel: int = 0) -> None:
    """The library reads and writes these arrays through raw device pointers with
    the documented layouts: check type, device, contiguity and size first."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < min_numel:
        raise ValueError(f"{name}: needs at least {min_numel} elements, has {t.numel()}")


def _need_workspace(ws: torch.Tensor) -> None:
    if not isinstance(ws, torch.Tensor) or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace: must be a contiguous device tensor")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def record_bytes(dtype: int, scale_mode: int, page_size: int, head_dim: int, which: int) -> int:
    return int(lib().kvq_record_bytes(dtype, scale_mode, page_size, head_dim, which))


class Cache:
    """One layer's paged cache: page pools allocated with torch (uint8, device)
    plus the C descriptor.  ``fill`` initialises the pools with a byte value."""

    def __init__(self, dtype: int, num_pages: int, num_kv_heads: int, page_size: int = 16,
                 head_dim: int = 128, scale_mode: int = KVQ_SCALE_PER_TOKEN_HEAD,
                 static_scales: Optional[torch.Tensor] = None, device="cuda", fill: Optional[int] = None,
                 max_seqs: int = 0, residual: int = 128, attn_flags: int = 0):
        self.dtype, self.scale_mode = dtype, scale_mode
        self.num_pages, self.num_kv_heads = num_pages, num_kv_heads
        self.page_size, self.head_dim = page_size, head_dim
        self.rec_k = record_bytes(dtype, scale_mode, page_size, head_dim, 0)
        self.rec_v = record_bytes(dtype, scale_mode, page_size, head_dim, 1)
        if self.rec_k == 0 or self.rec_v == 0:
            raise KvqError("kvq_record_bytes", KVQ_EINVAL)
        n = num_pages * num_kv_heads
        alloc = torch.empty if fill is None else (lambda *a, **k: torch.full(*a, fill, **k))
        self.k_pages = alloc((n * self.rec_k,), dtype=torch.uint8, device=device)
        self.v_pages = alloc((n * self.rec_v,), dtype=torch.uint8, device=device)
        self.static_scales = static_scales
        self.max_seqs, self.residual = max_seqs, residual
        self.window_tokens = residual + page_size if dtype in KIVI_DTYPES else 0
        self.k_window = self.v_window = None
        if dtype in KIVI_DTYPES and max_seqs > 0:
            shape = (max_seqs, num_kv_heads, self.window_tokens, head_dim)
            self.k_window = torch.zeros(shape, dtype=torch.float16, device=device)
            self.v_window = torch.zeros(shape, dtype=torch.float16, device=device)
        self.desc = CacheDesc(dtype, scale_mode, num_pages, page_size, num_kv_heads, head_dim,
                              self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                              None if static_scales is None else static_scales.data_ptr(),
                              None if self.k_window is None else self.k_window.data_ptr(),
                              None if self.v_window is None else self.v_window.data_ptr(),
                              max_seqs, self.window_tokens, residual, attn_flags)

    @property
    def attn_flags(self) -> int:
        return int(self.desc.attn_flags)

    @attn_flags.setter
    def attn_flags(self, flags: int) -> None:
        """kvq_attn_flag bits for the decode / verify calls (KVQ_ATTN_FP8_QK)."""
        self.desc.attn_flags = int(flags)

    def records(self, which: int) -> torch.Tensor:
        """Pool ``which`` (0 = K, 1 = V) viewed as [num_pages][num_kv_heads][record bytes]."""
        pool, rec = (self.k_pages, self.rec_k) if which == 0 else (self.v_pages, self.rec_v)
        return pool.view(self.num_pages, self.num_kv_heads, rec)


def append(cache: Cache, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Quantize bf16 K/V rows [T][n_kv][d] into their slots (kvq_append)."""
    _need(slot_mapping, "slot_mapping", torch.int32)
    T = int(slot_mapping.numel())
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, (T, cache.num_kv_heads, cache.head_dim))
    _check("kvq_append", lib().kvq_append(ctypes.byref(cache.desc), _ptr(k), _ptr(v), _ptr(slot_mapping),
                                          int(slot_mapping.numel()), _stream(stream)))


def kivi_append(cache: Cache, k: torch.Tensor, v: torch.Tensor, token_offsets: torch.Tensor,
                context_lens: torch.Tensor, block_table: torch.Tensor, max_new_tokens: int, stream=None) -> None:
    """KIVI INT4 / INT2 append (kvq_kivi_append): new bf16 rows [total][n_kv][d] of each
    sequence (rows token_offsets[b]..token_offsets[b+1]); context_lens = tokens
    held before the call."""
    _need(context_lens, "context_lens", torch.int32)
    num_seqs = int(context_lens.numel())
    _need(token_offsets, "token_offsets", torch.int32, (num_seqs + 1,))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] < num_seqs:
        raise ValueError(f"block_table: expected [>= {num_seqs}][max_pages], got {tuple(block_table.shape)}")
    for name, t in (("k", k), ("v", v)):
        _need(t, name, torch.bfloat16)
        if t.dim() != 3 or tuple(t.shape[1:]) != (cache.num_kv_heads, cache.head_dim):
            raise ValueError(f"{name}: expected [tokens][{cache.num_kv_heads}][{cache.head_dim}], got {tuple(t.shape)}")
    _check("kvq_kivi_append", lib().kvq_kivi_append(
        ctypes.byref(cache.desc), _ptr(k), _ptr(v), _ptr(token_offsets), _ptr(context_lens), _ptr(block_table),
        int(block_table.shape[1]), num_seqs, int(max_new_tokens), _stream(stream)))


def decode_workspace_bytes(cache: Cache, num_seqs: int, num_q_heads: int, max_context_len: int,
                           partition_pages: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check("kvq_decode_workspace_bytes",
           lib().kvq_decode_workspace_bytes(ctypes.byref(cache.desc), num_seqs, num_q_heads,
                                            max_context_len, partition_pages, ctypes.byref(out)))
    return int(out.value)


def _check_attention_args(cache, q, block_table, context_lens, workspace, out, lse, rows) -> None:
    """rows: the leading dimensions of q / out ([B][Hq] or [B][q_len][Hq])."""
    _need(q, "q", torch.bfloat16, rows + (cache.head_dim,))
    _need(out, "out", torch.float32, rows + (cache.head_dim,))
    _need(lse, "lse", torch.float32, rows, optional=True)
    _need(context_lens, "context_lens", torch.int32, (rows[0],))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] < rows[0]:
        raise ValueError(f"block_table: expected [>= {rows[0]}][max_pages], got {tuple(block_table.shape)}")
    _need_workspace(workspace)


def _decode(fn: str, cache, q, block_table, context_lens, max_context_len, softmax_scale, workspace, out,
            lse, partition_pages, stream):
    if q.dim() != 3:
        raise ValueError(f"q: expected [num_seqs][num_q_heads][head_dim], got {tuple(q.shape)}")
    num_seqs, num_q_heads = int(q.shape[0]), int(q.shape[1])
    _check_attention_args(cache, q, block_table, context_lens, workspace, out, lse, (num_seqs, num_q_heads))
    _check(fn, getattr(lib(), fn)(
        ctypes.byref(cache.desc), _ptr(q), num_seqs, num_q_heads, _ptr(block_table),
        int(block_table.shape[1]), _ptr(context_lens), int(max_context_len), float(softmax_scale),
        int(partition_pages), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _ptr(out), _ptr(lse), _stream(stream)))


def decode_attention(cache: Cache, q, block_table, context_lens, max_context_len: int, softmax_scale: float,
                     workspace, out, lse=None, partition_pages: int = 0, stream=None) -> None:
    """One decode step over the quantized paged cache (kvq_decode_attention)."""
    _decode("kvq_decode_attention", cache, q, block_table, context_lens, max_context_len, softmax_scale,
            workspace, out, lse, partition_pages, stream)


def decode_attention_noalloc(cache: Cache, q, block_table, context_lens, max_context_len: int,
                             softmax_scale: float, out, lse=None, partition_pages: int = 0,
                             stream=None) -> None:
    """kvq_decode_attention with the library's static device workspace (no
    allocation; calls overlapping on one device race)."""
    if q.dim() != 3:
        raise ValueError(f"q: expected [num_seqs][num_q_heads][head_dim], got {tuple(q.shape)}")
    num_seqs, num_q_heads = int(q.shape[0]), int(q.shape[1])
    _need(q, "q", torch.bfloat16, (num_seqs, num_q_heads, cache.head_dim))
    _need(out, "out", torch.float32, (num_seqs, num_q_heads, cache.head_dim))
    _need(lse, "lse", torch.float32, (num_seqs, num_q_heads), optional=True)
    _need(context_lens, "context_lens", torch.int32, (num_seqs,))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] < num_seqs:
        raise ValueError(f"block_table: expected [>= {num_seqs}][max_pages], got {tuple(block_table.shape)}")
    _check("kvq_decode_attention_noalloc", lib().kvq_decode_attention_noalloc(
        ctypes.byref(cache.desc), _ptr(q), num_seqs, num_q_heads, _ptr(block_table), int(block_table.shape[1]),
        _ptr(context_lens), int(max_context_len), float(softmax_scale), int(partition_pages), _ptr(out), _ptr(lse),
        _stream(stream)))


def kivi_decode_attention(cache: Cache, q, block_table, context_lens, max_context_len: int,
                          softmax_scale: float, workspace, out, lse=None, partition_pages: int = 0,
                          stream=None) -> None:
    """One decode step over a KIVI INT4 / INT2 cache plus its fp16 window
    (kvq_kivi_decode_attention)."""
    _decode("kvq_kivi_decode_attention", cache, q, block_table, context_lens, max_context_len, softmax_scale,
            workspace, out, lse, partition_pages, stream)


def decode_split(cache: Cache, q, block_table, context_lens, max_context_len: int, softmax_scale: float,
                 workspace, out, lse=None, partition_pages: int = 0, stream=None) -> None:
    _decode("kvq_decode_split", cache, q, block_table, context_lens, max_context_len, softmax_scale,
            workspace, out, lse, partition_pages, stream)


def decode_reduce(cache: Cache, num_seqs: int, num_q_heads: int, max_context_len: int, workspace, out,
                  lse=None, partition_pages: int = 0, stream=None) -> None:
    _need(out, "out", torch.float32, (num_seqs, num_q_heads, cache.head_dim))
    _need(lse, "lse", torch.float32, (num_seqs, num_q_heads), optional=True)
    _need_workspace(workspace)
    _check("kvq_decode_reduce", lib().kvq_decode_reduce(
        ctypes.byref(cache.desc), num_seqs, num_q_heads, int(max_context_len), int(partition_pages),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _ptr(out), _ptr(lse),
        _stream(stream)))


def verify_workspace_bytes(cache: Cache, num_seqs: int, q_len: int, num_q_heads: int, max_context_len: int,
                           partition_pages: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check("kvq_verify_workspace_bytes",
           lib().kvq_verify_workspace_bytes(ctypes.byref(cache.desc), num_seqs, q_len, num_q_heads,
                                            max_context_len, partition_pages, ctypes.byref(out)))
    return int(out.value)


def _verify(fn: str, cache, q, block_table, context_lens, max_context_len, softmax_scale, workspace, out,
            lse, partition_pages, stream):
    if q.dim() != 4:
        raise ValueError(f"q: expected [num_seqs][q_len][num_q_heads][head_dim], got {tuple(q.shape)}")
    num_seqs, q_len, num_q_heads = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    _check_attention_args(cache, q, block_table, context_lens, workspace, out, lse, (num_seqs, q_len, num_q_heads))
    _check(fn, getattr(lib(), fn)(
        ctypes.byref(cache.desc), _ptr(q), num_seqs, q_len, num_q_heads, _ptr(block_table),
        int(block_table.shape[1]), _ptr(context_lens), int(max_context_len), float(softmax_scale),
        int(partition_pages), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _ptr(out), _ptr(lse), _stream(stream)))


def verify_attention(cache: Cache, q, block_table, context_lens, max_context_len: int, softmax_scale: float,
                     workspace, out, lse=None, partition_pages: int = 0, stream=None) -> None:
    """Causal attention of the q_len newest positions per sequence (kvq_verify_attention);
    q [B][q_len][Hq][d] bf16, out [B][q_len][Hq][d] fp32."""
    _verify("kvq_verify_attention", cache, q, block_table, context_lens, max_context_len, softmax_scale,
            workspace, out, lse, partition_pages, stream)


def verify_split(cache: Cache, q, block_table, context_lens, max_context_len: int, softmax_scale: float,
                 workspace, out, lse=None, partition_pages: int = 0, stream=None) -> None:
    _verify("kvq_verify_split", cache, q, block_table, context_lens, max_context_len, softmax_scale,
            workspace, out, lse, partition_pages, stream)


def verify_reduce(cache: Cache, num_seqs: int, q_len: int, num_q_heads: int, max_context_len: int, workspace,
                  out, lse=None, partition_pages: int = 0, stream=None) -> None:
    _need(out, "out", torch.float32, (num_seqs, q_len, num_q_heads, cache.head_dim))
    _need(lse, "lse", torch.float32, (num_seqs, q_len, num_q_heads), optional=True)
    _need_workspace(workspace)
    _check("kvq_verify_reduce", lib().kvq_verify_reduce(
        ctypes.byref(cache.desc), num_seqs, q_len, num_q_heads, int(max_context_len), int(partition_pages),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _ptr(out), _ptr(lse),
        _stream(stream)))
