"""ctypes binding of ``libkvq_testing.so`` (``include/kvq_testing.h``): test
and measurement hooks beside the library, not part of the method.

- ``e4m3_encode`` / ``e5m2_encode``: the append kernel's FP8 encoders on plain
  float arrays (exhaustive device sweeps against the oracle's encoders);
- ``read_probe``: a plain streaming read of a device buffer (the attainable
  HBM read rate the decode kernels are compared with);
- ``plan_stats``: the decode kernels' split plan evaluated on the host for a
  batch of context lengths.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Sequence

import numpy as np
import torch

from . import KvqError, _need, _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_testing.so")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class PlanInfo(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int64), ("ranges_per_head", ctypes.c_int64),
                ("busy_ranges_per_head", ctypes.c_int64), ("segments_per_head", ctypes.c_int64),
                ("slots_used", ctypes.c_int64), ("slots", ctypes.c_int64),
                ("cost", ctypes.c_int32), ("max_segments_per_item", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvq_testing.so not built ({LIB_PATH}); run quantized_kv_cache_08_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for fn in ("kvq_e4m3_encode", "kvq_e5m2_encode"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = [_P, _P, ctypes.c_int64, _P]
        L.kvq_read_probe.restype = ctypes.c_int
        L.kvq_read_probe.argtypes = [_P, ctypes.c_int64, _P, _I32, _I32, _P]
        L.kvq_plan_stats.restype = ctypes.c_int
        L.kvq_plan_stats.argtypes = [_I32, _I32, _I32, _P, _I32, _I32, _I32, ctypes.POINTER(PlanInfo)]
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvqError(fn, status)


def e4m3_encode(x: torch.Tensor, codes: torch.Tensor, stream=None) -> None:
    """float32 -> OCP E4M3 codes with the encoder the append kernel uses."""
    _need(x, "x", torch.float32)
    _need(codes, "codes", torch.uint8, min_numel=x.numel())
    _check("kvq_e4m3_encode", lib().kvq_e4m3_encode(_ptr(x), _ptr(codes), int(x.numel()), _stream(stream)))


def e5m2_encode(x: torch.Tensor, codes: torch.Tensor, stream=None) -> None:
    """float32 -> OCP E5M2 codes with the encoder the append kernel uses for E5M2 caches."""
    _need(x, "x", torch.float32)
    _need(codes, "codes", torch.uint8, min_numel=x.numel())
    _check("kvq_e5m2_encode", lib().kvq_e5m2_encode(_ptr(x), _ptr(codes), int(x.numel()), _stream(stream)))


def read_probe(buf: torch.Tensor, sink: torch.Tensor, blocks_per_cu: int = 2, loads_per_thread: int = 3,
               stream=None) -> None:
    """Plain streaming read of a device byte buffer (kvq_read_probe)."""
    _need(buf, "buf", torch.uint8)
    _need(sink, "sink", torch.int32, min_numel=1)
    _check("kvq_read_probe", lib().kvq_read_probe(_ptr(buf), int(buf.numel()), _ptr(sink), int(blocks_per_cu),
                                                  int(loads_per_thread), _stream(stream)))


def plan_stats(page_size: int, num_kv_heads: int, total_waves: int, context_lens: Sequence[int],
               max_context_len: int, partition_pages: int = 0) -> Dict[str, int]:
    """The split plan for these context lengths (host computation, no GPU)."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    info = PlanInfo()
    _check("kvq_plan_stats", lib().kvq_plan_stats(
        int(page_size), int(num_kv_heads), int(total_waves),
        lens.ctypes.data_as(ctypes.c_void_p) if lens.size else None, int(lens.size), int(max_context_len),
        int(partition_pages), ctypes.byref(info)))
    return {name: int(getattr(info, name)) for name, _ in PlanInfo._fields_}
