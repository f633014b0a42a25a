"""Binding of libkvq_probe (include/kvq_probe.h): the streaming read that
benchmarks rate the decode's KV reads against.  A measurement aid, not part of
the attention path, which never imports this module."""
from __future__ import annotations

import ctypes
import os

import torch

from . import KvqError, _check_status_with, _ptr, _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_probe.so")
EXPORTS = ("kvq_stream_read",)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvqError(f"{LIB_PATH} is not built; run `python -m quantized_kv_cache_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]
        L.kvq_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of `src` once with the decode's load instructions and
    nothing else (kvq_stream_read).  `sink` holds at least workgroups * 4096 bytes."""
    if not src.is_contiguous() or not sink.is_contiguous() or not src.is_cuda or not sink.is_cuda:
        raise KvqError("stream_read: src and sink must be contiguous GPU tensors")
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < workgroups * 4096:
        raise KvqError("stream_read: sink smaller than workgroups * 4096 bytes")
    _check_status_with(lib().kvq_stream_read(_ptr(src), nbytes, workgroups, _ptr(sink),
                                             _stream(stream)), "kvq_stream_read")
