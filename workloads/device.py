"""Device-side generators: fill torch device buffers with the hash words of
workloads.splitmix64, a plain copy kernel for counter calibration, a
streaming reader (a concurrent load) and a table-free row-pattern mover (the
cost of the paged ops' access patterns by themselves)."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvx_workloads.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.wl_fill_hash.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_void_p]
        lib.wl_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_void_p]
        lib.wl_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p]
        lib.wl_row_pattern.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p] + [ctypes.c_int32] * 6 + [
                                       ctypes.c_uint32, ctypes.c_void_p]
        lib.wl_fill_hash.restype = lib.wl_copy.restype = lib.wl_read_stream.restype = ctypes.c_int
        lib.wl_row_pattern.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream(stream):
    return (stream or torch.cuda.current_stream()).cuda_stream


def fill_hash(t: torch.Tensor, seed: int, ctr0: int = 0, stream=None) -> None:
    """Word i of contiguous device tensor ``t`` <- splitmix64 output ctr0 + i."""
    if not t.is_contiguous() or not t.is_cuda:
        raise ValueError("fill_hash needs a contiguous device tensor")
    rc = _load().wl_fill_hash(t.data_ptr(), t.numel() * t.element_size(), seed, ctr0,
                              _stream(stream))
    if rc != 0:
        raise RuntimeError(f"wl_fill_hash failed ({rc})")


def copy_bytes(dst: torch.Tensor, src: torch.Tensor, nbytes: int, stream=None) -> None:
    """Plain copy of ``nbytes`` from src to dst (both contiguous device tensors)."""
    if nbytes > dst.numel() * dst.element_size() or nbytes > src.numel() * src.element_size():
        raise ValueError("copy larger than a buffer")
    rc = _load().wl_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"wl_copy failed ({rc})")


def read_stream(src: torch.Tensor, sink: torch.Tensor, blocks: int = 2048, stream=None) -> None:
    """Stream once through ``src`` (a decode-like HBM read load) with
    ``blocks`` workgroups; ``sink`` is a device tensor of at least 2048 int64
    words."""
    if sink.numel() * sink.element_size() < 2048 * 8:
        raise ValueError("sink too small")
    rc = _load().wl_read_stream(src.data_ptr(), src.numel() * src.element_size(),
                                sink.data_ptr(), blocks, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"wl_read_stream failed ({rc})")


PATTERN_READ, PATTERN_WRITE, PATTERN_RANDOM_SRC, PATTERN_RANDOM_DST = 1, 2, 4, 8


def row_pattern(src: torch.Tensor, dst: torch.Tensor, sink: torch.Tensor, Q: int, T: int, S: int,
                K: int, slot_set: int, mode: int, stream=None, row_bytes: int = 2048) -> None:
    """Table-free mover of Q x T rows of ``row_bytes`` (wl_row_pattern): read
    and/or write each row at a random slot of a [Q][S][R] buffer or at its
    contiguous place in a [Q][T][R] buffer, per the mode bits; slot sets
    0 .. S/T - 1 are disjoint.  ``sink``: at least 2048 int32 words."""
    if sink.numel() * sink.element_size() < 2048 * 4:
        raise ValueError("sink too small")
    rc = _load().wl_row_pattern(src.data_ptr(), src.numel() * src.element_size(),
                                dst.data_ptr(), dst.numel() * dst.element_size(),
                                sink.data_ptr(), Q, T, S, row_bytes, K, slot_set, mode,
                                _stream(stream))
    if rc != 0:
        raise RuntimeError(f"wl_row_pattern failed ({rc})")
