"""CPU oracle for the paged-KV gather / scatter / gather-scatter / permute path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it; the two meet only at the
seeded input generators in ``workloads``.

The arithmetic lives in ``kvx_oracle.c`` (a row-by-row ``memcpy`` loop, see its
header for the definitions and the passages they follow); this module only
marshals numpy arrays into it with ctypes.  Every buffer is a numpy array whose
bytes are copied verbatim, so the dtype of the KV values never matters: pass
``uint8`` views.

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_pins.py``: element-wise brute force on tiny pools,
exhaustive injective tables, ``numpy.take`` / ``torch.permute`` special cases,
round trips, untouched-row invariants and the page-printed KV byte counts.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32, _i64, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


def bind(path: str):
    """Open a build of kvx_oracle.c at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    pp = ctypes.POINTER(ctypes.c_void_p)
    lib.oracle_gather.argtypes = [_i32, _i64, pp, _i64, _i64, _i32, _i64, _i32, _p, _p, _p,
                                  _i64, _p, ctypes.c_int]
    lib.oracle_scatter.argtypes = [_i32, _i64, _p, _i32, _p, _p, _p, _i64, pp, _i64, _i64,
                                   _i32, _i64, ctypes.c_int]
    lib.oracle_gather_scatter.argtypes = [_i32, _i64, pp, _i64, _i64, _i32, _i64, _p, _p, _i64,
                                          _i32, _p, pp, _i64, _i64, _i32, _i64, _p, _p, _i64,
                                          ctypes.c_int]
    lib.oracle_gather_scatter_heads.argtypes = [
        _i32, _i32, _i64, pp, _i64, _i32, _i64, _p, _p, _i64, _i32, _i32, _i32, _i32, _p,
        pp, _i64, _i32, _i64, _p, _p, _i64, _i32, _i32, _i32, ctypes.c_int]
    lib.oracle_extract_permute.argtypes = [_i32, _i32, _i64, pp, _i64, _i64, _p, ctypes.c_int]
    lib.oracle_rebuild_permute.argtypes = [_i32, _i32, _i64, _p, _i64, pp, _i64, ctypes.c_int]
    for f in (lib.oracle_gather, lib.oracle_scatter, lib.oracle_gather_scatter,
              lib.oracle_gather_scatter_heads, lib.oracle_extract_permute,
              lib.oracle_rebuild_permute):
        f.restype = _i64
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = bind(_LIB_PATH)
    return _lib


def _ptr(a: np.ndarray) -> int:
    if not a.flags.c_contiguous:
        raise ValueError("oracle buffers must be C-contiguous")
    return a.ctypes.data


def _ptr_array(planes: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * len(planes))()
    for i, p in enumerate(planes):
        arr[i] = _ptr(p)
    return arr


def _csr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _check_table(name, num_reqs, tok_off, pg_off):
    """What the C loop relies on to stay inside its buffers.  The token CSR
    must follow its contract (starts at 0, never decreases): the oracle
    defines no result for one that does not.  The page table may hold
    anything -- start offsets anywhere, lists shorter than their tokens need,
    ids out of range: the loop reads entry pg_off[r] + t / page_size only when
    it lies in [0, len(ids)) and skips the row otherwise."""
    if tok_off.shape != (num_reqs + 1,) or pg_off.shape != (num_reqs + 1,):
        raise ValueError(f"{name}: offsets must have num_reqs+1 entries")
    n = np.diff(tok_off)
    if tok_off[0] != 0 or (n < 0).any():
        raise ValueError(f"{name}: token offsets must start at 0 and be non-decreasing")


def _check_planes(name, planes, stride, page_size, num_pages, R, page_stride=0):
    """Every row the loop may touch must lie inside each plane buffer."""
    ps = int(page_stride) if page_stride else int(page_size) * int(stride)
    need = ((int(num_pages) - 1) * ps + (int(page_size) - 1) * int(stride) + int(R)
            if int(num_pages) > 0 else 0)
    for p in planes:
        if p.nbytes < need:
            raise ValueError(f"{name}: plane of {p.nbytes} B is smaller than {need} B")


def gather(src_planes: Sequence[np.ndarray], stride: int, page_size: int, num_pages: int,
           row_bytes: int, tok_off, pg_off, ids, staging: np.ndarray, nthreads: int = 1,
           page_stride: int = 0) -> int:
    """Pool -> contiguous staging.  Returns the number of skipped rows.
    ``page_stride``: bytes between consecutive pages of a plane (0: page_size
    * stride, pages of one plane's rows only)."""
    tok_off, pg_off = _csr(tok_off, np.int64), _csr(pg_off, np.int64)
    ids = _csr(ids, np.int32)
    reqs = len(tok_off) - 1
    _check_table("src", reqs, tok_off, pg_off)
    Q = len(src_planes)
    R = int(row_bytes)
    _check_planes("src", src_planes, stride, page_size, num_pages, R, page_stride)
    if staging.nbytes < int(tok_off[-1]) * Q * R:
        raise ValueError("staging too small")
    return int(_load().oracle_gather(Q, R, _ptr_array(src_planes), stride, page_stride,
                                     page_size, num_pages, reqs, _ptr(tok_off), _ptr(pg_off),
                                     _ptr(ids), ids.size, _ptr(staging), nthreads))


def scatter(staging: np.ndarray, row_bytes: int, tok_off, pg_off, ids,
            dst_planes: Sequence[np.ndarray], stride: int, page_size: int, num_pages: int,
            nthreads: int = 1, page_stride: int = 0) -> int:
    """Contiguous staging -> pool.  Returns the number of skipped rows."""
    tok_off, pg_off = _csr(tok_off, np.int64), _csr(pg_off, np.int64)
    ids = _csr(ids, np.int32)
    reqs = len(tok_off) - 1
    _check_table("dst", reqs, tok_off, pg_off)
    Q = len(dst_planes)
    R = int(row_bytes)
    _check_planes("dst", dst_planes, stride, page_size, num_pages, R, page_stride)
    if staging.nbytes < int(tok_off[-1]) * Q * R:
        raise ValueError("staging too small")
    return int(_load().oracle_scatter(Q, R, _ptr(staging), reqs, _ptr(tok_off), _ptr(pg_off),
                                      _ptr(ids), ids.size, _ptr_array(dst_planes), stride,
                                      page_stride, page_size, num_pages, nthreads))


def gather_scatter(src_planes: Sequence[np.ndarray], src_stride: int, src_page_size: int,
                   src_num_pages: int, src_pg_off, src_ids, row_bytes: int, tok_off,
                   dst_planes: Sequence[np.ndarray], dst_stride: int, dst_page_size: int,
                   dst_num_pages: int, dst_pg_off, dst_ids, nthreads: int = 1,
                   src_page_stride: int = 0, dst_page_stride: int = 0) -> int:
    """Pool -> pool, row by row.  Returns the number of skipped rows."""
    tok_off = _csr(tok_off, np.int64)
    src_pg_off, dst_pg_off = _csr(src_pg_off, np.int64), _csr(dst_pg_off, np.int64)
    src_ids, dst_ids = _csr(src_ids, np.int32), _csr(dst_ids, np.int32)
    reqs = len(tok_off) - 1
    _check_table("src", reqs, tok_off, src_pg_off)
    _check_table("dst", reqs, tok_off, dst_pg_off)
    if len(src_planes) != len(dst_planes):
        raise ValueError("plane counts differ")
    _check_planes("src", src_planes, src_stride, src_page_size, src_num_pages, row_bytes,
                  src_page_stride)
    _check_planes("dst", dst_planes, dst_stride, dst_page_size, dst_num_pages, row_bytes,
                  dst_page_stride)
    return int(_load().oracle_gather_scatter(
        len(src_planes), int(row_bytes), _ptr_array(src_planes), src_stride, src_page_stride,
        src_page_size, src_num_pages, _ptr(src_pg_off), _ptr(src_ids), src_ids.size, reqs,
        _ptr(tok_off), _ptr_array(dst_planes), dst_stride, dst_page_stride, dst_page_size,
        dst_num_pages, _ptr(dst_pg_off), _ptr(dst_ids), dst_ids.size, nthreads))


def gather_scatter_heads(src_planes: Sequence[np.ndarray], src_stride: int, src_page_size: int,
                         src_num_pages: int, src_pg_off, src_ids, src_heads, head_bytes: int,
                         nh: int, tok_off, dst_planes: Sequence[np.ndarray], dst_stride: int,
                         dst_page_size: int, dst_num_pages: int, dst_pg_off, dst_ids, dst_heads,
                         nthreads: int = 1) -> int:
    """Pool -> pool, nh heads of every token row.  ``src_heads`` / ``dst_heads``
    are (kv_heads, head0, hnd) per side: heads per token row in that pool, the
    first head of the slice, and 1 for head-major (HND) blocks.  ``*_stride`` is
    the bytes of one token row.  Returns the number of skipped token rows."""
    tok_off = _csr(tok_off, np.int64)
    src_pg_off, dst_pg_off = _csr(src_pg_off, np.int64), _csr(dst_pg_off, np.int64)
    src_ids, dst_ids = _csr(src_ids, np.int32), _csr(dst_ids, np.int32)
    reqs = len(tok_off) - 1
    _check_table("src", reqs, tok_off, src_pg_off)
    _check_table("dst", reqs, tok_off, dst_pg_off)
    for name, (H, h0, hnd), stride in (("src", src_heads, src_stride),
                                        ("dst", dst_heads, dst_stride)):
        if h0 < 0 or h0 + nh > H or stride < H * head_bytes:
            raise ValueError(f"{name}: head slice outside the row")
    _check_planes("src", src_planes, src_stride, src_page_size, src_num_pages, src_stride)
    _check_planes("dst", dst_planes, dst_stride, dst_page_size, dst_num_pages, dst_stride)
    return int(_load().oracle_gather_scatter_heads(
        len(src_planes), nh, head_bytes, _ptr_array(src_planes), src_stride, src_page_size,
        src_num_pages, _ptr(src_pg_off), _ptr(src_ids), src_ids.size, *src_heads, reqs,
        _ptr(tok_off), _ptr_array(dst_planes), dst_stride, dst_page_size, dst_num_pages,
        _ptr(dst_pg_off), _ptr(dst_ids), dst_ids.size, *dst_heads, nthreads))


def extract_permute(hf_planes: Sequence[np.ndarray], kv_heads: int, head_bytes: int,
                    s_cap: int, seq: int, out: np.ndarray, nthreads: int = 1) -> None:
    """[1, H, s_cap, D] per plane -> [Q][seq][H][D] (head_bytes = D * element size)."""
    Q = len(hf_planes)
    if seq > s_cap or out.nbytes < Q * seq * kv_heads * head_bytes:
        raise ValueError("bad extract sizes")
    for p in hf_planes:
        if p.nbytes < kv_heads * s_cap * head_bytes:
            raise ValueError("hf plane too small")
    _load().oracle_extract_permute(Q, kv_heads, head_bytes, _ptr_array(hf_planes), s_cap, seq,
                                   _ptr(out), nthreads)


def rebuild_permute(flat: np.ndarray, kv_heads: int, head_bytes: int, seq: int,
                    hf_planes: Sequence[np.ndarray], s_cap: int, nthreads: int = 1) -> None:
    """[Q][seq][H][D] -> [1, H, s_cap, D] per plane; positions s >= seq untouched."""
    Q = len(hf_planes)
    if seq > s_cap or flat.nbytes < Q * seq * kv_heads * head_bytes:
        raise ValueError("bad rebuild sizes")
    for p in hf_planes:
        if p.nbytes < kv_heads * s_cap * head_bytes:
            raise ValueError("hf plane too small")
    _load().oracle_rebuild_permute(Q, kv_heads, head_bytes, _ptr(flat), seq,
                                   _ptr_array(hf_planes), s_cap, nthreads)


def kv_bytes(prompt_len: int, num_layers: int, kv_heads: int, head_dim: int,
             elem_bytes: int, num_kv: int = 2) -> int:
    """Bytes of one request's KV: num_kv x L x layers x kv_heads x head_dim x b.

    "DistServe 完全拆解" (pinghaoyang.com.cn), section "KV Cache 跨实例传输":
    the factor 2 counts K and V (num_kv = 1 for a single latent vector per
    layer), L is the prompt length and b the bytes per element.  This is also
    the staging size a gather of that request needs.
    """
    return num_kv * prompt_len * num_layers * kv_heads * head_dim * elem_bytes
