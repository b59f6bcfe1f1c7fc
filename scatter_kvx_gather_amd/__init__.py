"""kvx: paged KV-cache gather / scatter / gather-scatter and the HF
[1, H, S, D] <-> [S, H, D] permutes on one MI355X (gfx950).

A thin ctypes binding over ``libkvx.so`` (C ABI and contract: include/kvx.h).
It only marshals arguments -- torch tensors become device pointers and sizes,
streams become ``hipStream_t`` handles -- and every byte is moved by the HIP
kernels in the library.  PyTorch is used for device memory and streams only.

There is no CPU fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import bisect
import ctypes
import os
from typing import Optional, Sequence, Union

import numpy as np
import torch

__all__ = ["KvxError", "Layout", "Pool", "Requests", "Table", "Heads", "gather", "scatter",
           "gather_scatter", "gather_scatter_heads", "extract_permute", "rebuild_permute",
           "check_tables", "check_disjoint", "library_path", "DTYPE_CODES", "load_library"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkvx.so")
_lib = None

DTYPE_CODES = {"f16": 1, "bf16": 2, "fp8": 3, "f32": 4}
OUT_CACHED = 1          # kvx.h KVX_OUT_CACHED
_ELEM = {"f16": 2, "bf16": 2, "fp8": 1, "f32": 4}


class KvxError(RuntimeError):
    """A kvx call returned a nonzero status (nothing was enqueued)."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_str(status)} (status {status})")


class _CLayout(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_kv", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class _CPool(ctypes.Structure):
    _fields_ = [("planes", ctypes.POINTER(ctypes.c_void_p)), ("num_pages", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("slot_stride", ctypes.c_int64),
                ("page_stride", ctypes.c_int64)]


class _CReqs(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("tok_off", ctypes.c_void_p)]


class _CTable(ctypes.Structure):
    _fields_ = [("pg_off", ctypes.c_void_p), ("page_ids", ctypes.c_void_p),
                ("num_ids", ctypes.c_int64)]


class _CHeads(ctypes.Structure):
    _fields_ = [("kv_heads", ctypes.c_int32), ("head0", ctypes.c_int32),
                ("block_layout", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Open libkvx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    P, p64, vp = ctypes.POINTER, ctypes.c_int64, ctypes.c_void_p
    u32 = ctypes.c_uint32
    lib.kvx_gather.argtypes = [P(_CLayout), P(_CPool), P(_CTable), P(_CReqs), vp, p64, vp, u32,
                               vp]
    lib.kvx_scatter.argtypes = [P(_CLayout), vp, p64, P(_CReqs), P(_CPool), P(_CTable), vp, vp]
    lib.kvx_gather_scatter.argtypes = [P(_CLayout), P(_CPool), P(_CTable), P(_CReqs),
                                       P(_CPool), P(_CTable), vp, vp]
    lib.kvx_gather_scatter_heads.argtypes = [P(_CLayout), P(_CPool), P(_CTable), P(_CHeads),
                                             P(_CReqs), P(_CPool), P(_CTable), P(_CHeads), vp,
                                             vp]
    lib.kvx_extract_permute.argtypes = [P(_CLayout), P(vp), p64, p64, vp, p64, u32, vp]
    lib.kvx_rebuild_permute.argtypes = [P(_CLayout), vp, p64, p64, P(vp), p64, u32, vp]
    for f in (lib.kvx_gather, lib.kvx_scatter, lib.kvx_gather_scatter,
              lib.kvx_gather_scatter_heads, lib.kvx_extract_permute, lib.kvx_rebuild_permute):
        f.restype = ctypes.c_int
    lib.kvx_check_tables.argtypes = [ctypes.c_int32, p64, vp, vp, vp, p64, p64, ctypes.c_int32,
                                     ctypes.c_int32, P(p64)]
    lib.kvx_check_tables.restype = ctypes.c_int
    lib.kvx_check_disjoint.argtypes = [P(_CLayout), P(_CReqs), P(_CPool), P(_CTable), P(_CPool),
                                       P(_CTable), vp, p64, P(p64)]
    lib.kvx_check_disjoint.restype = ctypes.c_int
    lib.kvx_status_str.argtypes = [ctypes.c_int]
    lib.kvx_status_str.restype = ctypes.c_char_p
    lib.kvx_abi_version.argtypes = []
    lib.kvx_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _status_str(status: int) -> str:
    try:
        return load_library().kvx_status_str(status).decode()
    except Exception:  # noqa: BLE001 -- only used to format an error message
        return "unknown"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise KvxError(status, what)


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    raise TypeError(f"expected a tensor or a device pointer, got {type(x)}")


def _nbytes(x) -> int:
    return x.numel() * x.element_size() if isinstance(x, torch.Tensor) else 0


def _on_device(*args) -> None:
    """Every torch tensor a data-movement call will hand to the kernels must
    live on the GPU (a host pointer there would fault): pools' plane tensors,
    tables, token offsets, staging, counters.  Raw integer pointers are the
    caller's responsibility."""
    for a in args:
        if a is None or isinstance(a, int):
            continue
        if isinstance(a, Pool):
            _on_device(*(a._keep if isinstance(a._keep, (list, tuple)) else [a._keep]))
        elif isinstance(a, Table):
            _on_device(a.pg_off, a.page_ids)
        elif isinstance(a, Requests):
            _on_device(a.tok_off)
        elif isinstance(a, (list, tuple)):
            _on_device(*a)
        elif isinstance(a, torch.Tensor):
            if not a.is_cuda:
                raise ValueError("kvx data-movement calls take device tensors; got a "
                                 f"{a.device} tensor of shape {tuple(a.shape)}")


def _dense(what: str, t) -> None:
    """The library addresses a buffer from its base pointer and byte count,
    so a strided view would be read or written as if it were contiguous (and
    the bytes between its elements overwritten): refuse it."""
    if isinstance(t, torch.Tensor) and not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous tensor (got strides {t.stride()} "
                         f"for shape {tuple(t.shape)})")


def _planes_dense(what: str, planes) -> None:
    """Each plane of a tensor whose first dimension indexes planes, or each
    tensor of a plane list, must be contiguous."""
    if isinstance(planes, torch.Tensor):
        if planes.dim() > 0 and planes.shape[0] > 0:
            _dense(f"each plane of {what}", planes[0])
    elif isinstance(planes, (list, tuple)):
        for p in planes:
            _dense(f"each plane of {what}", p)


def _counter(skipped) -> None:
    if skipped is None or isinstance(skipped, int):
        return
    if skipped.dtype not in (torch.int64, torch.uint64) or skipped.numel() < 1:
        raise ValueError("skipped must be a tensor of at least one int64 or uint64 element "
                         "(the library adds to its first element)")


def _bytes_from(t: torch.Tensor, ptr: int) -> int:
    """Bytes of t's storage from address ptr to the storage's end."""
    st = t.untyped_storage()
    return st.data_ptr() + st.nbytes() - ptr


def _plane_tensors(keep, ptrs):
    """(tensor, plane address) for each plane address that lies inside the
    storage of one of the tensors in `keep` (a tensor or a sequence of them
    and raw pointers); addresses in no kept tensor are the caller's own."""
    tensors = [keep] if isinstance(keep, torch.Tensor) else \
        [t for t in keep if isinstance(t, torch.Tensor)]
    spans = {}
    for t in tensors:                       # one entry per storage
        st = t.untyped_storage()
        spans.setdefault(st.data_ptr(), (st.data_ptr() + st.nbytes(), t))
    los = sorted(spans)
    out = []
    for a in ptrs:
        if a is None:
            continue
        i = bisect.bisect_right(los, a) - 1     # the storage starting at or below a
        if i >= 0 and a < spans[los[i]][0]:
            out.append((spans[los[i]][1], a))
    return out


def _min_plane_bytes(planes, ptrs) -> Optional[int]:
    """Fewest bytes any tensor-backed plane holds from its base to the end of
    its tensor's storage (None when no plane is tensor-backed).  ptrs None:
    `planes` is one tensor whose first dimension indexes the planes, and the
    plane furthest into the storage, the shortest, decides.  Otherwise each
    plane address in `ptrs` is matched with the tensor of `planes` (a tensor
    or a sequence of tensors and pointers) whose storage holds it."""
    if ptrs is None:
        n = planes.shape[0]
        if n == 0:
            return None
        step = planes.stride(0) * planes.element_size()
        last = planes.data_ptr() + max(0, (n - 1) * step)
        st = planes.untyped_storage()
        return st.data_ptr() + st.nbytes() - last
    m = None
    if not isinstance(planes, torch.Tensor) and len(planes) == len(ptrs) and \
            all(isinstance(e, torch.Tensor) for e in planes):
        # one tensor per plane, ptrs[q] its base: each plane against its own storage
        for e, ptr in zip(planes, ptrs):
            st = e.untyped_storage()
            b = st.data_ptr() + st.nbytes() - ptr
            m = b if m is None else min(m, b)
        return m
    for t, ptr in _plane_tensors(planes, ptrs):
        b = _bytes_from(t, ptr)
        m = b if m is None else min(m, b)
    return m


def _check_pool(what: str, layout: "Layout", pool: "Pool", whole_pages: bool = False) -> None:
    """The C side reads planes[q] for every plane of the layout and addresses
    each plane from its base: the pool must have exactly layout.planes planes,
    and each tensor-backed plane must hold every byte a row of the pool can
    occupy -- (num_pages - 1) * page_stride + (page_size - 1) * slot_stride +
    R from its base, or num_pages * page_size * slot_stride for a pool of a
    head-sliced copy (whole pages) -- inside its tensor's storage."""
    if pool.num_planes != layout.planes:
        raise ValueError(f"{what}: the pool has {pool.num_planes} planes, the layout "
                         f"{layout.planes}")
    if pool.num_pages <= 0 or pool.page_size <= 0:
        return
    if whole_pages:
        need = pool.num_pages * pool.page_size * pool.slot_stride
    else:
        ps = pool.page_stride or pool.page_size * pool.slot_stride
        need = ((pool.num_pages - 1) * ps + (pool.page_size - 1) * pool.slot_stride
                + layout.row_bytes)
    if pool._min_bytes is not None and pool._min_bytes < need:
        raise ValueError(f"{what}: a plane holds {pool._min_bytes} bytes from its base, the "
                         f"pool's pages need {need}")


def _check_hf(layout: "Layout", hf_planes, s_cap: int, arr) -> None:
    """Extract / rebuild: one [1, H, s_cap, D] plane per plane of the layout,
    each tensor-backed plane holding H * s_cap * D elements from its base
    (`arr`: the planes' base pointers)."""
    n = hf_planes.shape[0] if isinstance(hf_planes, torch.Tensor) else len(hf_planes)
    if n != layout.planes:
        raise ValueError(f"hf_planes has {n} planes, the layout {layout.planes}")
    need = layout.kv_heads * max(int(s_cap), 0) * layout.head_dim * _ELEM[layout.dtype]
    if need == 0:
        return
    have = _min_plane_bytes(hf_planes, None if isinstance(hf_planes, torch.Tensor)
                            else list(arr)[:n])
    if have is not None and have < need:
        raise ValueError(f"an hf plane holds {have} bytes from its base, [1, H, s_cap, D] "
                         f"needs {need}")


def _check_table(what: str, table: "Table", reqs: "Requests") -> None:
    if table.pg_off.dim() != 1 or table.pg_off.numel() < reqs.num_reqs + 1:
        raise ValueError(f"{what}: pg_off needs num_reqs + 1 = {reqs.num_reqs + 1} entries, "
                         f"got {table.pg_off.numel()}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class Layout:
    """Row shape: Q = num_layers * num_kv planes of kv_heads x head_dim elements."""

    def __init__(self, num_layers: int, num_kv: int, kv_heads: int, head_dim: int,
                 dtype: str = "bf16"):
        if dtype not in DTYPE_CODES:
            raise ValueError(f"dtype must be one of {sorted(DTYPE_CODES)}")
        self.num_layers, self.num_kv, self.kv_heads, self.head_dim = (
            num_layers, num_kv, kv_heads, head_dim)
        self.dtype = dtype
        self._c = _CLayout(num_layers, num_kv, kv_heads, head_dim, DTYPE_CODES[dtype])

    @property
    def planes(self) -> int:
        return self.num_layers * self.num_kv

    @property
    def row_bytes(self) -> int:
        return self.kv_heads * self.head_dim * _ELEM[self.dtype]


def _plane_array(planes) -> ctypes.Array:
    """Host array of plane base pointers: planes[q] of a tensor (from its base
    pointer and first-dimension stride, without indexing it Q times), or the
    given tensors / pointers."""
    if isinstance(planes, torch.Tensor):
        base, step = planes.data_ptr(), planes.stride(0) * planes.element_size()
        n = planes.shape[0]
        if n > 0:
            a = np.arange(n, dtype=np.uint64) * np.uint64(step) + np.uint64(base)
            return (ctypes.c_void_p * n).from_buffer_copy(a.tobytes())
        ptrs = []
    else:
        ptrs = [_ptr(p) for p in planes]
    return (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)


class Pool:
    """A paged pool: Q plane base pointers, num_pages pages of page_size slots.

    ``planes`` is a device tensor whose first dimension indexes planes (each
    ``planes[q]`` starting at slot 0), or a sequence of tensors / device
    pointers, one per plane.  ``slot_stride`` (bytes between the rows of a
    page) defaults to the row size; ``page_stride`` (bytes between the pages
    of a plane) defaults to ``page_size * slot_stride`` and is the block
    length when a tensor's blocks hold several planes' pages.
    ``keep``: for planes given as pointers, the tensor (or tensors) that hold
    them; each plane's extent is checked inside the tensor that holds it.
    The pool keeps references to its tensors; the caller keeps them unchanged
    until the stream has passed every call that uses them.
    """

    def __init__(self, planes: Union[torch.Tensor, Sequence], num_pages: int,
                 page_size: int = 1, slot_stride: Optional[int] = None,
                 row_bytes: Optional[int] = None, page_stride: int = 0,
                 keep: Union[None, torch.Tensor, Sequence[torch.Tensor]] = None):
        self._keep = planes if keep is None else keep
        self._arr = _plane_array(planes)
        self.num_planes = planes.shape[0] if isinstance(planes, torch.Tensor) else len(planes)
        if slot_stride is None:
            if row_bytes is None:
                if not isinstance(planes, torch.Tensor):
                    raise ValueError("slot_stride or row_bytes is needed for pointer lists")
                _planes_dense("a pool tensor (pass slot_stride for strided slots)", planes)
                slots = num_pages * page_size
                if slots <= 0:
                    raise ValueError("an empty pool needs an explicit slot_stride")
                row_bytes = planes[0].numel() * planes.element_size() // slots
            slot_stride = row_bytes
        self.num_pages, self.page_size, self.slot_stride = num_pages, page_size, slot_stride
        self.page_stride = page_stride
        # the extent check of every call compares with this (the pool's
        # tensors stay as they are while the pool is in use)
        self._min_bytes = (_min_plane_bytes(planes, None) if isinstance(planes, torch.Tensor)
                           else _min_plane_bytes(self._keep,
                                                 list(self._arr)[:self.num_planes]))
        self._c = _CPool(ctypes.cast(self._arr, ctypes.POINTER(ctypes.c_void_p)), num_pages,
                         page_size, slot_stride, page_stride)


class Requests:
    """A batch: device int64 ``tok_off`` [num_reqs + 1] and its last entry."""

    def __init__(self, tok_off: torch.Tensor, total_tokens: int):
        if tok_off.dtype != torch.int64 or tok_off.dim() != 1:
            raise ValueError("tok_off must be a 1-D int64 tensor")
        _dense("tok_off", tok_off)
        self.tok_off = tok_off
        self.num_reqs = tok_off.numel() - 1
        self.total_tokens = int(total_tokens)
        self._c = _CReqs(self.num_reqs, self.total_tokens, _ptr(tok_off))


class Table:
    """Per-request page ids in one pool: device int64 ``pg_off`` and int32 ids."""

    def __init__(self, pg_off: torch.Tensor, page_ids: torch.Tensor):
        if pg_off.dtype != torch.int64 or page_ids.dtype != torch.int32:
            raise ValueError("pg_off must be int64 and page_ids int32")
        _dense("pg_off", pg_off)
        _dense("page_ids", page_ids)
        self.pg_off, self.page_ids = pg_off, page_ids
        self._c = _CTable(_ptr(pg_off), _ptr(page_ids) if page_ids.numel() else 0,
                          page_ids.numel())


class Heads:
    """The head slice one pool side of a head-sliced copy reads or writes:
    ``kv_heads`` per token row in that pool, slice start ``head0``, and the
    block layout, "nhd" ([page_size][H][D]) or "hnd" ([H][page_size][D])."""

    def __init__(self, kv_heads: int, head0: int = 0, block_layout: str = "nhd"):
        if block_layout not in ("nhd", "hnd"):
            raise ValueError('block_layout is "nhd" or "hnd"')
        self.kv_heads, self.head0, self.block_layout = kv_heads, head0, block_layout
        self._c = _CHeads(kv_heads, head0, 0 if block_layout == "nhd" else 1)


def gather(layout: Layout, src: Pool, src_table: Table, reqs: Requests, staging: torch.Tensor,
           skipped: Optional[torch.Tensor] = None, stream=None, cached_out: bool = False) -> None:
    """Pool -> contiguous staging [request][plane][token][H][D] (kvx_gather).
    ``cached_out``: the staging is read back soon on this GPU, so write it
    with ordinary stores (KVX_OUT_CACHED) instead of nontemporal ones."""
    _check_pool("src", layout, src)
    _check_table("src_table", src_table, reqs)
    _dense("staging", staging)
    _counter(skipped)
    _on_device(src, src_table, reqs, staging, skipped)
    lib = load_library()
    _check(lib.kvx_gather(ctypes.byref(layout._c), ctypes.byref(src._c),
                          ctypes.byref(src_table._c), ctypes.byref(reqs._c), _ptr(staging),
                          _nbytes(staging), _ptr(skipped), OUT_CACHED if cached_out else 0,
                          _stream(stream)), "kvx_gather")


def scatter(layout: Layout, staging: torch.Tensor, reqs: Requests, dst: Pool, dst_table: Table,
            skipped: Optional[torch.Tensor] = None, stream=None) -> None:
    """Contiguous staging -> pool (kvx_scatter)."""
    _check_pool("dst", layout, dst)
    _check_table("dst_table", dst_table, reqs)
    _dense("staging", staging)
    _counter(skipped)
    _on_device(staging, reqs, dst, dst_table, skipped)
    lib = load_library()
    _check(lib.kvx_scatter(ctypes.byref(layout._c), _ptr(staging), _nbytes(staging),
                           ctypes.byref(reqs._c), ctypes.byref(dst._c),
                           ctypes.byref(dst_table._c), _ptr(skipped), _stream(stream)),
           "kvx_scatter")


def gather_scatter(layout: Layout, src: Pool, src_table: Table, reqs: Requests, dst: Pool,
                   dst_table: Table, skipped: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Pool -> pool, row by row, no staging (kvx_gather_scatter)."""
    _check_pool("src", layout, src)
    _check_pool("dst", layout, dst)
    _check_table("src_table", src_table, reqs)
    _check_table("dst_table", dst_table, reqs)
    _counter(skipped)
    _on_device(src, src_table, reqs, dst, dst_table, skipped)
    lib = load_library()
    _check(lib.kvx_gather_scatter(ctypes.byref(layout._c), ctypes.byref(src._c),
                                  ctypes.byref(src_table._c), ctypes.byref(reqs._c),
                                  ctypes.byref(dst._c), ctypes.byref(dst_table._c),
                                  _ptr(skipped), _stream(stream)), "kvx_gather_scatter")


def gather_scatter_heads(layout: Layout, src: Pool, src_table: Table, src_heads: Heads,
                         reqs: Requests, dst: Pool, dst_table: Table, dst_heads: Heads,
                         skipped: Optional[torch.Tensor] = None, stream=None) -> None:
    """Pool -> pool, layout.kv_heads heads of every token row, from heads
    src_heads.head0.. to dst_heads.head0.. (kvx_gather_scatter_heads).  The
    pools' slot_stride is the bytes of one token row in that pool."""
    _check_pool("src", layout, src, whole_pages=True)
    _check_pool("dst", layout, dst, whole_pages=True)
    _check_table("src_table", src_table, reqs)
    _check_table("dst_table", dst_table, reqs)
    _counter(skipped)
    _on_device(src, src_table, reqs, dst, dst_table, skipped)
    lib = load_library()
    _check(lib.kvx_gather_scatter_heads(ctypes.byref(layout._c), ctypes.byref(src._c),
                                        ctypes.byref(src_table._c), ctypes.byref(src_heads._c),
                                        ctypes.byref(reqs._c), ctypes.byref(dst._c),
                                        ctypes.byref(dst_table._c), ctypes.byref(dst_heads._c),
                                        _ptr(skipped), _stream(stream)),
           "kvx_gather_scatter_heads")


def extract_permute(layout: Layout, hf_planes: Union[torch.Tensor, Sequence], s_cap: int,
                    seq_len: int, out: torch.Tensor, stream=None,
                    cached_out: bool = False) -> None:
    """[1, H, s_cap, D] per plane -> out [Q][seq_len][H][D] (kvx_extract_permute);
    ``cached_out`` as for gather."""
    arr = _plane_array(hf_planes)
    _check_hf(layout, hf_planes, s_cap, arr)
    _planes_dense("hf_planes", hf_planes)
    _dense("out", out)
    _on_device(hf_planes, out)
    lib = load_library()
    _check(lib.kvx_extract_permute(ctypes.byref(layout._c),
                                   ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), s_cap,
                                   seq_len, _ptr(out), _nbytes(out),
                                   OUT_CACHED if cached_out else 0, _stream(stream)),
           "kvx_extract_permute")


def rebuild_permute(layout: Layout, flat: torch.Tensor, seq_len: int,
                    hf_planes: Union[torch.Tensor, Sequence], s_cap: int, stream=None,
                    cached_out: bool = False) -> None:
    """flat [Q][seq_len][H][D] -> [1, H, s_cap, D] per plane (kvx_rebuild_permute);
    ``cached_out`` as for gather."""
    arr = _plane_array(hf_planes)
    _check_hf(layout, hf_planes, s_cap, arr)
    _dense("flat", flat)
    _planes_dense("hf_planes", hf_planes)
    _on_device(flat, hf_planes)
    lib = load_library()
    _check(lib.kvx_rebuild_permute(ctypes.byref(layout._c), _ptr(flat), _nbytes(flat), seq_len,
                                   ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), s_cap,
                                   OUT_CACHED if cached_out else 0, _stream(stream)),
           "kvx_rebuild_permute")


def check_tables(reqs: Requests, table: Table, pool: Pool, as_destination: bool = True) -> None:
    """Debug check of a batch's tables against a pool (kvx_check_tables).
    Copies the device tables to the host (this synchronises) and raises
    KvxError naming the first offending batch token when the offsets are
    inconsistent, a page id is out of range, or -- for a destination --
    two tokens map to the same row."""
    import numpy as np
    tok = np.ascontiguousarray(reqs.tok_off.cpu().numpy(), dtype=np.int64)
    pg = np.ascontiguousarray(table.pg_off.cpu().numpy(), dtype=np.int64)
    ids = np.ascontiguousarray(table.page_ids.cpu().numpy(), dtype=np.int32)
    bad = ctypes.c_int64(-1)
    st = load_library().kvx_check_tables(
        reqs.num_reqs, reqs.total_tokens, tok.ctypes.data, pg.ctypes.data,
        ids.ctypes.data if ids.size else None, ids.size, pool.num_pages, pool.page_size,
        1 if as_destination else 0, ctypes.byref(bad))
    if st != 0:
        raise KvxError(st, f"kvx_check_tables (batch token {bad.value})")


def check_disjoint(layout: Layout, reqs: Requests, src: Optional[Pool] = None,
                   src_table: Optional[Table] = None, dst: Optional[Pool] = None,
                   dst_table: Optional[Table] = None,
                   staging: Optional[torch.Tensor] = None) -> None:
    """Debug check that a gather, scatter or gather-scatter call writes
    pairwise disjoint rows, none of which overlaps a row it reads
    (kvx_check_disjoint).  Pass a pool and its table for each pool side and
    ``staging`` for the other side of a gather or scatter.  Copies the device
    tables to the host (this synchronises) and raises KvxError naming one
    offending batch token."""
    import numpy as np
    tok = np.ascontiguousarray(reqs.tok_off.cpu().numpy(), dtype=np.int64)
    host_reqs = _CReqs(reqs.num_reqs, reqs.total_tokens, tok.ctypes.data)
    keep = [tok]

    def host_table(t):
        if t is None:
            return None
        pg = np.ascontiguousarray(t.pg_off.cpu().numpy(), dtype=np.int64)
        ids = np.ascontiguousarray(t.page_ids.cpu().numpy(), dtype=np.int32)
        keep.extend([pg, ids])
        return ctypes.byref(_CTable(pg.ctypes.data, ids.ctypes.data if ids.size else None,
                                    ids.size))

    bad = ctypes.c_int64(-1)
    st = load_library().kvx_check_disjoint(
        ctypes.byref(layout._c), ctypes.byref(host_reqs),
        ctypes.byref(src._c) if src is not None else None, host_table(src_table),
        ctypes.byref(dst._c) if dst is not None else None, host_table(dst_table),
        _ptr(staging), _nbytes(staging), ctypes.byref(bad))
    if st != 0:
        raise KvxError(st, f"kvx_check_disjoint (batch token {bad.value})")
