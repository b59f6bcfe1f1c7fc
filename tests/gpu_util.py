"""Helpers for the GPU parity tests: upload a workload's tables, run a kvx call
through the C ABI, and run the oracle on host copies of the same bytes."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import scatter_kvx_gather_amd as kvx
import workloads as wl

DEV = torch.device("cuda:0")


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def layout_of(g: wl.Geometry) -> kvx.Layout:
    return kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)


def d(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def d_aligned(a: np.ndarray, align: int) -> torch.Tensor:
    """A device copy of `a` whose first byte sits at a multiple of `align`
    bytes (a view into a slightly larger allocation)."""
    flat = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    buf = torch.empty(flat.size + align, dtype=torch.uint8, device=DEV)
    off = (-buf.data_ptr()) % align
    t = buf[off:off + flat.size]
    t.copy_(torch.from_numpy(flat))
    assert t.data_ptr() % align == 0
    return t.view(a.shape)


def table(side: wl.Side) -> kvx.Table:
    return kvx.Table(d(side.pg_off.astype(np.int64)), d(side.ids.astype(np.int32)))


def requests(case: wl.PagedCase) -> kvx.Requests:
    return kvx.Requests(d(case.tok_off.astype(np.int64)), case.total_tokens)


def host_planes(pool: np.ndarray):
    """[Q][slots][R] uint8 host pool -> list of per-plane byte views."""
    return [pool[q].reshape(-1) for q in range(pool.shape[0])]


def oracle_gather(case, src_h, staging_h, nthreads=1):
    g = case.geom
    return oracle.gather(host_planes(src_h), g.row_bytes, case.src.page_size, case.src.num_pages,
                         g.row_bytes, case.tok_off, case.src.pg_off, case.src.ids, staging_h,
                         nthreads)


def oracle_scatter(case, staging_h, dst_h, nthreads=1):
    g = case.geom
    return oracle.scatter(staging_h, g.row_bytes, case.tok_off, case.dst.pg_off, case.dst.ids,
                          host_planes(dst_h), g.row_bytes, case.dst.page_size,
                          case.dst.num_pages, nthreads)


def oracle_gather_scatter(case, src_h, dst_h, nthreads=1):
    g = case.geom
    R = g.row_bytes
    return oracle.gather_scatter(host_planes(src_h), R, case.src.page_size, case.src.num_pages,
                                 case.src.pg_off, case.src.ids, R, case.tok_off,
                                 host_planes(dst_h), R, case.dst.page_size, case.dst.num_pages,
                                 case.dst.pg_off, case.dst.ids, nthreads)


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    idx = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
    if idx.size == 0:
        return "equal"
    return f"{idx.size} bytes differ, first at flat index {idx[0]}"


def assert_bytes_equal(got: np.ndarray, exp: np.ndarray, what: str):
    if not np.array_equal(got, exp):
        raise AssertionError(f"{what}: {first_mismatch(got, exp)}")
