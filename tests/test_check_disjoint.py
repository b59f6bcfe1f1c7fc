"""kvx_check_disjoint on the host (no GPU): the overlap checker against a
brute-force pairwise comparison of every row a call reads and writes.

Plane pointers and staging are fake addresses: the checker compares them as
numbers and never dereferences them."""
import ctypes

import numpy as np
import pytest

import scatter_kvx_gather_amd as kvx
import workloads as wl

OK, E_NULL, E_SHAPE, E_UNSUPPORTED, E_DUPLICATE, E_OVERLAP = 0, 1, 2, 6, 8, 9
BASE = 0x7F0000000000
PLANE_GAP = 1 << 24


class Side:
    """A pool side: fake plane bases plus a page table (host arrays)."""

    def __init__(self, side, bases, stride, page_stride=0):
        self.side, self.bases, self.stride = side, [int(b) for b in bases], int(stride)
        self.page_stride = int(page_stride) or side.page_size * self.stride
        self._planes = (ctypes.c_void_p * len(self.bases))(*self.bases)
        self._pg = np.ascontiguousarray(side.pg_off, dtype=np.int64)
        self._ids = np.ascontiguousarray(side.ids, dtype=np.int32)
        self.pool = kvx._CPool(ctypes.cast(self._planes, ctypes.POINTER(ctypes.c_void_p)),
                               side.num_pages, side.page_size, self.stride, int(page_stride))
        self.table = kvx._CTable(self._pg.ctypes.data,
                                 self._ids.ctypes.data if self._ids.size else None,
                                 self._ids.size)

    def slot(self, r, k):
        """Slot of token k of request r, or None where the call skips it."""
        s = self.side
        idx = int(s.pg_off[r]) + k // s.page_size
        if idx < 0 or idx >= s.ids.size:
            return None
        page = int(s.ids[idx])
        if page < 0 or page >= s.num_pages:
            return None
        return page * s.page_size + k % s.page_size

    def offset(self, slot):
        """Byte offset of a slot from its plane's base."""
        return ((slot // self.side.page_size) * self.page_stride
                + (slot % self.side.page_size) * self.stride)


def call(geom, tok_off, src, dst, staging=0, staging_bytes=0):
    lib = kvx.load_library()
    lay = kvx._CLayout(geom.num_layers, geom.num_kv, geom.kv_heads, geom.head_dim,
                       {"f16": 1, "bf16": 2, "fp8": 3, "f32": 4}[geom.dtype])
    tok = np.ascontiguousarray(tok_off, dtype=np.int64)
    reqs = kvx._CReqs(tok.size - 1, int(tok[-1]), tok.ctypes.data)
    bad = ctypes.c_int64(-7)
    st = lib.kvx_check_disjoint(
        ctypes.byref(lay), ctypes.byref(reqs),
        ctypes.byref(src.pool) if src else None, ctypes.byref(src.table) if src else None,
        ctypes.byref(dst.pool) if dst else None, ctypes.byref(dst.table) if dst else None,
        staging or None, staging_bytes, ctypes.byref(bad))
    return st, bad.value


def brute(geom, tok_off, src, dst, staging=0):
    """(status, tokens at fault) from all pairs of rows."""
    Q, R = geom.planes, geom.row_bytes
    reads, writes = [], []
    for r in range(len(tok_off) - 1):
        off, n = int(tok_off[r]), int(tok_off[r + 1] - tok_off[r])
        for k in range(n):
            ss = src.slot(r, k) if src else -1
            ds = dst.slot(r, k) if dst else -1
            if ss is None or ds is None:
                continue
            for q in range(Q):
                stage = staging + ((off * Q + q * n + k) * R)
                lo_r = src.bases[q] + src.offset(ss) if src else stage
                lo_w = dst.bases[q] + dst.offset(ds) if dst else stage
                reads.append((lo_r, lo_r + R, off + k))
                writes.append((lo_w, lo_w + R, off + k))
    dup = {t for i, (a, b, t) in enumerate(writes) for (c, e, u) in writes[:i] if a < e and c < b}
    dup |= {u for i, (a, b, t) in enumerate(writes) for (c, e, u) in writes[:i] if a < e and c < b}
    if dup:
        return E_DUPLICATE, dup
    ov = {t for (a, b, t) in writes for (c, e, _) in reads if a < e and c < b}
    return (E_OVERLAP, ov) if ov else (OK, set())


def check(geom, case, src, dst, staging=0, nbytes=0):
    st, bad = call(geom, case.tok_off, src, dst, staging, nbytes)
    exp, fault = brute(geom, case.tok_off, src, dst, staging)
    assert st == exp, (case.name, st, exp)
    if st == OK:
        assert bad == -1
    else:
        assert bad in fault, (case.name, bad, sorted(fault)[:10])
    return st


def planes(Q, base, gap=PLANE_GAP):
    return [base + q * gap for q in range(Q)]


@pytest.mark.parametrize("seed", range(24))
def test_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    page = int(rng.choice([1, 2, 4]))
    case = wl.random_case(9500 + seed, max_reqs=4, max_len=24, src_page=page, dst_page=page,
                          oor_frac=0.1 if seed % 3 == 0 else 0.0, slack_pages=3)
    g = case.geom
    Q, R = g.planes, g.row_bytes
    nst = case.total_tokens * Q * R
    seen = set()
    # gather-scatter between two separate pools: only planted duplicates fail
    a = Side(case.src, planes(Q, BASE), R)
    b = Side(case.dst, planes(Q, BASE + (1 << 36)), R)
    seen.add(check(g, case, a, b))
    if case.dst.ids.size > 1:
        ids = case.dst.ids.copy()
        ids[-1] = ids[0]
        dup = wl.Side(case.dst.num_pages, case.dst.page_size, case.dst.pg_off, ids)
        seen.add(check(g, case, a, Side(dup, planes(Q, BASE + (1 << 36)), R)))
    # gather-scatter inside one pool: source and destination slots may meet
    same = Side(case.dst, planes(Q, BASE), R)
    seen.add(check(g, case, a, same))
    # token-major planes (plane q at q * R, stride Q * R) are disjoint; a
    # stride one vector short makes neighbouring planes' rows overlap
    seen.add(check(g, case, a, Side(case.dst, planes(Q, BASE + (1 << 36), R), Q * R)))
    if Q > 1:
        seen.add(check(g, case, a, Side(case.dst, planes(Q, BASE + (1 << 36), R - 16), Q * R)))
    # gather into staging placed in the middle of the source's plane 0, and
    # far away; scatter from staging placed over the destination
    mid = BASE + (int(rng.integers(0, 8)) * R)
    seen.add(check(g, case, a, None, staging=mid, nbytes=nst))
    seen.add(check(g, case, a, None, staging=BASE + (1 << 38), nbytes=nst))
    seen.add(check(g, case, None, b, staging=BASE + (1 << 36) + 16 * R, nbytes=nst))
    assert OK in seen


@pytest.mark.parametrize("seed", range(8))
def test_index_faults_against_brute_force(seed):
    """Page-table offsets that send lookups outside the page-id array or into
    another request's list: those tokens are left out on both sides."""
    case = wl.random_case(9700 + seed, max_reqs=5, max_len=20, src_page=1 + seed % 3,
                          dst_page=1 + seed % 2, slack_pages=3, index_faults=True)
    g = case.geom
    Q, R = g.planes, g.row_bytes
    a = Side(case.src, planes(Q, BASE), R)
    b = Side(case.dst, planes(Q, BASE + (1 << 36)), R)
    check(g, case, a, b)
    check(g, case, a, None, staging=BASE + (1 << 38), nbytes=case.total_tokens * Q * R)
    check(g, case, a, Side(case.dst, planes(Q, BASE), R))


def test_offsets_at_the_ends_of_int64():
    """Requests whose page lists start at the ends of the int64 range: the
    index pg_off[r] + t / B runs past 2**63 - 1 or starts at -2**63, and
    those tokens are left out (the index is a plain integer; it does not
    wrap).  kvx_check_tables refuses such offsets as a contract violation
    (KVX_E_SHAPE), again without forming a sum that overflows."""
    i64max, i64min = (1 << 63) - 1, -(1 << 63)
    lens = [3, 6, 6, 2]
    tok = wl.csr_from_lengths(lens)
    ids = np.array([4, 1, 6, 3, 0, 5], np.int32)
    g = wl.Geometry(1, 2, 1, 8)
    Q, R = g.planes, g.row_bytes
    for B in (1, 2):
        src = wl.Side(8, B, np.array([0, i64max - 1, i64min, 2, 6], np.int64), ids)
        dst = wl.Side(8, B, np.array([3, i64min + 1, i64max, 0, 6], np.int64), ids[::-1].copy())
        case = wl.PagedCase(f"ends{B}", g, tok, src, dst, 0, 0, 0)
        a = Side(src, planes(Q, BASE), R)
        b = Side(dst, planes(Q, BASE + (1 << 36)), R)
        assert check(g, case, a, b) in (OK, E_DUPLICATE)
        check(g, case, a, None, staging=BASE + (1 << 38), nbytes=case.total_tokens * Q * R)
        check(g, case, None, b, staging=BASE + (1 << 38), nbytes=case.total_tokens * Q * R)
        lib = kvx.load_library()
        bad = ctypes.c_int64(-7)
        for side in (src, dst):
            pg = np.ascontiguousarray(side.pg_off, np.int64)
            st = lib.kvx_check_tables(len(lens), int(tok[-1]), tok.ctypes.data, pg.ctypes.data,
                                      side.ids.ctypes.data, side.ids.size, side.num_pages, B, 1,
                                      ctypes.byref(bad))
            assert st == E_SHAPE and bad.value == 0, (B, st, bad.value)   # request 0 ends out of range


@pytest.mark.parametrize("tok_off,total", [([0, 9 + 7], 7), ([0, 5, 3, 7], 7), ([1, 7], 7),
                                           ([0, 6], 7)])
def test_token_offsets_breaking_the_contract(tok_off, total):
    """A token CSR that runs past total_tokens, decreases, starts above 0 or
    ends short is refused with KVX_E_SHAPE before anything is indexed by it."""
    g = wl.Geometry(1, 2, 1, 8)
    side = wl.Side(16, 1, np.zeros(len(tok_off), np.int64), np.arange(16, dtype=np.int32))
    a = Side(side, planes(g.planes, BASE), g.row_bytes)
    b = Side(side, planes(g.planes, BASE + (1 << 36)), g.row_bytes)
    lib = kvx.load_library()
    lay = kvx._CLayout(1, 2, 1, 8, 2)
    tok = np.ascontiguousarray(tok_off, dtype=np.int64)
    reqs = kvx._CReqs(tok.size - 1, total, tok.ctypes.data)
    bad = ctypes.c_int64(-7)
    assert lib.kvx_check_disjoint(ctypes.byref(lay), ctypes.byref(reqs), ctypes.byref(a.pool),
                                  ctypes.byref(a.table), ctypes.byref(b.pool),
                                  ctypes.byref(b.table), None, 0, ctypes.byref(bad)) == E_SHAPE
    assert bad.value == -1


def test_workload_tables_are_disjoint():
    # the two-pool workloads, with pools laid out as the bench allocates them
    for case in (wl.qwen15b_128tok_page1(), wl.kv144k_2048tok_page1(5), wl.kv144k_64req_page16()):
        g = case.geom
        Q, R = g.planes, g.row_bytes
        span = case.src.num_slots * R
        a = Side(case.src, planes(Q, BASE, span), R)
        b = Side(case.dst, planes(Q, BASE + Q * span, span), R)
        assert call(g, case.tok_off, a, b) == (OK, -1)
        st, bad = call(g, case.tok_off, a, a)     # the same table read and written: every row
        assert st == E_OVERLAP and 0 <= bad < case.total_tokens
    # the fragmented batch gathered into a staging buffer after its pool
    case = wl.kv144k_32req_fragmented()
    g = case.geom
    span = case.src.num_slots * g.row_bytes
    a = Side(case.src, planes(g.planes, BASE, span), g.row_bytes)
    nst = case.total_tokens * g.token_bytes
    assert call(g, case.tok_off, a, None, BASE + g.planes * span, nst) == (OK, -1)
    st, bad = call(g, case.tok_off, a, None, BASE + span // 2, nst)
    assert st == E_OVERLAP and 0 <= bad < case.total_tokens


def test_arguments():
    case = wl.random_case(9600, max_reqs=3, max_len=10, src_page=1, dst_page=1)
    g = case.geom
    Q, R = g.planes, g.row_bytes
    a = Side(case.src, planes(Q, BASE), R)
    assert call(g, case.tok_off, None, None, BASE, 1 << 30) == (E_UNSUPPORTED, -1)
    nst = case.total_tokens * Q * R
    if nst:
        assert call(g, case.tok_off, a, None, BASE + (1 << 38), nst - 16)[0] == E_SHAPE
        assert call(g, case.tok_off, a, None, 0, nst)[0] == E_NULL
    lay = kvx._CLayout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, 2)
    tok = np.ascontiguousarray(case.tok_off, dtype=np.int64)
    reqs = kvx._CReqs(tok.size - 1, int(tok[-1]) + 1, tok.ctypes.data)   # total disagrees
    lib = kvx.load_library()
    assert lib.kvx_check_disjoint(ctypes.byref(lay), ctypes.byref(reqs), ctypes.byref(a.pool),
                                  ctypes.byref(a.table), None, None, BASE + (1 << 38),
                                  1 << 40, None) == E_SHAPE
    # a pool without its table
    reqs = kvx._CReqs(tok.size - 1, int(tok[-1]), tok.ctypes.data)
    assert lib.kvx_check_disjoint(ctypes.byref(lay), ctypes.byref(reqs), ctypes.byref(a.pool),
                                  None, None, None, BASE, 1 << 40, None) == E_NULL


def test_python_binding():
    import torch
    case = wl.qwen15b_128tok_page1()
    g = case.geom
    lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
    a = torch.empty((g.planes, case.src.num_slots * g.row_bytes), dtype=torch.uint8)
    b = torch.empty((g.planes, case.dst.num_slots * g.row_bytes), dtype=torch.uint8)
    st = torch.empty(case.total_tokens * g.token_bytes, dtype=torch.uint8)
    reqs = kvx.Requests(torch.from_numpy(case.tok_off), case.total_tokens)
    ts = kvx.Table(torch.from_numpy(case.src.pg_off), torch.from_numpy(case.src.ids))
    td = kvx.Table(torch.from_numpy(case.dst.pg_off), torch.from_numpy(case.dst.ids))
    pa, pb = kvx.Pool(a, case.src.num_pages), kvx.Pool(b, case.dst.num_pages)
    kvx.check_disjoint(lay, reqs, pa, ts, pb, td)
    kvx.check_disjoint(lay, reqs, pa, ts, staging=st)
    kvx.check_disjoint(lay, reqs, dst=pb, dst_table=td, staging=st)
    with pytest.raises(kvx.KvxError) as e:
        kvx.check_disjoint(lay, reqs, pa, ts, pa, ts)
    assert e.value.status == E_OVERLAP
    with pytest.raises(kvx.KvxError) as e:               # staging laid over the source pool
        kvx.check_disjoint(lay, reqs, pa, ts, staging=a.view(-1)[:st.numel()])
    assert e.value.status == E_OVERLAP


@pytest.mark.parametrize("v_offset_rows,expect", [(4, OK), (2, E_DUPLICATE), (1, E_DUPLICATE)])
def test_blocks_holding_k_and_v(v_offset_rows, expect):
    """Destination blocks hold a layer's K and V pages together ([blocks][2][B]
    rows, page stride 2 * B * R): V planes B rows after K do not collide;
    placed fewer rows after K they overlap K's rows of the same block."""
    g = wl.Geometry(2, 2, 1, 8, "bf16")
    R, B = g.row_bytes, 4
    case = wl.random_case(4242, geom=g, max_reqs=3, max_len=12, src_page=1, dst_page=B,
                          slack_pages=2)
    src = Side(case.src, [BASE + q * PLANE_GAP for q in range(g.planes)], R)
    layer = [BASE + (16 + l) * PLANE_GAP for l in range(g.num_layers)]
    dst_bases = [layer[q // 2] + (q % 2) * v_offset_rows * R for q in range(g.planes)]
    dst = Side(case.dst, dst_bases, R, page_stride=2 * B * R)
    st, bad = call(g, case.tok_off, src, dst)
    want, toks = brute(g, case.tok_off, src, dst)
    assert st == want == expect
    if st != OK:
        assert bad in toks
