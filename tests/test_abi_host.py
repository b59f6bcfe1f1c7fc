"""The C-ABI library on the host (no GPU): it loads, exports every function
include/kvx.h declares, and rejects bad arguments with the documented status
before anything reaches the GPU (validation never touches a device pointer)."""
import ctypes
import os
import re
import subprocess

import pytest

import scatter_kvx_gather_amd as kvx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvx.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_RANGE = 0, 1, 2, 3, 4, 5
E_UNSUPPORTED = 6

# Fake, 16-byte aligned "device" addresses: validation only looks at their
# values, never dereferences them, and every call below fails validation.
A = 0x7F0000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvx_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert names == sorted(["kvx_gather", "kvx_scatter", "kvx_gather_scatter",
                            "kvx_gather_scatter_heads", "kvx_extract_permute",
                            "kvx_rebuild_permute", "kvx_check_tables", "kvx_check_disjoint",
                            "kvx_status_str", "kvx_abi_version"])
    lib = ctypes.CDLL(kvx.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvx.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (kvx_\w+)", out))
    assert set(names) <= exported


def test_abi_version_and_strings():
    lib = kvx.load_library()
    assert lib.kvx_abi_version() == 6
    for s in range(10):
        assert lib.kvx_status_str(s).startswith(b"KVX_")
    assert lib.kvx_status_str(99) == b"unknown kvx_status"


def _layout(L=2, kv=2, H=8, D=128, dtype=2):
    return kvx._CLayout(L, kv, H, D, dtype)


def _pool(Q, num_pages=16, page_size=1, stride=2048, base=A):
    arr = (ctypes.c_void_p * Q)(*[base + q * (1 << 20) for q in range(Q)])
    return kvx._CPool(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), num_pages, page_size,
                      stride), arr


def _reqs(n=1, T=4):
    return kvx._CReqs(n, T, A + 0x100000)


def _table(n_ids=4):
    return kvx._CTable(A + 0x200000, A + 0x300000, n_ids)


def gather(layout, pool, table, reqs, staging=A + 0x400000, nbytes=1 << 30, flags=0):
    lib = kvx.load_library()
    return lib.kvx_gather(ctypes.byref(layout) if layout is not None else None,
                          ctypes.byref(pool) if pool is not None else None,
                          ctypes.byref(table) if table is not None else None,
                          ctypes.byref(reqs) if reqs is not None else None,
                          staging, nbytes, None, flags, None)


def test_gather_validation():
    lay = _layout()
    pool, keep = _pool(4)
    tab, reqs = _table(), _reqs()
    assert gather(None, pool, tab, reqs) == E_NULL
    assert gather(_layout(dtype=9), pool, tab, reqs) == E_DTYPE
    assert gather(_layout(H=1, D=4), pool, tab, reqs) == E_ALIGN            # R = 8 bytes
    assert gather(_layout(kv=3), pool, tab, reqs) == E_SHAPE
    assert gather(_layout(L=0), pool, tab, reqs) == E_SHAPE
    assert gather(_layout(H=512, D=128), pool, tab, reqs) == E_RANGE        # R = 128 KiB
    i32max = (1 << 31) - 1                 # R = heads * dim * 4 past 2^63: refused, not formed
    assert gather(_layout(H=i32max, D=i32max, dtype=4), pool, tab, reqs) == E_RANGE
    assert gather(lay, None, tab, reqs) == E_NULL
    assert gather(lay, pool, None, reqs) == E_NULL
    assert gather(lay, pool, tab, None) == E_NULL
    bad, k2 = _pool(4, base=A + 8)
    assert gather(lay, bad, tab, reqs) == E_ALIGN
    small, k3 = _pool(4, stride=1024)                                         # stride < R
    assert gather(lay, small, tab, reqs) == E_SHAPE
    odd, k4 = _pool(4, stride=2056)
    assert gather(lay, odd, tab, reqs) == E_ALIGN
    assert gather(lay, pool, tab, _reqs(1, -1)) == E_SHAPE
    assert gather(lay, pool, tab, _reqs(0, 5)) == E_SHAPE
    assert gather(lay, pool, tab, reqs, staging=A + 0x400008) == E_ALIGN
    assert gather(lay, pool, tab, reqs, nbytes=4 * 4 * 2048 - 16) == E_SHAPE
    assert gather(lay, pool, tab, reqs, staging=None) == E_NULL
    assert gather(lay, pool, tab, reqs, flags=2) == E_UNSUPPORTED          # unknown output flag
    assert gather(None, pool, tab, reqs, flags=4) == E_UNSUPPORTED
    zero_pages, k5 = _pool(4, num_pages=-1)
    assert gather(lay, zero_pages, tab, reqs) == E_SHAPE
    empty_src, k7 = _pool(4, num_pages=0)                    # no slot to read
    assert gather(lay, empty_src, tab, reqs) == E_SHAPE
    huge, k6 = _pool(4, num_pages=1 << 62, page_size=16)
    assert gather(lay, huge, tab, reqs) == E_RANGE
    # a NULL plane pointer
    arr = (ctypes.c_void_p * 4)(A, None, A, A)
    p = kvx._CPool(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), 16, 1, 2048)
    assert gather(lay, p, tab, reqs) == E_NULL
    # an empty pool (no pages) may come with NULL planes; as the source of a
    # batch with tokens it is still refused (skipped rows read its first slot)
    nulls = (ctypes.c_void_p * 4)(None, None, None, None)
    p0 = kvx._CPool(ctypes.cast(nulls, ctypes.POINTER(ctypes.c_void_p)), 0, 1, 2048)
    assert gather(lay, p0, tab, reqs) == E_SHAPE
    assert gather(lay, p0, _table(0), _reqs(0, 0), staging=None, nbytes=0) == OK


def test_empty_batch_enqueues_nothing():
    # zero tokens: valid, nothing to move, returns before any device query
    lay = _layout()
    pool, keep = _pool(4)
    assert gather(lay, pool, _table(0), _reqs(0, 0), staging=None, nbytes=0) == OK


def test_permute_validation():
    lib = kvx.load_library()
    lay = _layout(L=2, kv=2, H=4, D=128, dtype=1)
    arr = (ctypes.c_void_p * 4)(*[A + q * (1 << 24) for q in range(4)])
    hf = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    need = 4 * 100 * 4 * 256
    ex = lambda s_cap, seq, out=A + 0x1000000, nb=need: lib.kvx_extract_permute(  # noqa: E731
        ctypes.byref(lay), hf, s_cap, seq, out, nb, 0, None)
    assert ex(50, 100) == E_SHAPE                  # seq > s_cap
    assert ex(100, -1) == E_SHAPE
    assert ex(100, 100, nb=need - 16) == E_SHAPE
    assert ex(100, 100, out=A + 4) == E_ALIGN
    assert ex(100, 100, out=None) == E_NULL
    assert lib.kvx_extract_permute(ctypes.byref(lay), None, 100, 100, A, need, 0, None) == E_NULL
    lay_odd = _layout(L=1, kv=2, H=2, D=4, dtype=2)    # head row of 8 bytes
    assert lib.kvx_extract_permute(ctypes.byref(lay_odd), hf, 10, 10, A, 1 << 20, 0, None) == E_ALIGN
    assert lib.kvx_extract_permute(ctypes.byref(lay), hf, 100, 0, None, 0, 0, None) == OK
    # empty HF planes (s_cap = 0, e.g. zero-size tensors) may be NULL; with
    # s_cap > 0 a NULL plane is refused even when seq_len is 0
    nulls = (ctypes.c_void_p * 4)(None, None, None, None)
    hf0 = ctypes.cast(nulls, ctypes.POINTER(ctypes.c_void_p))
    assert lib.kvx_extract_permute(ctypes.byref(lay), hf0, 0, 0, None, 0, 0, None) == OK
    assert lib.kvx_rebuild_permute(ctypes.byref(lay), None, 0, 0, hf0, 0, 0, None) == OK
    assert lib.kvx_extract_permute(ctypes.byref(lay), hf0, 1, 0, None, 0, 0, None) == E_NULL
    assert lib.kvx_rebuild_permute(ctypes.byref(lay), None, 0, 0, hf0, 1, 0, None) == E_NULL
    rb = lambda seq, inp=A + 0x1000000, nb=need, flags=0: lib.kvx_rebuild_permute(  # noqa: E731
        ctypes.byref(lay), inp, nb, seq, hf, 100, flags, None)
    assert rb(101) == E_SHAPE
    assert rb(100, nb=need - 1) == E_SHAPE
    assert rb(100, inp=None) == E_NULL
    # output flags: KVX_OUT_CACHED (1) is the only one; others are refused
    # before anything else is looked at
    assert ex(100, 0) == OK
    assert lib.kvx_extract_permute(ctypes.byref(lay), hf, 100, 0, None, 0, 1, None) == OK
    assert lib.kvx_extract_permute(ctypes.byref(lay), hf, 100, 0, None, 0, 2, None) == \
        E_UNSUPPORTED
    assert rb(0, flags=1) == OK
    assert rb(0, flags=1 << 31) == E_UNSUPPORTED
    # sizes whose products pass int64: refused with KVX_E_RANGE, never formed
    big = 1 << 62
    assert ex(big, 0) == E_RANGE                   # s_cap * H * Db > 2^63
    assert ex(big, big) == E_RANGE                 # seq * H as well
    assert ex(big, 1 << 29) == E_RANGE
    assert lib.kvx_rebuild_permute(ctypes.byref(lay), A, need, 0, hf, big, 0, None) == E_RANGE


def test_heads_validation():
    lib = kvx.load_library()
    lay = _layout(L=1, kv=2, H=2, D=128)                 # slice of 2 heads, Db = 256
    pool, keep = _pool(2, stride=4 * 256)                 # 4 heads per token row
    tab, reqs = _table(), _reqs()

    def call(sh, dh, src=pool):
        return lib.kvx_gather_scatter_heads(ctypes.byref(lay), ctypes.byref(src),
                                            ctypes.byref(tab), ctypes.byref(sh) if sh else None,
                                            ctypes.byref(reqs), ctypes.byref(pool),
                                            ctypes.byref(tab), ctypes.byref(dh), None, None)
    ok = kvx._CHeads(4, 2, 1)
    assert call(None, ok) == E_NULL
    assert call(kvx._CHeads(4, 3, 0), ok) == E_SHAPE          # 3 + 2 > 4 heads
    assert call(kvx._CHeads(4, -1, 0), ok) == E_SHAPE
    assert call(kvx._CHeads(4, 0, 7), ok) == E_SHAPE          # unknown block layout
    assert call(kvx._CHeads(8, 0, 0), ok) == E_SHAPE          # row stride < 8 heads
    empty_src, keep2 = _pool(2, num_pages=0, stride=4 * 256)   # no slot to read
    assert call(ok, ok, src=empty_src) == E_SHAPE
    lay_odd = _layout(L=1, kv=2, H=2, D=4)                    # Db = 8 bytes
    assert lib.kvx_gather_scatter_heads(ctypes.byref(lay_odd), ctypes.byref(pool),
                                        ctypes.byref(tab), ctypes.byref(ok), ctypes.byref(reqs),
                                        ctypes.byref(pool), ctypes.byref(tab),
                                        ctypes.byref(ok), None, None) == E_ALIGN
    empty = _reqs(0, 0)
    assert lib.kvx_gather_scatter_heads(ctypes.byref(lay), ctypes.byref(pool),
                                        ctypes.byref(_table(0)), ctypes.byref(ok),
                                        ctypes.byref(empty), ctypes.byref(pool),
                                        ctypes.byref(_table(0)), ctypes.byref(ok),
                                        None, None) == OK


def test_page_stride_validation():
    """A nonzero page stride: a multiple of 16 and of the slot stride,
    non-negative, and at least (page_size - 1) * slot_stride + R so a plane's
    pages never overlap; the head-sliced copy takes only the default."""
    lib = kvx.load_library()
    lay = _layout()                                       # R = 2048
    tab, empty = _table(0), _reqs(0, 0)

    def pool_with(page_stride, page_size=4):
        p, keep = _pool(4, page_size=page_size)
        p.page_stride = page_stride
        return p, keep

    def gather(p):
        return lib.kvx_gather(ctypes.byref(lay), ctypes.byref(p), ctypes.byref(tab),
                              ctypes.byref(empty), None, 0, None, 0, None)
    for ps, want in [(0, OK), (4 * 2048, OK), (8 * 2048, OK), (3 * 2048 + 2048, OK),
                     (3 * 2048 + 2032, E_SHAPE), (-16, E_SHAPE), (8 * 2048 + 8, E_ALIGN),
                     (8 * 2048 + 16, E_UNSUPPORTED), (1 << 62, E_RANGE)]:
        p, keep = pool_with(ps)
        assert gather(p) == want, ps
    lay_h = _layout(L=1, kv=2, H=2, D=128)
    ok = kvx._CHeads(4, 0, 0)
    for ps, want in [(0, OK), (4 * 1024, OK), (8 * 1024, E_UNSUPPORTED)]:
        p, keep = _pool(2, page_size=4, stride=4 * 256)
        p.page_stride = ps
        st = lib.kvx_gather_scatter_heads(ctypes.byref(lay_h), ctypes.byref(p), ctypes.byref(tab),
                                          ctypes.byref(ok), ctypes.byref(empty), ctypes.byref(p),
                                          ctypes.byref(tab), ctypes.byref(ok), None, None)
        assert st == want, ps


def test_python_binding_raises():
    with pytest.raises(ValueError):
        kvx.Layout(1, 2, 1, 8, dtype="int4")
    err = kvx.KvxError(3, "kvx_gather")
    assert "KVX_E_ALIGN" in str(err) and err.status == 3


def test_flat_copy_row_division_is_exact():
    """The flat copy finds a vector's row as umulhi(i, ceil(2^32 / V)) (V > 1)
    or i itself (V = 1); check it equals i // V for every vector index of a
    chunk, for every row size the library accepts (16 B .. 64 KiB)."""
    import numpy as np
    for V in range(1, 4097):
        R = 16 * V
        if R % 1024 == 0 and R // 1024 in (1, 2, 4, 8, 16):
            continue                                   # wide copy, no division
        U = min(64, max(1, 16384 // R))
        i = np.arange(U * V, dtype=np.uint64)
        if V == 1:
            u = i
        else:
            magic = np.uint64(((1 << 32) + V - 1) // V)
            u = (i * magic) >> np.uint64(32)
        assert np.array_equal(u, i // np.uint64(V)), V


def _check(case_side, tok_off, total, as_dst=True):
    import numpy as np
    import torch
    reqs = kvx.Requests(torch.from_numpy(np.asarray(tok_off, np.int64)), total)
    tab = kvx.Table(torch.from_numpy(np.asarray(case_side.pg_off, np.int64)),
                    torch.from_numpy(np.asarray(case_side.ids, np.int32)))
    pool = kvx.Pool([A], case_side.num_pages, case_side.page_size, slot_stride=16)
    try:
        kvx.check_tables(reqs, tab, pool, as_destination=as_dst)
        return 0, None
    except kvx.KvxError as e:
        return e.status, int(str(e).split("batch token ")[1].split(")")[0])


def _brute(case_side, tok_off, as_dst):
    """First offending batch token by the plain definition."""
    seen = set()
    for r in range(len(tok_off) - 1):
        for t in range(int(tok_off[r + 1] - tok_off[r])):
            page = int(case_side.ids[case_side.pg_off[r] + t // case_side.page_size])
            if not 0 <= page < case_side.num_pages:
                return 5, int(tok_off[r]) + t
            slot = page * case_side.page_size + t % case_side.page_size
            if as_dst and slot in seen:
                return 8, int(tok_off[r]) + t
            seen.add(slot)
    return 0, None


def test_check_tables_against_brute_force():
    import numpy as np
    import workloads as wl
    for seed in range(40):
        case = wl.random_case(9000 + seed, max_reqs=6, max_len=40,
                              oor_frac=0.05 if seed % 4 == 0 else 0.0)
        side = case.dst
        if seed % 3 == 1 and side.ids.size > 2:          # plant a duplicate destination page
            ids = side.ids.copy()
            ids[-1] = ids[0]
            side = wl.Side(side.num_pages, side.page_size, side.pg_off, ids)
        for as_dst in (True, False):
            got = _check(side, case.tok_off, case.total_tokens, as_dst)
            exp = _brute(side, case.tok_off, as_dst)
            assert got == exp, (seed, as_dst, got, exp)
    # the five workloads' destination tables are valid
    for case in (wl.qwen15b_128tok_page1(), wl.kv144k_2048tok_page1(3), wl.kv144k_64req_page16()):
        assert _check(case.dst, case.tok_off, case.total_tokens) == (0, None)


def test_check_tables_shapes():
    import numpy as np
    import workloads as wl
    side = wl.side_from_page_lists([np.array([0, 1]), np.array([2])], 4, 4)
    ok_tok = [0, 5, 9]
    assert _check(side, ok_tok, 9) == (0, None)
    assert _check(side, [0, 5, 9], 10)[0] == 2              # total disagrees
    assert _check(side, [0, 9, 5], 5)[0] == 2               # decreasing
    short = wl.side_from_page_lists([np.array([0]), np.array([2])], 4, 4)
    assert _check(short, ok_tok, 9) == (2, 0)               # request 0 needs 2 pages


def test_header_is_plain_c():
    """include/kvx.h compiles as C99 (with the platform define every HIP host
    program built by a plain C compiler needs)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Wextra", "-Werror",
                        "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I",
                        os.path.join(rocm, "include"), HEADER], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr


def test_binding_refuses_host_tensors():
    """A host tensor never reaches a kernel: the binding refuses it before the
    library is called (on the GPU it would be dereferenced as a device
    address)."""
    import torch
    lay = kvx.Layout(1, 2, 1, 8, "bf16")
    pool = kvx.Pool(torch.zeros((2, 4, 16), dtype=torch.uint8), 4)
    tab = kvx.Table(torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int32))
    reqs = kvx.Requests(torch.tensor([0, 2], dtype=torch.int64), 2)
    st = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensors"):
        kvx.gather(lay, pool, tab, reqs, st)
    with pytest.raises(ValueError, match="device tensors"):
        kvx.scatter(lay, st, reqs, pool, tab)
    with pytest.raises(ValueError, match="device tensors"):
        kvx.gather_scatter(lay, pool, tab, reqs, pool, tab)
    with pytest.raises(ValueError, match="device tensors"):
        kvx.gather_scatter_heads(lay, pool, tab, kvx.Heads(1, 0), reqs, pool, tab,
                                 kvx.Heads(1, 0))
    with pytest.raises(ValueError, match="device tensors"):
        kvx.extract_permute(lay, torch.zeros((2, 16), dtype=torch.uint8), 1, 1, st)
    with pytest.raises(ValueError, match="device tensors"):
        kvx.rebuild_permute(lay, st, 1, [torch.zeros(16, dtype=torch.uint8)] * 2, 1)


def test_binding_refuses_strided_views():
    """The library takes a buffer as base pointer plus byte count, so the
    binding refuses strided views (their elements are not the contiguous
    bytes the kernels would write) and a skip counter it cannot add to."""
    import torch
    lay = kvx.Layout(1, 2, 1, 8, "bf16")
    pool = kvx.Pool(torch.zeros((2, 4, 16), dtype=torch.uint8), 4)
    tab = kvx.Table(torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int32))
    reqs = kvx.Requests(torch.tensor([0, 2], dtype=torch.int64), 2)
    st = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="tok_off must be a contiguous"):
        kvx.Requests(torch.zeros(6, dtype=torch.int64)[::2], 0)
    with pytest.raises(ValueError, match="pg_off must be a contiguous"):
        kvx.Table(torch.zeros(4, dtype=torch.int64)[::2], torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="page_ids must be a contiguous"):
        kvx.Table(torch.zeros(2, dtype=torch.int64), torch.zeros(4, dtype=torch.int32)[::2])
    with pytest.raises(ValueError, match="each plane of a pool tensor"):
        kvx.Pool(torch.zeros((4, 2, 16), dtype=torch.uint8).transpose(0, 1), 4)
    # an explicit slot stride describes a strided (token-major) pool: accepted
    kvx.Pool(torch.zeros((4, 2, 16), dtype=torch.uint8).transpose(0, 1), 4, slot_stride=32)
    strided = torch.zeros(128, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="staging must be a contiguous"):
        kvx.gather(lay, pool, tab, reqs, strided)
    with pytest.raises(ValueError, match="staging must be a contiguous"):
        kvx.scatter(lay, strided, reqs, pool, tab)
    with pytest.raises(ValueError, match="out must be a contiguous"):
        kvx.extract_permute(lay, torch.zeros((2, 16), dtype=torch.uint8), 1, 1, strided)
    with pytest.raises(ValueError, match="flat must be a contiguous"):
        kvx.rebuild_permute(lay, strided, 1, torch.zeros((2, 16), dtype=torch.uint8), 1)
    with pytest.raises(ValueError, match="each plane of hf_planes"):
        kvx.extract_permute(lay, torch.zeros((16, 2), dtype=torch.uint8).t(), 1, 1, st)
    with pytest.raises(ValueError, match="skipped must be"):
        kvx.gather(lay, pool, tab, reqs, st, skipped=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="skipped must be"):
        kvx.gather_scatter(lay, pool, tab, reqs, pool, tab,
                           skipped=torch.zeros(0, dtype=torch.int64))


def test_binding_checks_plane_counts_and_extents():
    """The C side reads one plane pointer per plane of the layout and
    addresses each plane from its base, so the binding refuses a pool or an
    HF plane list with another plane count, a tensor-backed plane whose
    storage ends before the pool's last row (or last whole page, for a
    head-sliced copy) or before [1, H, s_cap, D], and a page-offset array
    shorter than num_reqs + 1 -- before anything reaches the library."""
    import torch
    lay = kvx.Layout(1, 2, 1, 8, "bf16")                      # Q = 2, R = 16
    reqs = kvx.Requests(torch.tensor([0, 2], dtype=torch.int64), 2)
    tab = kvx.Table(torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int32))
    st = torch.zeros(64, dtype=torch.uint8)
    three = kvx.Pool(torch.zeros((3, 4, 16), dtype=torch.uint8), 4)
    with pytest.raises(ValueError, match="3 planes, the layout 2"):
        kvx.gather(lay, three, tab, reqs, st)
    with pytest.raises(ValueError, match="3 planes, the layout 2"):
        kvx.gather_scatter(lay, three, tab, reqs, three, tab)
    one = kvx.Pool([torch.zeros(64, dtype=torch.uint8)], 4, slot_stride=16)
    with pytest.raises(ValueError, match="1 planes, the layout 2"):
        kvx.scatter(lay, st, reqs, one, tab)
    # a pool that claims more pages than its tensor holds
    big = kvx.Pool(torch.zeros((2, 4, 16), dtype=torch.uint8), 5, slot_stride=16)
    with pytest.raises(ValueError, match="the pool's pages need 80"):
        kvx.gather(lay, big, tab, reqs, st)
    planes = [torch.zeros(64, dtype=torch.uint8), torch.zeros(48, dtype=torch.uint8)]
    with pytest.raises(ValueError, match="holds 48 bytes"):
        kvx.gather(lay, kvx.Pool(planes, 4, slot_stride=16), tab, reqs, st)
    # token-major planes (stride Q * R, bases R apart) fit in their storage
    tm = torch.zeros((4, 2, 16), dtype=torch.uint8)
    kvx._check_pool("tm", lay, kvx.Pool(tm.transpose(0, 1), 4, slot_stride=32))
    with pytest.raises(ValueError, match="the pool's pages need"):
        kvx._check_pool("tm", lay, kvx.Pool(tm.transpose(0, 1), 5, slot_stride=32))
    # head-sliced copies address whole pages: 4 pages x 2 rows x 32 bytes per plane
    hp = kvx.Pool(torch.zeros((2, 255), dtype=torch.uint8), 4, page_size=2, slot_stride=32)
    with pytest.raises(ValueError, match="need 256"):
        kvx.gather_scatter_heads(lay, hp, tab, kvx.Heads(2, 0), reqs, hp, tab, kvx.Heads(2, 0))
    # page offsets for every request plus one
    with pytest.raises(ValueError, match="pg_off needs num_reqs \\+ 1 = 2"):
        kvx.gather(lay, kvx.Pool(torch.zeros((2, 4, 16), dtype=torch.uint8), 4),
                   kvx.Table(torch.zeros(1, dtype=torch.int64), torch.zeros(2, dtype=torch.int32)),
                   reqs, st)
    # HF planes: one per plane, each [1, H, s_cap, D]
    with pytest.raises(ValueError, match="hf_planes has 3 planes"):
        kvx.extract_permute(lay, torch.zeros((3, 32), dtype=torch.uint8), 2, 1, st)
    with pytest.raises(ValueError, match="hf_planes has 1 planes"):
        kvx.rebuild_permute(lay, st, 1, [torch.zeros(32, dtype=torch.uint8)], 2)
    with pytest.raises(ValueError, match="needs 48"):
        kvx.extract_permute(lay, torch.zeros((2, 32), dtype=torch.uint8), 3, 1, st)


def test_binding_extent_check_follows_plane_addresses():
    """Planes given as raw addresses inside kept tensors (blocks holding K and
    V of a layer: plane q inside layer tensor q // 2) are checked against the
    tensor that holds them, whatever the order of the kept list."""
    import torch
    lay = kvx.Layout(2, 2, 1, 8, "bf16")                      # Q = 4, R = 16
    B, P = 2, 3
    layers = [torch.zeros(P * 2 * B * 16, dtype=torch.uint8) for _ in range(2)]
    ptrs = [layers[q // 2].data_ptr() + (q % 2) * B * 16 for q in range(4)]
    pool = kvx.Pool(ptrs, P, B, slot_stride=16, page_stride=2 * B * 16, keep=layers)
    kvx._check_pool("blocks", lay, pool)                     # V's last row ends at the tensor end
    pool = kvx.Pool(ptrs, P + 1, B, slot_stride=16, page_stride=2 * B * 16, keep=layers[::-1])
    with pytest.raises(ValueError, match="the pool's pages need"):
        kvx._check_pool("blocks", lay, pool)


def test_binding_plane_pointers_and_cached_extent(monkeypatch):
    """Plane base pointers of a strided tensor are planes[q]'s addresses; a
    pool's extent is measured once, when it is made, so the check of each
    call does not walk its planes again (it is on every call's host path)."""
    import torch
    t = torch.zeros((5, 3, 32), dtype=torch.uint8)[:, 1:]
    arr = kvx._plane_array(t)
    assert [arr[q] for q in range(5)] == [t[q].data_ptr() for q in range(5)]
    lay = kvx.Layout(1, 2, 1, 8, "bf16")                          # Q = 2, R = 16
    A = torch.zeros((2, 8, 16), dtype=torch.uint8)
    pool = kvx.Pool(A, 8)
    assert pool._min_bytes == 8 * 16                              # the last plane's extent
    tensors = [torch.zeros(8 * 16, dtype=torch.uint8), torch.zeros(7 * 16, dtype=torch.uint8)]
    short = kvx.Pool(tensors, 8, slot_stride=16)
    assert short._min_bytes == 7 * 16

    def walk(*a):
        raise AssertionError("plane walk on the per-call path")
    monkeypatch.setattr(kvx, "_plane_tensors", walk)
    monkeypatch.setattr(kvx, "_min_plane_bytes", walk)
    kvx._check_pool("src", lay, pool)
    with pytest.raises(ValueError, match="the pool's pages need"):
        kvx._check_pool("src", lay, short)
