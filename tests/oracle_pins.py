"""Pins for the CPU oracle: each check ties it to something other than itself.

Every ``check_*`` function raises AssertionError on a mismatch.  They are run
by ``test_oracle_pins.py`` against the real oracle build, and by
``test_oracle_mutants.py`` against builds with a planted mistake (each mutant
must fail at least one check).

Independent references used here:
* element-by-element Python loops over [Q][slots][H][D] arrays;
* ``numpy.take`` (page size 1: gather is a row take per plane);
* page tables expanded into explicit slot lists built from whole pages;
* the permute the mini-infer PD page describes (section "KV 序列化格式选择"):
  batch 0 and the first seq positions, head and sequence axes swapped, and
  its inverse with a leading unit axis -- evaluated with torch's axis moves
  on the CPU;
* round trips, untouched-byte invariants and the page-printed byte counts.
"""
from __future__ import annotations

import itertools
import os

import numpy as np

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "kv_sizes.txt")


# --------------------------------------------------------------- helpers --

def rand_pool(rng, Q, S, H, D):
    """[Q][S][H][D] of random 16-bit words (every bit pattern, NaNs included)."""
    return rng.integers(0, 1 << 16, size=(Q, S, H, D), dtype=np.uint16)


def planes_of(pool):
    return [pool[q].reshape(-1).view(np.uint8) for q in range(pool.shape[0])]


def slot_of(side, r, t):
    """Slot of token t of request r, written out from the definition: entry
    pg_off[r] + t // B of the page-id list (-1 when that index is outside the
    list), page id out of [0, num_pages) -> -1, else page * B + t % B."""
    idx = int(side.pg_off[r]) + t // side.page_size
    if idx < 0 or idx >= side.ids.size:
        return -1
    page = int(side.ids[idx])
    if page < 0 or page >= side.num_pages:
        return -1
    return page * side.page_size + t % side.page_size


def slot_lists(case, side):
    """Per-request slot lists, token by token (-1 marks a skipped token)."""
    out = []
    for r in range(case.num_reqs):
        n = int(case.tok_off[r + 1] - case.tok_off[r])
        out.append(np.array([slot_of(side, r, t) for t in range(n)], dtype=np.int64))
    return out


def bf_gather(pool, case, side):
    """Staging built element by element: per request, a [Q, n, H, D] block."""
    Q, S, H, D = pool.shape
    blocks, skipped = [], 0
    for r, slots in enumerate(slot_lists(case, side)):
        blk = np.zeros((Q, len(slots), H, D), np.uint16)
        for q in range(Q):
            for t, s in enumerate(slots):
                if s < 0:
                    skipped += 1
                    continue
                for h in range(H):
                    for d in range(D):
                        blk[q, t, h, d] = pool[q, s, h, d]
        blocks.append(blk.reshape(-1))
    flat = np.concatenate(blocks) if blocks else np.zeros(0, np.uint16)
    return flat, skipped


def bf_scatter(stage_blocks, case, side, pool):
    """Write per-request [Q, n, H, D] blocks into a copy of pool, element-wise."""
    out = pool.copy()
    Q, S, H, D = pool.shape
    skipped = 0
    for r, slots in enumerate(slot_lists(case, side)):
        blk = stage_blocks[r]
        for q in range(Q):
            for t, s in enumerate(slots):
                if s < 0:
                    skipped += 1
                    continue
                for h in range(H):
                    for d in range(D):
                        out[q, s, h, d] = blk[q, t, h, d]
    return out, skipped


def split_blocks(flat, case, Q, H, D):
    blocks = []
    for r in range(case.num_reqs):
        a, b = int(case.tok_off[r]), int(case.tok_off[r + 1])
        blocks.append(flat[a * Q * H * D:b * Q * H * D].reshape(Q, b - a, H, D))
    return blocks


def o_gather(pool, case, side, staging, nthreads=1):
    Q, S, H, D = pool.shape
    return oracle.gather(planes_of(pool), H * D * 2, side.page_size, side.num_pages, H * D * 2,
                         case.tok_off, side.pg_off, side.ids, staging.view(np.uint8), nthreads)


def o_scatter(staging, case, side, pool, nthreads=1):
    Q, S, H, D = pool.shape
    return oracle.scatter(staging.view(np.uint8), H * D * 2, case.tok_off, side.pg_off, side.ids,
                          planes_of(pool), H * D * 2, side.page_size, side.num_pages, nthreads)


def o_gather_scatter(src_pool, case, dst_pool, nthreads=1):
    Q, S, H, D = src_pool.shape
    R = H * D * 2
    return oracle.gather_scatter(planes_of(src_pool), R, case.src.page_size, case.src.num_pages,
                                 case.src.pg_off, case.src.ids, R, case.tok_off,
                                 planes_of(dst_pool), R, case.dst.page_size, case.dst.num_pages,
                                 case.dst.pg_off, case.dst.ids, nthreads)


def tiny_cases(oor=0.0, index_faults=False):
    geoms = [wl.Geometry(1, 2, 1, 8), wl.Geometry(2, 1, 3, 8), wl.Geometry(1, 2, 2, 16)]
    cases = []
    for i, g in enumerate(geoms):
        for bs, bd in [(1, 1), (2, 4), (4, 2), (3, 1)]:
            cases.append(wl.random_case(100 * i + 10 * bs + bd + (7 if index_faults else 0),
                                        geom=g, max_reqs=4 if index_faults else 3, max_len=9,
                                        src_page=bs, dst_page=bd, oor_frac=oor, slack_pages=2,
                                        index_faults=index_faults))
    return cases


# (out-of-range page-id fraction, page-table index faults) of the brute-force sweeps
FAULTS = [(0.0, False), (0.2, False), (0.0, True), (0.2, True)]


def pools_for(case, rng):
    g = case.geom
    src = rand_pool(rng, g.planes, case.src.num_slots, g.kv_heads, g.head_dim)
    dst = rand_pool(rng, g.planes, case.dst.num_slots, g.kv_heads, g.head_dim)
    return src, dst


# ----------------------------------------------------------------- checks --

def check_gather_bruteforce():
    rng = np.random.default_rng(7)
    for oor, faults in FAULTS:
        for case in tiny_cases(oor, faults):
            src, _ = pools_for(case, rng)
            g = case.geom
            expect, bf_skip = bf_gather(src, case, case.src)
            got = np.full(expect.size, 0xABCD, np.uint16)
            # rows the brute force skipped keep the prefill in both
            expect = np.where(_skipped_mask(case, case.src, g), 0xABCD, expect)
            skipped = o_gather(src, case, case.src, got)
            assert skipped == bf_skip, (case.name, skipped, bf_skip)
            assert np.array_equal(got, expect), case.name


def _skipped_mask(case, side, g):
    """Element mask over staging of rows whose page id is out of range."""
    Q, H, D = g.planes, g.kv_heads, g.head_dim
    parts = []
    for slots in slot_lists(case, side):
        m = np.broadcast_to((slots < 0)[None, :, None, None], (Q, len(slots), H, D))
        parts.append(m.reshape(-1))
    return np.concatenate(parts) if parts else np.zeros(0, bool)


def check_scatter_bruteforce():
    rng = np.random.default_rng(8)
    for oor, faults in FAULTS:
        for case in tiny_cases(oor, faults):
            g = case.geom
            _, dst = pools_for(case, rng)
            stage = rng.integers(0, 1 << 16, size=case.total_tokens * g.planes * g.kv_heads
                                 * g.head_dim, dtype=np.uint16)
            expect, bf_skip = bf_scatter(split_blocks(stage, case, g.planes, g.kv_heads,
                                                      g.head_dim), case, case.dst, dst)
            got = dst.copy()
            skipped = o_scatter(stage, case, case.dst, got)
            assert skipped == bf_skip, case.name
            assert np.array_equal(got, expect), case.name


def check_gather_scatter_bruteforce():
    rng = np.random.default_rng(9)
    for oor, faults in FAULTS:
        for case in tiny_cases(oor, faults):
            g = case.geom
            src, dst = pools_for(case, rng)
            got = dst.copy()
            skipped = o_gather_scatter(src, case, got)
            expect = dst.copy()
            bf_skip = 0
            for r, (ss, ds) in enumerate(zip(slot_lists(case, case.src),
                                             slot_lists(case, case.dst))):
                for q in range(g.planes):
                    for t in range(len(ss)):
                        if ss[t] < 0 or ds[t] < 0:
                            bf_skip += 1
                            continue
                        for h in range(g.kv_heads):
                            for d in range(g.head_dim):
                                expect[q, ds[t], h, d] = src[q, ss[t], h, d]
            assert skipped == bf_skip, case.name
            assert np.array_equal(got, expect), case.name


def check_exhaustive_injective():
    """Every injective table of n <= 5 tokens into a 5-slot pool (326 tables)."""
    rng = np.random.default_rng(10)
    S, Q, H, D = 5, 2, 1, 8
    src = rand_pool(rng, Q, S, H, D)
    dst0 = rand_pool(rng, Q, S, H, D)
    for n in range(0, S + 1):
        for perm in itertools.permutations(range(S), n):
            slots = np.array(perm, np.int64)
            case = wl.PagedCase("inj", wl.Geometry(1, 2, H, D), wl.csr_from_lengths([n]),
                                wl.side_from_slot_lists([slots], S),
                                wl.side_from_slot_lists([slots[::-1].copy()], S), 0, 0, 0)
            st = np.zeros(Q * n * H * D, np.uint16)
            assert o_gather(src, case, case.src, st) == 0
            assert np.array_equal(st.reshape(Q, n, H, D), src[:, slots]), perm
            got = dst0.copy()
            o_scatter(st, case, case.dst, got)
            exp = dst0.copy()
            for t, s in enumerate(slots[::-1]):
                exp[:, s] = src[:, slots[t]]
            assert np.array_equal(got, exp), perm
            got2 = dst0.copy()
            o_gather_scatter(src, case, got2)
            assert np.array_equal(got2, exp), perm


def check_take_special_case():
    """Page size 1: gather of plane q is numpy.take(plane, slots) per request;
    the identity table is the plain slice copy pool[:, :n]."""
    rng = np.random.default_rng(11)
    Q, S, H, D = 3, 40, 2, 8
    pool = rand_pool(rng, Q, S, H, D)
    lens = [7, 0, 13, 5]
    lists = [rng.integers(0, S, size=n) for n in lens]          # repeats allowed
    case = wl.PagedCase("take", wl.Geometry(1, 3, H, D), wl.csr_from_lengths(lens),
                        wl.side_from_slot_lists(lists, S), None, 0, 0, 0)
    st = np.zeros(sum(lens) * Q * H * D, np.uint16)
    o_gather(pool, case, case.src, st)
    pos = 0
    for sl in lists:
        blk = np.stack([np.take(pool[q], sl, axis=0) for q in range(Q)])
        assert np.array_equal(st[pos:pos + blk.size].reshape(blk.shape), blk)
        pos += blk.size
    ident = wl.PagedCase("ident", wl.Geometry(1, 3, H, D), wl.csr_from_lengths([S]),
                         wl.side_from_slot_lists([np.arange(S)], S), None, 0, 0, 0)
    st2 = np.zeros(S * Q * H * D, np.uint16)
    o_gather(pool, ident, ident.src, st2)
    assert np.array_equal(st2.reshape(pool.shape), pool)


def check_page_expansion():
    """A page-B table gives the same bytes as the page-1 table of its slots."""
    rng = np.random.default_rng(12)
    for B in (2, 3, 16):
        case = wl.random_case(300 + B, geom=wl.Geometry(2, 2, 1, 8), max_reqs=4, max_len=40,
                              src_page=B, dst_page=B)
        g = case.geom
        src, dst = pools_for(case, rng)
        exp_src = wl.side_from_slot_lists(slot_lists(case, case.src), case.src.num_slots)
        exp_dst = wl.side_from_slot_lists(slot_lists(case, case.dst), case.dst.num_slots)
        n = case.total_tokens * g.planes * g.kv_heads * g.head_dim
        a, b = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
        o_gather(src, case, case.src, a)
        o_gather(src, case, exp_src, b)
        assert np.array_equal(a, b), B
        c, d = dst.copy(), dst.copy()
        o_scatter(a, case, case.dst, c)
        o_scatter(a, case, exp_dst, d)
        assert np.array_equal(c, d), B


def check_batch_is_concatenation():
    """A batch of requests equals the single-request calls laid end to end."""
    rng = np.random.default_rng(13)
    case = wl.random_case(14, geom=wl.Geometry(2, 2, 2, 8), max_reqs=5, max_len=30, src_page=4,
                          dst_page=2)
    g = case.geom
    src, dst = pools_for(case, rng)
    whole = np.zeros(case.total_tokens * g.planes * g.kv_heads * g.head_dim, np.uint16)
    o_gather(src, case, case.src, whole)
    parts = []
    for r in range(case.num_reqs):
        n = int(case.lengths[r])
        pages = case.src.ids[case.src.pg_off[r]:case.src.pg_off[r + 1]]
        one = wl.PagedCase("one", g, wl.csr_from_lengths([n]),
                           wl.side_from_page_lists([pages], case.src.num_pages,
                                                   case.src.page_size), None, 0, 0, 0)
        st = np.zeros(n * g.planes * g.kv_heads * g.head_dim, np.uint16)
        o_gather(src, one, one.src, st)
        parts.append(st)
    assert np.array_equal(whole, np.concatenate(parts))


def check_roundtrips():
    """gather(scatter(x)) == x for distinct destination rows, and
    scatter(gather(pool)) == gather_scatter(pool) over the whole destination."""
    rng = np.random.default_rng(15)
    for seed in range(6):
        case = wl.random_case(400 + seed, max_reqs=4, max_len=25)
        g = case.geom
        src, dst = pools_for(case, rng)
        n = case.total_tokens * g.planes * g.kv_heads * g.head_dim
        x = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
        pool = dst.copy()
        o_scatter(x, case, case.dst, pool)
        back = np.zeros(n, np.uint16)
        o_gather(pool, case, case.dst, back)
        assert np.array_equal(back, x), case.name
        st = np.zeros(n, np.uint16)
        o_gather(src, case, case.src, st)
        via_staging = dst.copy()
        o_scatter(st, case, case.dst, via_staging)
        direct = dst.copy()
        o_gather_scatter(src, case, direct)
        assert np.array_equal(via_staging, direct), case.name


def check_untouched_and_extent():
    """Gather writes exactly [0, total*Q*R) of staging (two prefills differ
    nowhere inside, agree everywhere outside); scatter and gather-scatter leave
    every slot outside the table as it was."""
    rng = np.random.default_rng(16)
    for seed in range(5):
        case = wl.random_case(500 + seed, max_reqs=4, max_len=30)
        g = case.geom
        src, dst = pools_for(case, rng)
        n = case.total_tokens * g.planes * g.kv_heads * g.head_dim
        guard = 64
        a = np.zeros(n + guard, np.uint16)
        b = np.full(n + guard, 0xFFFF, np.uint16)
        o_gather(src, case, case.src, a)
        o_gather(src, case, case.src, b)
        assert np.array_equal(a[:n], b[:n]), case.name
        assert (a[n:] == 0).all() and (b[n:] == 0xFFFF).all(), case.name
        touched = np.zeros(case.dst.num_slots, bool)
        for sl in slot_lists(case, case.dst):
            touched[sl[sl >= 0]] = True
        out = dst.copy()
        o_gather_scatter(src, case, out)
        assert np.array_equal(out[:, ~touched], dst[:, ~touched]), case.name
        out2 = dst.copy()
        o_scatter(a[:n], case, case.dst, out2)
        assert np.array_equal(out2[:, ~touched], dst[:, ~touched]), case.name


def check_token_major_pool():
    """A token-major pool (plane q of slot s at (s*Q + q)*R, stride Q*R) gives
    the same bytes as the layer-major pool holding the same rows."""
    rng = np.random.default_rng(17)
    case = wl.random_case(600, geom=wl.Geometry(2, 2, 2, 8), max_reqs=3, max_len=20,
                          src_page=2, dst_page=3)
    g = case.geom
    Q, R = g.planes, g.row_bytes
    src, dst = pools_for(case, rng)
    tm_src = np.ascontiguousarray(src.transpose(1, 0, 2, 3)).reshape(-1).view(np.uint8)
    tm_dst = np.ascontiguousarray(dst.transpose(1, 0, 2, 3)).reshape(-1).view(np.uint8)
    src_planes = [tm_src[q * R:] for q in range(Q)]
    dst_planes = [tm_dst[q * R:] for q in range(Q)]
    n = case.total_tokens * Q * R
    a = np.zeros(n, np.uint8)
    oracle.gather(src_planes, Q * R, case.src.page_size, case.src.num_pages, R, case.tok_off,
                  case.src.pg_off, case.src.ids, a)
    b = np.zeros(n // 2, np.uint16)
    o_gather(src, case, case.src, b)
    assert np.array_equal(a, b.view(np.uint8))
    oracle.gather_scatter(src_planes, Q * R, case.src.page_size, case.src.num_pages,
                          case.src.pg_off, case.src.ids, R, case.tok_off, dst_planes, Q * R,
                          case.dst.page_size, case.dst.num_pages, case.dst.pg_off, case.dst.ids)
    ref = dst.copy()
    o_gather_scatter(src, case, ref)
    back = tm_dst.view(np.uint16).reshape(dst.shape[1], Q, g.kv_heads, g.head_dim)
    assert np.array_equal(back.transpose(1, 0, 2, 3), ref)


def check_mixed_strides():
    """Source and destination pools with different slot strides."""
    rng = np.random.default_rng(18)
    case = wl.random_case(700, geom=wl.Geometry(1, 2, 1, 8), max_reqs=3, max_len=20)
    g = case.geom
    Q, R = g.planes, g.row_bytes
    src, dst = pools_for(case, rng)
    pad = 3 * R                                 # destination slots padded to 4R
    dstp = np.zeros((Q, case.dst.num_slots, 4 * R), np.uint8)
    dstp[:, :, :R] = dst.reshape(Q, case.dst.num_slots, R // 2).view(np.uint8)
    planes = [dstp[q].reshape(-1) for q in range(Q)]
    oracle.gather_scatter(planes_of(src), R, case.src.page_size, case.src.num_pages,
                          case.src.pg_off, case.src.ids, R, case.tok_off, planes, R + pad,
                          case.dst.page_size, case.dst.num_pages, case.dst.pg_off, case.dst.ids)
    ref = dst.copy()
    o_gather_scatter(src, case, ref)
    got = dstp[:, :, :R].copy().view(np.uint16).reshape(ref.shape)
    assert np.array_equal(got, ref)
    assert (dstp[:, :, R:] == 0).all()


def _page_of(side, r, t):
    """Page id of token t of request r, or None when its page-table index or
    the id there is out of range."""
    idx = int(side.pg_off[r]) + t // side.page_size
    if idx < 0 or idx >= side.ids.size:
        return None
    page = int(side.ids[idx])
    return page if 0 <= page < side.num_pages else None


def check_block_interleaved_pools():
    """Pools whose blocks hold K and V of a layer together ([blocks][2][B][H][D]
    per layer) or every plane ([blocks][L][2][B][H][D]), addressed through a
    page stride = the block length: gather, scatter and gather-scatter
    against element-by-element reads and writes of those arrays, out-of-range
    ids included."""
    rng = np.random.default_rng(31)
    for seed, (bs, bd) in enumerate([(4, 2), (2, 4), (1, 3), (3, 1)]):
        case = wl.random_case(900 + seed, geom=wl.Geometry(2, 2, 2, 8), max_reqs=4, max_len=14,
                              src_page=bs, dst_page=bd, oor_frac=0.1, slack_pages=3)
        g = case.geom
        L, H, D, Q = g.num_layers, g.kv_heads, g.head_dim, g.planes
        R = H * D * 2
        nbs, nbd = case.src.num_pages, case.dst.num_pages
        # source: one [blocks][2][B][H][D] tensor per layer
        src = [rng.integers(0, 1 << 16, (nbs, 2, bs, H, D), dtype=np.uint16) for _ in range(L)]
        src_b = [a.reshape(-1).view(np.uint8) for a in src]
        src_planes = [src_b[q // 2][(q % 2) * bs * R:] for q in range(Q)]
        # destination: one [blocks][L][2][B][H][D] tensor
        dst = rng.integers(0, 1 << 16, (nbd, L, 2, bd, H, D), dtype=np.uint16)
        dst_planes_of = lambda a: [a.reshape(-1).view(np.uint8)[q * bd * R:]  # noqa: E731
                                   for q in range(Q)]
        n = case.total_tokens * Q * R
        # expected staging and destination, element by element
        exp_st = np.zeros((n // 2,), np.uint16)
        exp_gs = dst.copy()
        for r in range(case.num_reqs):
            o, e = int(case.tok_off[r]), int(case.tok_off[r + 1])
            for t in range(e - o):
                ps, pd = _page_of(case.src, r, t), _page_of(case.dst, r, t)
                for q in range(Q):
                    l, kv = divmod(q, 2)
                    base = ((o * Q + q * (e - o) + t) * R) // 2
                    if ps is not None:
                        exp_st[base:base + H * D] = src[l][ps, kv, t % bs].reshape(-1)
                    if ps is not None and pd is not None:
                        exp_gs[pd, l, kv, t % bd] = src[l][ps, kv, t % bs]
        st = np.zeros(n, np.uint8)
        oracle.gather(src_planes, R, bs, nbs, R, case.tok_off, case.src.pg_off, case.src.ids, st,
                      page_stride=2 * bs * R)
        assert np.array_equal(st.view(np.uint16), exp_st)
        got = dst.copy()
        oracle.gather_scatter(src_planes, R, bs, nbs, case.src.pg_off, case.src.ids, R,
                              case.tok_off, dst_planes_of(got), R, bd, nbd, case.dst.pg_off,
                              case.dst.ids, src_page_stride=2 * bs * R,
                              dst_page_stride=L * 2 * bd * R)
        assert np.array_equal(got, exp_gs)
        # scatter of a random staging buffer into the [blocks][L][2][B][H][D] pool
        stage_in = rng.integers(0, 256, n, dtype=np.uint8)
        exp_sc = dst.copy()
        s16 = stage_in.view(np.uint16)
        for r in range(case.num_reqs):
            o, e = int(case.tok_off[r]), int(case.tok_off[r + 1])
            for t in range(e - o):
                pd = _page_of(case.dst, r, t)
                if pd is None:
                    continue
                for q in range(Q):
                    l, kv = divmod(q, 2)
                    base = ((o * Q + q * (e - o) + t) * R) // 2
                    exp_sc[pd, l, kv, t % bd] = s16[base:base + H * D].reshape(H, D)
        got = dst.copy()
        oracle.scatter(stage_in, R, case.tok_off, case.dst.pg_off, case.dst.ids,
                       dst_planes_of(got), R, bd, nbd, page_stride=L * 2 * bd * R)
        assert np.array_equal(got, exp_sc)


def check_threads_agree():
    rng = np.random.default_rng(19)
    case = wl.random_case(800, max_reqs=6, max_len=40, oor_frac=0.1)
    g = case.geom
    src, dst = pools_for(case, rng)
    n = case.total_tokens * g.planes * g.kv_heads * g.head_dim
    a, b = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    sa = o_gather(src, case, case.src, a, nthreads=1)
    sb = o_gather(src, case, case.src, b, nthreads=5)
    assert sa == sb and np.array_equal(a, b)
    c, d = dst.copy(), dst.copy()
    assert o_gather_scatter(src, case, c, 1) == o_gather_scatter(src, case, d, 7)
    assert np.array_equal(c, d)


def check_oor_boundaries():
    """Ids 0 and num_pages-1 are copied; -1, num_pages, INT32_MIN and INT32_MAX
    are skipped, counted, and leave their destination rows untouched."""
    rng = np.random.default_rng(23)
    Q, H, D, B, P = 2, 1, 8, 2, 4
    # one spare page of real memory past the pool, so a wrong bound reads or
    # writes valid bytes (and is then caught here) instead of faulting
    pool = rand_pool(rng, Q, (P + 1) * B, H, D)
    ids = np.array([0, P - 1, -1, P, np.iinfo(np.int32).min, np.iinfo(np.int32).max], np.int32)
    n = len(ids) * B
    side = wl.Side(P, B, np.array([0, len(ids)], np.int64), ids)
    case = wl.PagedCase("oor", wl.Geometry(1, 2, H, D), wl.csr_from_lengths([n]), side, side,
                        0, 0, 0)
    st = np.full(Q * n * H * D, 0x5A5A, np.uint16)
    assert o_gather(pool, case, case.src, st) == Q * 4 * B
    blk = st.reshape(Q, n, H, D)
    assert np.array_equal(blk[:, 0:B], pool[:, 0:B])
    assert np.array_equal(blk[:, B:2 * B], pool[:, (P - 1) * B:P * B])
    assert (blk[:, 2 * B:] == 0x5A5A).all()
    out = pool.copy()
    assert o_scatter(st, case, case.dst, out) == Q * 4 * B
    assert np.array_equal(out[:, P * B:], pool[:, P * B:])
    out2 = pool.copy()
    assert o_gather_scatter(pool, case, out2) == Q * 4 * B
    assert np.array_equal(out2[:, P * B:], pool[:, P * B:])


def check_empty_page_table():
    """A side whose page-id list is empty: every table index is outside
    [0, 0), so every row of a gather, scatter or gather-scatter is skipped and
    counted and every destination byte keeps its value, whatever pg_off says;
    with the other side empty instead, the copy still moves nothing."""
    rng = np.random.default_rng(31)
    Q, H, D, B, P = 2, 1, 8, 4, 4
    lens = [5, 0, 7]
    tok_off = wl.csr_from_lengths(lens)
    n = sum(lens)
    pg = np.array([0, 2, 2, 4], np.int64)
    full = wl.Side(P, B, pg, np.array([2, 0, 3, 1], np.int32))
    empty = wl.Side(P, B, pg, np.zeros(0, np.int32))
    pool = rand_pool(rng, Q, P * B, H, D)
    dst = rand_pool(rng, Q, P * B, H, D)
    case = wl.PagedCase("empty", wl.Geometry(1, 2, H, D), tok_off, empty, full, 0, 0, 0)
    st = np.full((n * Q, H, D), 0x5A5A, np.uint16)
    assert o_gather(pool, case, case.src, st.reshape(-1)) == Q * n
    assert (st == 0x5A5A).all()
    stage = rng.integers(0, 1 << 16, size=(n * Q, H, D), dtype=np.uint16)
    got = dst.copy()
    assert o_scatter(stage.reshape(-1), case, empty, got) == Q * n
    assert np.array_equal(got, dst)
    for src_side, dst_side in ((empty, full), (full, empty)):
        c = wl.PagedCase("empty_gs", wl.Geometry(1, 2, H, D), tok_off, src_side, dst_side, 0, 0, 0)
        got = dst.copy()
        assert o_gather_scatter(pool, c, got) == Q * n
        assert np.array_equal(got, dst)
    # the full side alone moves every row (the same tables, brute force)
    c = wl.PagedCase("full_gs", wl.Geometry(1, 2, H, D), tok_off, full, full, 0, 0, 0)
    got = dst.copy()
    assert o_gather_scatter(pool, c, got) == 0
    exp = dst.copy()
    for r in range(len(lens)):
        for t in range(lens[r]):
            exp[:, slot_of(full, r, t)] = pool[:, slot_of(full, r, t)]
    assert np.array_equal(got, exp)


def check_table_index_boundaries():
    """A worked example of the page-table reads (pages of B = 2 tokens, seven
    requests, three page ids held between two guard entries that name real
    pages): request 0's list starts one entry before the array (its first
    page is skipped), request 1's second page lies one past the end
    (skipped), request 2 has an empty list and reads on into the entries
    after its start, requests 3 and 4 start 2**62 entries before and after
    the array (skipped), and requests 5 and 6 start at the ends of the int64
    range, where the index pg_off[r] + t / B runs past 2**63 - 1 (request 5's
    source, request 6's destination: three pages of tokens) or starts at
    -2**63 (skipped: the index is a plain integer, it does not wrap).
    Expected rows are written out by hand; every skipped row is counted and
    leaves its destination untouched, and the guards are never read."""
    rng = np.random.default_rng(27)
    Q, H, D, B, P = 2, 1, 8, 2, 4
    big = 1 << 62
    i64max, i64min = (1 << 63) - 1, -(1 << 63)
    lens = [4, 4, 2, 2, 2, 6, 6]
    tok_off = wl.csr_from_lengths(lens)
    guard = 2                                   # a real page: reading a guard copies rows
    s_buf = np.array([guard, 1, 3, 0, guard], np.int32)
    d_buf = np.array([guard, 1, 3, 0, guard], np.int32)
    src_side = wl.Side(P, B, np.array([-1, 2, 0, -big, big, i64max - 1, i64min, 3], np.int64),
                       s_buf[1:4])
    dst_side = wl.Side(P, B, np.array([-1, 2, 1, -big, big, i64min + 1, i64max, 3], np.int64),
                       d_buf[1:4])
    assert src_side.ids.base is s_buf          # a view: the guards sit around it in memory
    case = wl.PagedCase("idx", wl.Geometry(1, 2, H, D), tok_off, src_side, dst_side, 0, 0, 0)
    # (request, token) -> slot, by hand
    src_slots = {(0, 2): 2, (0, 3): 3, (1, 0): 0, (1, 1): 1, (2, 0): 2, (2, 1): 3}
    dst_slots = {(0, 2): 2, (0, 3): 3, (1, 0): 0, (1, 1): 1, (2, 0): 6, (2, 1): 7}
    tokens = [(r, t) for r, n in enumerate(lens) for t in range(n)]
    pool = rand_pool(rng, Q, P * B, H, D)
    # gather
    n = sum(lens)
    st = np.full((n * Q, H, D), 0x7E7E, np.uint16)
    assert o_gather(pool, case, case.src, st.reshape(-1)) == Q * (n - len(src_slots))
    exp = np.full_like(st, 0x7E7E)
    for (r, t) in tokens:
        if (r, t) in src_slots:
            for q in range(Q):
                exp[tok_off[r] * Q + q * lens[r] + t] = pool[q, src_slots[(r, t)]]
    assert np.array_equal(st, exp)
    # scatter
    stage = rng.integers(0, 1 << 16, size=(n * Q, H, D), dtype=np.uint16)
    dst = rand_pool(rng, Q, P * B, H, D)
    got = dst.copy()
    assert o_scatter(stage.reshape(-1), case, case.dst, got) == Q * (n - len(dst_slots))
    exp = dst.copy()
    for (r, t), slot in dst_slots.items():
        for q in range(Q):
            exp[q, slot] = stage[tok_off[r] * Q + q * lens[r] + t]
    assert np.array_equal(got, exp)
    # gather-scatter, and the head-sliced copy of the whole row
    both = [k for k in tokens if k in src_slots and k in dst_slots]
    exp = dst.copy()
    for (r, t) in both:
        exp[:, dst_slots[(r, t)]] = pool[:, src_slots[(r, t)]]
    got = dst.copy()
    assert o_gather_scatter(pool, case, got) == Q * (n - len(both))
    assert np.array_equal(got, exp)
    got = dst.copy()
    assert o_heads(case, pool.reshape(Q, -1).view(np.uint8), got.reshape(Q, -1).view(np.uint8),
                   H, 0, 0, H, 0, 0, H, D) == Q * (n - len(both))
    assert np.array_equal(got, exp)


# -------------------------------------------------- head-sliced copies --

def head_view(pool_bytes, Q, P, B, H, D, hnd):
    """uint16 view [Q, pages, B, H, D] (NHD) or [Q, pages, H, B, D] (HND)."""
    w = pool_bytes.view(np.uint16)
    return w.reshape(Q, P, H, B, D) if hnd else w.reshape(Q, P, B, H, D)


def o_heads(case, src_b, dst_b, sH, sh0, shnd, dH, dh0, dhnd, nh, D, nthreads=1):
    Q = case.geom.planes
    Db = D * 2
    return oracle.gather_scatter_heads(
        [src_b[q] for q in range(Q)], sH * Db, case.src.page_size, case.src.num_pages,
        case.src.pg_off, case.src.ids, (sH, sh0, shnd), Db, nh, case.tok_off,
        [dst_b[q] for q in range(Q)], dH * Db, case.dst.page_size, case.dst.num_pages,
        case.dst.pg_off, case.dst.ids, (dH, dh0, dhnd), nthreads)


def heads_case(seed, oor=0.0, index_faults=False):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([8, 16]))
    sH, dH = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    nh = int(rng.integers(1, min(sH, dH) + 1))
    sh0, dh0 = int(rng.integers(0, sH - nh + 1)), int(rng.integers(0, dH - nh + 1))
    shnd, dhnd = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    case = wl.random_case(seed, geom=wl.Geometry(int(rng.integers(1, 3)), 2, nh, D), max_reqs=3,
                          max_len=12, src_page=int(rng.choice([1, 2, 4])),
                          dst_page=int(rng.choice([1, 3, 4])), oor_frac=oor, slack_pages=2,
                          index_faults=index_faults)
    return case, D, (sH, sh0, shnd), (dH, dh0, dhnd), nh


def check_heads_bruteforce():
    """Element by element over NHD / HND views of both pools."""
    for seed in range(32):
        case, D, (sH, sh0, shnd), (dH, dh0, dhnd), nh = heads_case(
            900 + seed, oor=0.2 if seed % 3 else 0, index_faults=seed >= 16)
        rng = np.random.default_rng(seed)
        Q = case.geom.planes
        Ps, Pd, Bs, Bd = case.src.num_pages, case.dst.num_pages, case.src.page_size, \
            case.dst.page_size
        src_b = rng.integers(0, 256, (Q, Ps * Bs * sH * D * 2), dtype=np.uint8)
        dst_b = rng.integers(0, 256, (Q, Pd * Bd * dH * D * 2), dtype=np.uint8)
        got = dst_b.copy()
        skipped = o_heads(case, src_b, got, sH, sh0, shnd, dH, dh0, dhnd, nh, D)
        sv = head_view(src_b, Q, Ps, Bs, sH, D, shnd)
        exp = dst_b.copy()
        dv = head_view(exp, Q, Pd, Bd, dH, D, dhnd)
        bf_skip = 0
        for r in range(case.num_reqs):
            for t in range(int(case.lengths[r])):
                ps, pd = _page_of(case.src, r, t), _page_of(case.dst, r, t)
                for q in range(Q):
                    if ps is None or pd is None:
                        bf_skip += 1
                        continue
                    for j in range(nh):
                        for e in range(D):
                            v = (sv[q, ps, sh0 + j, t % Bs, e] if shnd
                                 else sv[q, ps, t % Bs, sh0 + j, e])
                            if dhnd:
                                dv[q, pd, dh0 + j, t % Bd, e] = v
                            else:
                                dv[q, pd, t % Bd, dh0 + j, e] = v
        assert skipped == bf_skip, seed
        assert np.array_equal(got, exp), seed


def check_heads_full_row_is_row_copy():
    """Slice = whole row, NHD on both sides: the pinned row gather-scatter."""
    rng = np.random.default_rng(24)
    for seed in range(4):
        case = wl.random_case(950 + seed, geom=wl.Geometry(2, 2, 3, 8), max_reqs=3, max_len=20)
        g = case.geom
        src, dst = pools_for(case, rng)
        a, b = dst.copy(), dst.copy()
        o_gather_scatter(src, case, a)
        Q = g.planes
        sb = src.reshape(Q, -1).view(np.uint8)
        bb = b.reshape(Q, -1).view(np.uint8)
        o_heads(case, sb, bb, 3, 0, 0, 3, 0, 0, 3, 8)
        assert np.array_equal(a, b)


def check_heads_layout_conversion():
    """NHD -> HND with the whole row equals numpy's per-page transpose of the
    row-copied result."""
    rng = np.random.default_rng(25)
    case = wl.random_case(960, geom=wl.Geometry(1, 2, 4, 8), max_reqs=3, max_len=30,
                          src_page=4, dst_page=4)
    g = case.geom
    Q, H, D, B = g.planes, 4, 8, 4
    src, dst = pools_for(case, rng)
    ref = dst.copy()
    o_gather_scatter(src, case, ref)                     # NHD result
    P = case.dst.num_pages
    dst_hnd = np.ascontiguousarray(dst.reshape(Q, P, B, H, D).transpose(0, 1, 3, 2, 4))
    got = dst_hnd.reshape(Q, -1).view(np.uint8).copy()
    o_heads(case, src.reshape(Q, -1).view(np.uint8), got, H, 0, 0, H, 0, 1, H, D)
    back = got.view(np.uint16).reshape(Q, P, H, B, D).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(np.ascontiguousarray(back).reshape(ref.shape), ref)


def check_heads_tp_merge_and_split():
    """Two P shards of H/2 heads into one D pool of H heads (two calls) equal
    one row copy from the unsharded pool; one P pool split into two D shards
    equals the row copy cut in halves."""
    rng = np.random.default_rng(26)
    case = wl.random_case(970, geom=wl.Geometry(2, 2, 4, 8), max_reqs=3, max_len=25,
                          src_page=2, dst_page=4)
    Q, H, D = case.geom.planes, 4, 8
    full_src, dst = pools_for(case, rng)
    ref = dst.copy()
    o_gather_scatter(full_src, case, ref)
    shards = [np.ascontiguousarray(full_src[..., 2 * k:2 * k + 2, :]) for k in range(2)]
    merged = dst.copy().reshape(Q, -1).view(np.uint8)
    for k, sh in enumerate(shards):
        o_heads(case, sh.reshape(Q, -1).view(np.uint8), merged, 2, 0, 0, 4, 2 * k, 0, 2, D)
    assert np.array_equal(merged.view(np.uint16).reshape(ref.shape), ref)
    for k in range(2):
        part = np.ascontiguousarray(dst[..., 2 * k:2 * k + 2, :])
        pb = part.reshape(Q, -1).view(np.uint8)
        o_heads(case, full_src.reshape(Q, -1).view(np.uint8), pb, 4, 2 * k, 0, 2, 0, 0, 2, D)
        assert np.array_equal(pb.view(np.uint16).reshape(part.shape), ref[..., 2 * k:2 * k + 2, :])


def _torch():
    import torch
    return torch


def check_permute_torch():
    """Extract equals torch's swap of the head and sequence axes of batch 0,
    cut to the first seq positions, per plane; rebuild equals the swap back
    with a leading unit axis, written into positions < seq, with positions
    >= seq untouched (mini-infer PD page, "KV 序列化格式选择")."""
    torch = _torch()
    rng = np.random.default_rng(20)
    for Q, H, S_cap, seq, D in [(3, 2, 9, 9, 8), (2, 3, 12, 7, 16), (4, 1, 5, 5, 8),
                                (2, 4, 6, 1, 8), (1, 2, 3, 0, 8)]:
        hf = rng.integers(0, 1 << 16, size=(Q, 1, H, S_cap, D), dtype=np.uint16)
        out = np.zeros(Q * seq * H * D, np.uint16)
        oracle.extract_permute([hf[q].reshape(-1).view(np.uint8) for q in range(Q)], H, D * 2,
                               S_cap, seq, out.view(np.uint8))
        for q in range(Q):
            x = torch.from_numpy(hf[q].astype(np.int32))
            ref = torch.movedim(x.squeeze(0), 1, 0)[:seq].contiguous().numpy().astype(np.uint16)
            assert np.array_equal(out.reshape(Q, seq, H, D)[q], ref)
        flat = rng.integers(0, 1 << 16, size=(Q, seq, H, D), dtype=np.uint16)
        tgt = rng.integers(0, 1 << 16, size=(Q, 1, H, S_cap, D), dtype=np.uint16)
        before = tgt.copy()
        oracle.rebuild_permute(flat.reshape(-1).view(np.uint8), H, D * 2, seq,
                               [tgt[q].reshape(-1).view(np.uint8) for q in range(Q)], S_cap)
        for q in range(Q):
            k = torch.from_numpy(flat[q].astype(np.int32))
            ref = k.transpose(0, 1)[None].contiguous().numpy().astype(np.uint16)
            assert np.array_equal(tgt[q][:, :, :seq], ref)
            assert np.array_equal(tgt[q][:, :, seq:], before[q][:, :, seq:])
        # round trips
        back = np.zeros_like(out)
        oracle.extract_permute([tgt[q].reshape(-1).view(np.uint8) for q in range(Q)], H, D * 2,
                               S_cap, seq, back.view(np.uint8))
        assert np.array_equal(back, flat.reshape(-1))
        tgt2 = np.zeros_like(hf)
        oracle.rebuild_permute(out.view(np.uint8), H, D * 2, seq,
                               [tgt2[q].reshape(-1).view(np.uint8) for q in range(Q)], S_cap)
        assert np.array_equal(tgt2[:, :, :, :seq], hf[:, :, :, :seq])
        # H = 1 or seq = 1: the permute is a plain copy of the first seq positions
        if H == 1:
            assert np.array_equal(out.reshape(Q, seq * D), hf[:, 0, 0, :seq].reshape(Q, -1))
        if seq == 1:
            assert np.array_equal(out.reshape(Q, H, D), hf[:, 0, :, 0, :])


def check_numpy_transpose():
    """Extract equals numpy.transpose of the first seq positions, axes (1, 0, 2)."""
    rng = np.random.default_rng(21)
    Q, H, S_cap, seq, D = 3, 5, 11, 8, 16
    hf = rng.integers(0, 1 << 16, size=(Q, 1, H, S_cap, D), dtype=np.uint16)
    out = np.zeros(Q * seq * H * D, np.uint16)
    oracle.extract_permute([hf[q].reshape(-1).view(np.uint8) for q in range(Q)], H, D * 2,
                           S_cap, seq, out.view(np.uint8))
    ref = np.stack([np.transpose(hf[q, 0, :, :seq, :], (1, 0, 2)) for q in range(Q)])
    assert np.array_equal(out.reshape(ref.shape), ref)


def golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                p = line.split()
                rows.append((p[0], *map(int, p[1:7]), float(p[7])))
    return rows


def check_closed_form_sizes():
    """The KV byte formula reproduces every size the pages print, and a gather
    of such a request fills exactly that many staging bytes."""
    for name, L, nkv, H, D, b, seq, mib in golden_rows():
        nbytes = oracle.kv_bytes(seq, L, H, D, b, num_kv=nkv)
        assert round(nbytes / 2 ** 20, 2) == mib, (name, seq, nbytes / 2 ** 20, mib)
        # the same count from the Mooncake page's form p * l * (2 d / gqa) * s,
        # where 2 d / gqa (d = hidden size, gqa = query heads per KV head)
        # equals num_kv * kv_heads * head_dim
        assert seq * L * (nkv * H * D) * b == nbytes
    # gather of a Qwen2.5-1.5B request of 128 tokens: 3.50 MiB of staging
    rng = np.random.default_rng(22)
    L, H, D, n = 28, 2, 128, 128
    Q = 2 * L
    pool = rand_pool(rng, Q, 256, H, D)
    case = wl.PagedCase("sz", wl.Geometry(L, 2, H, D, "f16"), wl.csr_from_lengths([n]),
                        wl.side_from_slot_lists([rng.permutation(256)[:n]], 256), None, 0, 0, 0)
    size = oracle.kv_bytes(n, L, H, D, 2)
    a = np.zeros(size // 2 + 8, np.uint16)
    b = np.full(size // 2 + 8, 0xFFFF, np.uint16)
    o_gather(pool, case, case.src, a)
    o_gather(pool, case, case.src, b)
    written = np.flatnonzero(a != b)
    assert written.size == 8 and written[0] == size // 2
    assert size == 3.5 * 2 ** 20


ALL_CHECKS = [
    check_gather_bruteforce,
    check_scatter_bruteforce,
    check_gather_scatter_bruteforce,
    check_exhaustive_injective,
    check_take_special_case,
    check_page_expansion,
    check_batch_is_concatenation,
    check_roundtrips,
    check_untouched_and_extent,
    check_token_major_pool,
    check_mixed_strides,
    check_block_interleaved_pools,
    check_threads_agree,
    check_permute_torch,
    check_numpy_transpose,
    check_closed_form_sizes,
    check_oor_boundaries,
    check_table_index_boundaries,
    check_empty_page_table,
    check_heads_bruteforce,
    check_heads_full_row_is_row_copy,
    check_heads_layout_conversion,
    check_heads_tp_merge_and_split,
]
