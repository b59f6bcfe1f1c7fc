"""GPU parity at small sizes: every kvx call through the C ABI against the CPU
oracle, byte for byte over the whole destination (pool, staging plus guard
bytes, or HF tensors), on seeded random inputs that span several chunks and a
ragged tail, across row sizes that take both copy variants."""
import numpy as np
import pytest
import torch

import oracle
import scatter_kvx_gather_amd as kvx
import workloads as wl
from tests.gpu_util import (DEV, assert_bytes_equal, d, d_aligned, layout_of, oracle_gather,
                            oracle_gather_scatter, oracle_scatter, requests, say, table)

pytestmark = pytest.mark.gpu

# (geometry, max tokens per request): row sizes 16 B .. 32 KiB, wide (multiples
# of 1 KiB in {1, 2, 4, 8, 16} KiB) and flat (everything else), four dtypes
GEOMS = [
    (wl.Geometry(1, 2, 1, 8, "bf16"), 300),      # R = 16
    (wl.Geometry(2, 1, 3, 8, "f16"), 200),       # R = 48
    (wl.Geometry(1, 2, 3, 16, "bf16"), 200),     # R = 96
    (wl.Geometry(2, 2, 1, 128, "f16"), 150),     # R = 256
    (wl.Geometry(1, 2, 2, 128, "f16"), 150),     # R = 512
    (wl.Geometry(2, 2, 3, 128, "bf16"), 100),    # R = 768
    (wl.Geometry(2, 2, 4, 128, "bf16"), 100),    # R = 1 KiB  (wide)
    (wl.Geometry(3, 1, 1, 576, "bf16"), 100),    # R = 1152   (MLA-sized row)
    (wl.Geometry(2, 2, 8, 128, "bf16"), 70),     # R = 2 KiB  (wide)
    (wl.Geometry(1, 2, 12, 128, "bf16"), 60),    # R = 3 KiB
    (wl.Geometry(1, 2, 16, 128, "bf16"), 50),    # R = 4 KiB  (wide)
    (wl.Geometry(1, 2, 32, 128, "bf16"), 20),    # R = 8 KiB  (wide)
    (wl.Geometry(1, 1, 64, 128, "bf16"), 12),    # R = 16 KiB (wide)
    (wl.Geometry(1, 1, 128, 128, "bf16"), 8),    # R = 32 KiB (flat, several passes)
    (wl.Geometry(1, 2, 2, 8, "fp8"), 300),       # R = 16, 1-byte elements
    (wl.Geometry(1, 2, 33, 8, "bf16"), 100),     # R = 528: smallest row-loop row
    (wl.Geometry(1, 1, 1023, 8, "bf16"), 10),    # R = 16368: largest row-loop row
    (wl.Geometry(1, 1, 4095, 8, "bf16"), 5),     # R = 65520 (flat)
    (wl.Geometry(1, 1, 256, 128, "bf16"), 5),    # R = 64 KiB: the largest row accepted
    (wl.Geometry(2, 2, 2, 128, "f32"), 80),      # R = 1 KiB, 4-byte elements
]


def run_paged_case(case, seed, guard=256, align=0):
    """gather (nontemporal and cached staging stores), scatter and
    gather-scatter of a case, every destination byte and the skip counts
    against the oracle; `align`: the pools' and staging buffers' first bytes
    at that multiple."""
    g = case.geom
    dev_pool = (lambda a: d_aligned(a, align)) if align else d
    Q, R = g.planes, g.row_bytes
    rng = np.random.default_rng(seed)
    src_h = rng.integers(0, 256, (Q, case.src.num_slots, R), dtype=np.uint8)
    dst_h = rng.integers(0, 256, (Q, case.dst.num_slots, R), dtype=np.uint8)
    n = case.total_tokens * Q * R
    stage_prefill = rng.integers(0, 256, n + guard, dtype=np.uint8)
    stage_in = rng.integers(0, 256, n, dtype=np.uint8)
    lay = layout_of(g)
    reqs = requests(case)
    st, dt = table(case.src), table(case.dst)
    src_d = dev_pool(src_h)
    src = kvx.Pool(src_d, case.src.num_pages, case.src.page_size)
    skipped = torch.zeros(3, dtype=torch.int64, device=DEV)

    say(case.name, f"Q={Q} R={R} T={case.total_tokens} pages {case.src.page_size}/"
        f"{case.dst.page_size}: gather")
    staging = dev_pool(stage_prefill)
    kvx.gather(lay, src, st, reqs, staging, skipped=skipped[0:1])
    # the same gather with ordinary stores for the staging (KVX_OUT_CACHED)
    say(case.name, "gather, cached output")
    staging_c = dev_pool(stage_prefill)
    kvx.gather(lay, src, st, reqs, staging_c, cached_out=True)
    say(case.name, "scatter")
    dst_d1 = dev_pool(dst_h)
    kvx.scatter(lay, dev_pool(stage_in), reqs, kvx.Pool(dst_d1, case.dst.num_pages, case.dst.page_size),
                dt, skipped=skipped[1:2])
    say(case.name, "gather_scatter")
    dst_d2 = dev_pool(dst_h)
    kvx.gather_scatter(lay, src, st, reqs,
                       kvx.Pool(dst_d2, case.dst.num_pages, case.dst.page_size), dt,
                       skipped=skipped[2:3])
    torch.cuda.synchronize()

    exp_stage = stage_prefill.copy()
    s0 = oracle_gather(case, src_h, exp_stage)
    exp_dst1 = dst_h.copy()
    s1 = oracle_scatter(case, stage_in, exp_dst1)
    exp_dst2 = dst_h.copy()
    s2 = oracle_gather_scatter(case, src_h, exp_dst2)
    assert_bytes_equal(staging.cpu().numpy(), exp_stage, f"{case.name} gather")
    assert_bytes_equal(staging_c.cpu().numpy(), exp_stage, f"{case.name} gather, cached output")
    assert_bytes_equal(dst_d1.cpu().numpy(), exp_dst1, f"{case.name} scatter")
    assert_bytes_equal(dst_d2.cpu().numpy(), exp_dst2, f"{case.name} gather_scatter")
    assert skipped.cpu().tolist() == [s0, s1, s2], case.name


@pytest.mark.parametrize("gi", range(len(GEOMS)))
@pytest.mark.parametrize("pages", [(1, 1), (16, 16), (1, 16), (3, 2)])
def test_paged_ops(gi, pages):
    g, max_len = GEOMS[gi]
    seed = 1000 * gi + 10 * pages[0] + pages[1]
    case = wl.random_case(seed, geom=g, max_reqs=5, max_len=max_len, src_page=pages[0],
                          dst_page=pages[1])
    run_paged_case(case, seed)


@pytest.mark.parametrize("seed", range(12))
def test_paged_out_of_range_ids(seed):
    g, max_len = GEOMS[seed % len(GEOMS)]
    case = wl.random_case(5000 + seed, geom=g, max_reqs=6, max_len=max_len, oor_frac=0.15)
    run_paged_case(case, seed)


@pytest.mark.parametrize("seed", range(16))
def test_paged_table_index_faults(seed):
    """Page-table offsets that send lookups below 0, past the end of the
    page-id array or into another request's list (random_case's
    index_faults), alone and with out-of-range ids: whole destinations and
    skip counts against the oracle.  Seeds 12-15 take batches above 64
    requests (the many-request lookup)."""
    g, max_len = GEOMS[(3 * seed) % len(GEOMS)]
    many = seed >= 12
    k = 0
    while True:                     # the first seed of the family that fits
        case = wl.random_case(5600 + 100 * k + seed, geom=g, max_reqs=120 if many else 6,
                              max_len=min(max_len, 6) if many else max_len,
                              oor_frac=0.1 if seed % 2 else 0.0, index_faults=True)
        if not many or case.num_reqs > 64:
            break
        k += 1
    run_paged_case(case, seed)


def test_paged_table_index_worked_example():
    """The oracle pin's worked example of the page-table reads on the GPU:
    a list starting one entry early, a page one past the end of the array, an
    empty list that reads on into the next entries, offsets 2**62 before and
    after the array, and offsets at the ends of the int64 range, where the
    index runs past 2**63 - 1 or starts at -2**63 (skipped, not wrapped)."""
    big = 1 << 62
    i64max, i64min = (1 << 63) - 1, -(1 << 63)
    lens = [4, 4, 2, 2, 2, 6, 6]
    src = wl.Side(4, 2, np.array([-1, 2, 0, -big, big, i64max - 1, i64min, 3], np.int64),
                  np.array([1, 3, 0], np.int32))
    dst = wl.Side(4, 2, np.array([-1, 2, 1, -big, big, i64min + 1, i64max, 3], np.int64),
                  np.array([1, 3, 0], np.int32))
    for g in (wl.Geometry(1, 2, 1, 8), wl.Geometry(2, 2, 8, 128)):
        case = wl.PagedCase(f"idx_example_R{g.row_bytes}", g, wl.csr_from_lengths(lens), src,
                            dst, 0, 0, 0)
        run_paged_case(case, 11)


def test_paged_empty_page_tables():
    """A side whose page-id array is empty (num_ids 0, page_ids passed as
    NULL): every index is out of range, so every row is skipped and counted
    and leaves its destination untouched, while the other side's table is an
    ordinary one."""
    lens = [5, 0, 7]
    pg = np.array([0, 2, 2, 4], np.int64)
    ids = np.array([2, 0, 3, 1], np.int32)
    empty = np.zeros(0, np.int32)
    for g in (wl.Geometry(1, 2, 1, 8), wl.Geometry(2, 2, 8, 128)):
        for name, sids, dids in (("src", empty, ids), ("dst", ids, empty), ("both", empty, empty)):
            case = wl.PagedCase(f"empty_table_{name}_R{g.row_bytes}", g, wl.csr_from_lengths(lens),
                                wl.Side(4, 4, pg, sids), wl.Side(4, 4, pg, dids), 0, 0, 0)
            run_paged_case(case, 13)


def test_many_requests_and_empty_ones():
    # 300 requests, a third of them empty: the token -> request search and the
    # chunks that straddle request boundaries
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 9, 300)
    lens[::3] = 0
    g = wl.Geometry(1, 2, 8, 128, "bf16")
    S = int(lens.sum()) + 50
    perm_s, perm_d = rng.permutation(S), rng.permutation(S)
    lists_s, lists_d, pos = [], [], 0
    for n in lens:
        lists_s.append(perm_s[pos:pos + n])
        lists_d.append(perm_d[pos:pos + n])
        pos += int(n)
    case = wl.PagedCase("many_reqs", g, wl.csr_from_lengths(lens),
                        wl.side_from_slot_lists(lists_s, S), wl.side_from_slot_lists(lists_d, S),
                        0, 0, 0)
    run_paged_case(case, 3)


def big_case(name, g, lens, src_page, dst_page, seed, oor_frac=0.0):
    """Ragged batch of given lengths: source pages drawn with replacement,
    distinct destination pages, optionally some ids out of range."""
    rng = np.random.default_rng(seed)
    ps = [-(-int(n) // src_page) for n in lens]
    pd = [-(-int(n) // dst_page) for n in lens]
    ns, nd = sum(ps) + 5, sum(pd) + 5
    src = wl.side_from_page_lists([rng.integers(0, ns, p) for p in ps], ns, src_page)
    perm = rng.permutation(nd)
    dl, pos = [], 0
    for p in pd:
        dl.append(perm[pos:pos + p])
        pos += p
    dst = wl.side_from_page_lists(dl, nd, dst_page)
    for side in (src, dst):
        if oor_frac:
            m = rng.random(side.ids.size) < oor_frac
            side.ids = np.where(m, side.num_pages + 3, side.ids).astype(np.int32)
    return wl.PagedCase(name, g, wl.csr_from_lengths(lens), src, dst, 0, 0, 0)


# Launches above 64 MiB each way move 2 KiB per wave (below it, 8 KiB
# chunks): two 1 KiB rows, one 2 KiB row, or a 2 KiB piece of a 4, 8 or
# 16 KiB row (a skipped row counted once); ragged and empty requests, mixed
# page sizes, out-of-range ids.
BIG = [
    (wl.Geometry(8, 2, 4, 128, "bf16"), [1500, 0, 2333, 1801], 1, 1, 0.0),     # R = 1 KiB
    (wl.Geometry(8, 2, 4, 128, "bf16"), [2600, 2, 2100], 16, 3, 0.02),         # R = 1 KiB
    (wl.Geometry(4, 2, 8, 128, "bf16"), [3000, 1700, 7], 1, 16, 0.02),         # R = 2 KiB
    (wl.Geometry(2, 2, 16, 128, "bf16"), [2100, 1, 2500], 16, 16, 0.0),        # R = 4 KiB
    (wl.Geometry(2, 2, 16, 128, "bf16"), [1900, 0, 2700], 1, 2, 0.03),         # R = 4 KiB
    (wl.Geometry(1, 2, 32, 128, "bf16"), [3200, 1000, 17], 16, 3, 0.02),       # R = 8 KiB
    (wl.Geometry(1, 1, 64, 128, "bf16"), [2500, 2000, 5], 1, 1, 0.0),          # R = 16 KiB
]


@pytest.mark.parametrize("bi", range(len(BIG)))
def test_one_row_per_wave_launches(bi):
    g, lens, sp, dp, oor = BIG[bi]
    assert sum(lens) * g.planes * g.row_bytes > 64 << 20
    run_paged_case(big_case(f"big{bi}", g, lens, sp, dp, 700 + bi, oor), 700 + bi)


# Pools whose pages hold runs of at least 64 KiB of a plane, planes aligned
# to 128 KiB, in launches above 64 MiB each way: the kernels take each
# request's tokens in DRAM-page order (rows 32 KiB apart on the two waves of
# one workgroup, or in one wave for 1 KiB rows; the same 2 KiB piece of two
# 4-16 KiB rows on the two waves of one workgroup; a block past the
# request's end in natural order).  One side or both paired (a staging side
# pairs at any page size), ragged requests whose starts are not block
# aligned, partial last pages, out-of-range ids, a batch above 64 requests.
# (geometry, lengths, src page, dst page, oor)
DRAM = [
    (wl.Geometry(36, 2, 8, 128, "bf16"), [300, 0, 257, 64, 1], 64, 64, 0.0),   # 2 KiB
    (wl.Geometry(36, 2, 8, 128, "bf16"), [500, 130, 33], 32, 64, 0.02),
    (wl.Geometry(36, 2, 8, 128, "bf16"), [420, 65], 64, 1, 0.0),               # source only
    (wl.Geometry(36, 2, 8, 128, "bf16"), [400, 97], 1, 32, 0.01),              # destination only
    (wl.Geometry(36, 2, 8, 128, "bf16"), [600, 70, 1], 64, 32, 0.01),
    (wl.Geometry(28, 2, 4, 128, "bf16"), [700, 129, 500], 128, 64, 0.02),      # 1 KiB
    (wl.Geometry(36, 2, 4, 128, "bf16"), [900, 250], 64, 128, 0.0),
    (wl.Geometry(36, 2, 8, 128, "bf16"), "many", 32, 32, 0.01),                # > 64 requests
    (wl.Geometry(36, 2, 8, 128, "bf16"), [700, 3, 120], 1, 1, 0.01),           # staging only
    (wl.Geometry(8, 2, 16, 128, "bf16"), [600, 17, 500], 16, 32, 0.02),        # 4 KiB pieces
    (wl.Geometry(8, 2, 16, 128, "bf16"), [1200], 1, 16, 0.0),
    (wl.Geometry(4, 2, 32, 128, "bf16"), [700, 450], 8, 16, 0.01),             # 8 KiB pieces
    (wl.Geometry(2, 2, 64, 128, "bf16"), [1000, 3, 150], 4, 1, 0.01),          # 16 KiB pieces
]


@pytest.mark.parametrize("di", range(len(DRAM)))
def test_dram_page_order(di):
    g, lens, sp, dp, oor = DRAM[di]
    if lens == "many":
        rng = np.random.default_rng(880 + di)
        lens = [int(x) for x in rng.integers(0, 61, 70)]
    assert sum(lens) * g.planes * g.row_bytes > 64 << 20
    run_paged_case(big_case(f"dram{di}", g, lens, sp, dp, 880 + di, oor), 880 + di,
                   align=128 << 10)


# One-row-per-wave launches of batches above 64 requests (the kernels with
# the guessed window and the 64-way search): equal lengths, where the guess
# hits, and ragged lengths with empty requests, where it often misses.
# (geometry, requests, max length, empty fraction, src page, dst page, oor)
BIG_MANY = [
    (wl.Geometry(4, 2, 8, 128, "bf16"), 6000, 3, 0.0, 1, 1, 0.0),       # R = 2 KiB, equal
    (wl.Geometry(4, 2, 8, 128, "bf16"), 6000, 6, 0.3, 1, 1, 0.0),       # R = 2 KiB, ragged
    (wl.Geometry(8, 2, 4, 128, "bf16"), 3000, 12, 0.2, 16, 3, 0.02),    # R = 1 KiB
    (wl.Geometry(2, 2, 16, 128, "bf16"), 70000, 1, 0.6, 1, 2, 0.0),     # R = 4 KiB, 2 search rounds
    (wl.Geometry(1, 2, 32, 128, "bf16"), 5000, 6, 0.3, 2, 1, 0.02),     # R = 8 KiB
]


@pytest.mark.parametrize("bi", range(len(BIG_MANY)))
def test_one_row_per_wave_many_requests(bi):
    g, nreq, maxlen, zf, sp, dp, oor = BIG_MANY[bi]
    rng = np.random.default_rng(760 + bi)
    if zf == 0.0:
        lens = np.full(nreq, maxlen, np.int64)
    else:
        lens = np.where(rng.random(nreq) < zf, 0, rng.integers(1, maxlen + 1, nreq))
    lens[-1] = max(int(lens[-1]), 1)
    assert lens.sum() * g.planes * g.row_bytes > 64 << 20 and nreq > 64
    run_paged_case(big_case(f"bigmany{bi}", g, list(lens), sp, dp, 760 + bi, oor), 760 + bi)


# Gathers of short requests (at most 64 KiB of rows per plane on average)
# run in token-major chunk order: every copy shape (flat, row-loop, wide with
# several rows or one row per chunk, 2 KiB pieces of larger rows), ragged
# lengths with empty requests, below and above 64 requests, page sizes 1-16,
# some ids out of range.  (geometry, requests, max length, src page, dst page)
SHORT = [
    (wl.Geometry(1, 2, 1, 8, "bf16"), 40, 30, 1, 1),          # R = 16, flat
    (wl.Geometry(2, 2, 3, 128, "bf16"), 90, 40, 2, 16),       # R = 768, row-loop
    (wl.Geometry(3, 1, 1, 576, "bf16"), 300, 50, 1, 3),       # R = 1152, row-loop
    (wl.Geometry(2, 2, 4, 128, "bf16"), 70, 60, 16, 1),       # R = 1 KiB, wide
    (wl.Geometry(2, 2, 8, 128, "bf16"), 2000, 20, 1, 2),      # R = 2 KiB, wide
    (wl.Geometry(1, 2, 32, 128, "bf16"), 400, 12, 1, 1),      # R = 8 KiB
    (wl.Geometry(4, 2, 8, 128, "bf16"), 6000, 3, 1, 1),       # R = 2 KiB, above one round
    (wl.Geometry(2, 2, 16, 128, "bf16"), 3000, 8, 1, 1),      # R = 4 KiB, 2 KiB pieces
]


@pytest.mark.parametrize("si", range(len(SHORT)))
def test_gather_short_requests(si):
    g, nreq, maxlen, sp, dp = SHORT[si]
    rng = np.random.default_rng(940 + si)
    lens = np.where(rng.random(nreq) < 0.15, 0, rng.integers(1, maxlen + 1, nreq))
    lens[-1] = max(int(lens[-1]), 1)
    assert lens.sum() * g.row_bytes <= (64 << 10) * nreq      # the short-request order
    run_paged_case(big_case(f"short{si}", g, list(lens), sp, dp, 940 + si, 0.02), 940 + si)


@pytest.mark.parametrize("nreq", [1, 2, 63, 64, 65, 130])
@pytest.mark.parametrize("R", [2048, 512])
def test_request_lookup_limits(nreq, R):
    """Batches around the 64-request limit of the wave-parallel request lookup,
    with tiny and empty requests so one chunk crosses many request ends."""
    rng = np.random.default_rng(nreq * 7 + R)
    lens = rng.integers(0, 6, nreq)
    lens[rng.integers(nreq)] = 0
    lens[-1] = max(int(lens[-1]), 1)
    g = wl.Geometry(1, 2, R // 256, 128, "bf16")
    S = int(lens.sum()) + 40
    perm_s, perm_d = rng.permutation(S), rng.permutation(S)
    ls, ld, pos = [], [], 0
    for n in lens:
        ls.append(perm_s[pos:pos + n])
        ld.append(perm_d[pos:pos + n])
        pos += int(n)
    case = wl.PagedCase(f"lookup_{nreq}", g, wl.csr_from_lengths(lens),
                        wl.side_from_slot_lists(ls, S), wl.side_from_slot_lists(ld, S), 0, 0, 0)
    run_paged_case(case, nreq)


# Batches of more than 64 requests take the 64-way search for a chunk's first
# request: one round up to 4096 requests, two up to 262144, three above.
# Mostly-empty batches make one chunk (up to 64 tokens) cross more than 63
# request starts, so some lanes finish past the 64-request window.
# (requests, fraction empty, row bytes)
LARGE_BATCHES = [
    (256, 0.3, 2048), (256, 0.3, 16),
    (4096, 0.3, 512), (4097, 0.3, 2048), (4097, 0.0, 16),
    (9000, 0.5, 512), (70000, 0.3, 16), (70000, 0.3, 512),
    (300000, 0.6, 16), (300000, 0.6, 512),
    (700, 0.9, 16), (3000, 0.97, 16), (3000, 0.97, 512), (20000, 0.9, 2048),
]


@pytest.mark.parametrize("bi", range(len(LARGE_BATCHES)))
def test_request_lookup_large_batches(bi):
    nreq, zf, R = LARGE_BATCHES[bi]
    rng = np.random.default_rng(9100 + bi)
    lens = np.where(rng.random(nreq) < zf, 0, rng.integers(1, 4, nreq))
    lens[-1] = max(int(lens[-1]), 1)
    g = wl.Geometry(1, 2, 1, R // 2, "bf16")
    S = int(lens.sum()) + 40
    perm_s, perm_d = rng.permutation(S), rng.permutation(S)
    offs = np.concatenate([[0], np.cumsum(lens)])
    ls = np.split(perm_s[:offs[-1]], offs[1:-1])
    ld = np.split(perm_d[:offs[-1]], offs[1:-1])
    case = wl.PagedCase(f"lookup_{nreq}_{zf}_{R}", g, wl.csr_from_lengths(lens),
                        wl.side_from_slot_lists(ls, S), wl.side_from_slot_lists(ld, S), 0, 0, 0)
    run_paged_case(case, 9100 + bi)


def run_paged_case_token_major(case, seed):
    """gather, scatter and gather-scatter with both pools token-major (plane q
    of slot s at (s * Q + q) * R), which the kernels move in token-major chunk
    order where they write such a pool; every byte against the oracle."""
    g = case.geom
    Q, R = g.planes, g.row_bytes
    rng = np.random.default_rng(seed)
    src_h = rng.integers(0, 256, case.src.num_slots * Q * R, dtype=np.uint8)
    dst_h = rng.integers(0, 256, case.dst.num_slots * Q * R, dtype=np.uint8)
    n = case.total_tokens * Q * R
    stage_in = rng.integers(0, 256, n, dtype=np.uint8)
    lay, reqs = layout_of(g), requests(case)
    st, dt = table(case.src), table(case.dst)

    def pool(t, side):
        p = kvx.Pool([t.data_ptr() + q * R for q in range(Q)], side.num_pages, side.page_size,
                     slot_stride=Q * R, keep=t)
        return p

    def planes(flat):
        return [flat[q * R:] for q in range(Q)]

    src_d = d(src_h)
    skipped = torch.zeros(3, dtype=torch.int64, device=DEV)
    say(case.name, f"token-major Q={Q} R={R} T={case.total_tokens} pages "
        f"{case.src.page_size}/{case.dst.page_size}: gather")
    staging = torch.zeros(n, dtype=torch.uint8, device=DEV)
    kvx.gather(lay, pool(src_d, case.src), st, reqs, staging, skipped=skipped[0:1])
    say(case.name, "token-major scatter")
    dst_d1 = d(dst_h)
    kvx.scatter(lay, d(stage_in), reqs, pool(dst_d1, case.dst), dt, skipped=skipped[1:2])
    say(case.name, "token-major gather_scatter")
    dst_d2 = d(dst_h)
    kvx.gather_scatter(lay, pool(src_d, case.src), st, reqs, pool(dst_d2, case.dst), dt,
                       skipped=skipped[2:3])
    torch.cuda.synchronize()

    exp_stage = np.zeros(n, np.uint8)
    s0 = oracle.gather(planes(src_h), Q * R, case.src.page_size, case.src.num_pages, R,
                       case.tok_off, case.src.pg_off, case.src.ids, exp_stage)
    exp_dst1 = dst_h.copy()
    s1 = oracle.scatter(stage_in, R, case.tok_off, case.dst.pg_off, case.dst.ids,
                        planes(exp_dst1), Q * R, case.dst.page_size, case.dst.num_pages)
    exp_dst2 = dst_h.copy()
    s2 = oracle.gather_scatter(planes(src_h), Q * R, case.src.page_size, case.src.num_pages,
                               case.src.pg_off, case.src.ids, R, case.tok_off, planes(exp_dst2),
                               Q * R, case.dst.page_size, case.dst.num_pages, case.dst.pg_off,
                               case.dst.ids)
    assert_bytes_equal(staging.cpu().numpy(), exp_stage, f"{case.name} token-major gather")
    assert_bytes_equal(dst_d1.cpu().numpy(), exp_dst1, f"{case.name} token-major scatter")
    assert_bytes_equal(dst_d2.cpu().numpy(), exp_dst2, f"{case.name} token-major gather_scatter")
    assert skipped.cpu().tolist() == [s0, s1, s2], case.name


def _ragged(rng, nreq, maxlen, zf):
    lens = np.where(rng.random(nreq) < zf, 0, rng.integers(1, maxlen + 1, nreq))
    lens[-1] = max(int(lens[-1]), 1)
    return list(lens)


# Token-major pools: small launches (8 KiB chunks), launches above 64 MiB each
# way (one 2 KiB row or two 1 KiB rows per wave), batches above 64 requests,
# mixed page sizes and out-of-range ids.
# (geometry, requests, max length, empty fraction, src page, dst page, oor)
TOKEN_MAJOR = [
    (wl.Geometry(2, 2, 8, 128, "bf16"), 3, 60, 0.0, 1, 1, 0.0),
    (wl.Geometry(2, 2, 4, 128, "f16"), 5, 50, 0.2, 16, 1, 0.05),
    (wl.Geometry(3, 2, 1, 8, "bf16"), 4, 80, 0.0, 3, 2, 0.0),          # R = 16, flat copy
    (wl.Geometry(3, 1, 1, 576, "bf16"), 4, 90, 0.0, 1, 16, 0.0),       # R = 1152, row loop
    (wl.Geometry(4, 2, 8, 128, "bf16"), 200, 6, 0.3, 1, 1, 0.02),      # > 64 requests
    (wl.Geometry(8, 2, 8, 128, "bf16"), 8, 700, 0.0, 1, 1, 0.0),       # > 64 MiB each way
    (wl.Geometry(8, 2, 4, 128, "bf16"), 3000, 12, 0.2, 16, 3, 0.02),   # both, 1 KiB rows
]


@pytest.mark.parametrize("ti", range(len(TOKEN_MAJOR)))
def test_token_major_pools(ti):
    g, nreq, maxlen, zf, sp, dp, oor = TOKEN_MAJOR[ti]
    rng = np.random.default_rng(8800 + ti)
    lens = _ragged(rng, nreq, maxlen, zf)
    run_paged_case_token_major(big_case(f"tm{ti}", g, lens, sp, dp, 8800 + ti, oor), 8800 + ti)


def run_paged_case_blocks(case, seed, align=0):
    """gather, scatter and gather-scatter between pools whose blocks hold
    several planes' pages: the source one [blocks][2][B][R] tensor per layer
    (K and V pages of a block together), the destination one
    [blocks][layers][2][B][R] tensor; each plane addressed through the block
    length as its page stride.  Every byte against the oracle.  `align`: the
    tensors' first bytes at that multiple."""
    dev_t = (lambda a: d_aligned(a, align)) if align else d
    g = case.geom
    Q, R, L = g.planes, g.row_bytes, g.num_layers
    kv = g.num_kv
    bs, bd = case.src.page_size, case.dst.page_size
    rng = np.random.default_rng(seed)
    src_h = [rng.integers(0, 256, case.src.num_pages * kv * bs * R, dtype=np.uint8)
             for _ in range(L)]
    dst_h = rng.integers(0, 256, case.dst.num_pages * Q * bd * R, dtype=np.uint8)
    n = case.total_tokens * Q * R
    stage_in = rng.integers(0, 256, n, dtype=np.uint8)
    lay, reqs = layout_of(g), requests(case)
    st, dt = table(case.src), table(case.dst)
    src_d = [dev_t(a) for a in src_h]
    src = kvx.Pool([src_d[q // kv].data_ptr() + (q % kv) * bs * R for q in range(Q)],
                   case.src.num_pages, bs, slot_stride=R, page_stride=kv * bs * R,
                   keep=src_d)

    def dst_pool(t):
        p = kvx.Pool([t.data_ptr() + q * bd * R for q in range(Q)], case.dst.num_pages, bd,
                     slot_stride=R, page_stride=Q * bd * R, keep=t)
        return p

    src_planes = [src_h[q // kv][(q % kv) * bs * R:] for q in range(Q)]

    def dst_planes(flat):
        return [flat[q * bd * R:] for q in range(Q)]

    skipped = torch.zeros(3, dtype=torch.int64, device=DEV)
    say(case.name, f"blocks Q={Q} R={R} T={case.total_tokens} pages {bs}/{bd}: gather")
    staging = torch.zeros(n, dtype=torch.uint8, device=DEV)
    kvx.gather(lay, src, st, reqs, staging, skipped=skipped[0:1])
    say(case.name, "blocks scatter")
    dst_d1 = dev_t(dst_h)
    kvx.scatter(lay, d(stage_in), reqs, dst_pool(dst_d1), dt, skipped=skipped[1:2])
    say(case.name, "blocks gather_scatter")
    dst_d2 = dev_t(dst_h)
    kvx.gather_scatter(lay, src, st, reqs, dst_pool(dst_d2), dt, skipped=skipped[2:3])
    torch.cuda.synchronize()

    exp_stage = np.zeros(n, np.uint8)
    s0 = oracle.gather(src_planes, R, bs, case.src.num_pages, R, case.tok_off, case.src.pg_off,
                       case.src.ids, exp_stage, page_stride=kv * bs * R)
    exp_dst1 = dst_h.copy()
    s1 = oracle.scatter(stage_in, R, case.tok_off, case.dst.pg_off, case.dst.ids,
                        dst_planes(exp_dst1), R, bd, case.dst.num_pages,
                        page_stride=Q * bd * R)
    exp_dst2 = dst_h.copy()
    s2 = oracle.gather_scatter(src_planes, R, bs, case.src.num_pages, case.src.pg_off,
                               case.src.ids, R, case.tok_off, dst_planes(exp_dst2), R, bd,
                               case.dst.num_pages, case.dst.pg_off, case.dst.ids,
                               src_page_stride=kv * bs * R, dst_page_stride=Q * bd * R)
    assert_bytes_equal(staging.cpu().numpy(), exp_stage, f"{case.name} blocks gather")
    assert_bytes_equal(dst_d1.cpu().numpy(), exp_dst1, f"{case.name} blocks scatter")
    assert_bytes_equal(dst_d2.cpu().numpy(), exp_dst2, f"{case.name} blocks gather_scatter")
    assert skipped.cpu().tolist() == [s0, s1, s2], case.name


# Pools whose blocks hold several planes' pages (page stride = block length):
# small launches, launches above 64 MiB each way, batches above 64 requests,
# page sizes 1 to 16 and out-of-range ids.
# (geometry, requests, max length, empty fraction, src page, dst page, oor)
BLOCKS = [
    (wl.Geometry(2, 2, 8, 128, "bf16"), 3, 60, 0.0, 16, 16, 0.0),
    (wl.Geometry(2, 2, 4, 128, "f16"), 5, 50, 0.2, 16, 1, 0.05),
    (wl.Geometry(3, 2, 1, 8, "bf16"), 4, 80, 0.0, 3, 2, 0.0),          # R = 16, flat copy
    (wl.Geometry(3, 1, 1, 576, "bf16"), 4, 90, 0.0, 1, 16, 0.0),       # R = 1152, row loop
    (wl.Geometry(4, 2, 8, 128, "bf16"), 200, 6, 0.3, 16, 16, 0.02),    # > 64 requests
    (wl.Geometry(8, 2, 8, 128, "bf16"), 8, 700, 0.0, 16, 16, 0.0),     # > 64 MiB each way
    (wl.Geometry(8, 2, 4, 128, "bf16"), 3000, 12, 0.2, 16, 2, 0.02),   # both, 1 KiB rows
    (wl.Geometry(2, 2, 32, 128, "bf16"), 12, 700, 0.0, 16, 4, 0.0),    # R = 8 KiB, 2 KiB pieces
]


@pytest.mark.parametrize("bi", range(len(BLOCKS)))
def test_block_interleaved_pools(bi):
    g, nreq, maxlen, zf, sp, dp, oor = BLOCKS[bi]
    rng = np.random.default_rng(8900 + bi)
    lens = _ragged(rng, nreq, maxlen, zf)
    run_paged_case_blocks(big_case(f"blocks{bi}", g, lens, sp, dp, 8900 + bi, oor), 8900 + bi)


# The same block pools, tensors aligned to 128 KiB, in launches above 64 MiB
# each way with one 2 KiB row or two 1 KiB rows per wave: where a block's K
# and V pages (32 or 64 KiB each) share DRAM pages, the kernels run the two
# planes of a token on the two waves of one workgroup (plane-pair order).
# (geometry, requests, max length, empty fraction, src page, dst page, oor)
BLOCKS_PAIRED = [
    (wl.Geometry(36, 2, 8, 128, "bf16"), 3, 600, 0.0, 16, 16, 0.01),   # both sides
    (wl.Geometry(36, 2, 8, 128, "bf16"), 3, 700, 0.0, 32, 3, 0.0),     # source, 64 KiB pages
    (wl.Geometry(36, 2, 4, 128, "bf16"), 4, 900, 0.0, 1, 32, 0.02),    # destination, 1 KiB rows
    (wl.Geometry(35, 2, 8, 128, "bf16"), 90, 20, 0.2, 16, 16, 0.01),   # > 64 requests
]


@pytest.mark.parametrize("bi", range(len(BLOCKS_PAIRED)))
def test_block_pools_plane_pairs(bi):
    g, nreq, maxlen, zf, sp, dp, oor = BLOCKS_PAIRED[bi]
    rng = np.random.default_rng(8950 + bi)
    lens = _ragged(rng, nreq, maxlen, zf)
    assert sum(lens) * g.planes * g.row_bytes > 64 << 20
    run_paged_case_blocks(big_case(f"pairs{bi}", g, lens, sp, dp, 8950 + bi, oor), 8950 + bi,
                          align=128 << 10)


def test_plane_pairs_odd_plane_count():
    """Three planes (one per layer, num_kv = 1) whose pages lie one page apart
    in [blocks][4][16][R] tensors (a block's fourth page unused), aligned to
    128 KiB, in a launch above 64 MiB each way: planes 0 and 1 run as a pair,
    plane 2 alone.  Pools, staging and skip counts against the oracle."""
    g = wl.Geometry(3, 1, 8, 128, "bf16")               # Q = 3, R = 2 KiB
    Q, R, B = g.planes, g.row_bytes, 16
    case = big_case("odd_pairs", g, [6000, 5500], B, B, 8990, 0.01)
    assert case.total_tokens * Q * R > 64 << 20
    rng = np.random.default_rng(8990)
    blk = 4 * B * R                                     # block length (page stride)
    src_h = rng.integers(0, 256, case.src.num_pages * blk, dtype=np.uint8)
    dst_h = rng.integers(0, 256, case.dst.num_pages * blk, dtype=np.uint8)
    n = case.total_tokens * Q * R
    stage_in = rng.integers(0, 256, n, dtype=np.uint8)
    lay, reqs = layout_of(g), requests(case)
    st, dt = table(case.src), table(case.dst)
    align = 128 << 10

    def pool(t, pages):
        return kvx.Pool([t.data_ptr() + q * B * R for q in range(Q)], pages, B, slot_stride=R,
                        page_stride=blk, keep=t)

    def planes(flat):
        return [flat[q * B * R:] for q in range(Q)]

    src_d = d_aligned(src_h, align)
    skipped = torch.zeros(3, dtype=torch.int64, device=DEV)
    say("odd_pairs gather")
    staging = d_aligned(np.zeros(n, np.uint8), align)
    kvx.gather(lay, pool(src_d, case.src.num_pages), st, reqs, staging, skipped=skipped[0:1])
    say("odd_pairs scatter")
    dst_d1 = d_aligned(dst_h, align)
    kvx.scatter(lay, d_aligned(stage_in, align), reqs, pool(dst_d1, case.dst.num_pages), dt,
                skipped=skipped[1:2])
    say("odd_pairs gather_scatter")
    dst_d2 = d_aligned(dst_h, align)
    kvx.gather_scatter(lay, pool(src_d, case.src.num_pages), st, reqs,
                       pool(dst_d2, case.dst.num_pages), dt, skipped=skipped[2:3])
    torch.cuda.synchronize()
    exp_stage = np.zeros(n, np.uint8)
    s0 = oracle.gather(planes(src_h), R, B, case.src.num_pages, R, case.tok_off, case.src.pg_off,
                       case.src.ids, exp_stage, page_stride=blk)
    exp_dst1 = dst_h.copy()
    s1 = oracle.scatter(stage_in, R, case.tok_off, case.dst.pg_off, case.dst.ids,
                        planes(exp_dst1), R, B, case.dst.num_pages, page_stride=blk)
    exp_dst2 = dst_h.copy()
    s2 = oracle.gather_scatter(planes(src_h), R, B, case.src.num_pages, case.src.pg_off,
                               case.src.ids, R, case.tok_off, planes(exp_dst2), R, B,
                               case.dst.num_pages, case.dst.pg_off, case.dst.ids,
                               src_page_stride=blk, dst_page_stride=blk)
    assert_bytes_equal(staging.cpu().numpy(), exp_stage, "odd_pairs gather")
    assert_bytes_equal(dst_d1.cpu().numpy(), exp_dst1, "odd_pairs scatter")
    assert_bytes_equal(dst_d2.cpu().numpy(), exp_dst2, "odd_pairs gather_scatter")
    assert skipped.cpu().tolist() == [s0, s1, s2]


def test_more_than_128_planes():
    # Q = 160 planes: the host splits the launch into plane ranges of 128
    case = wl.random_case(77, geom=wl.Geometry(80, 2, 1, 8, "bf16"), max_reqs=3, max_len=40,
                          src_page=2, dst_page=1)
    run_paged_case(case, 77)


def test_token_major_pools_and_mixed_strides():
    """Source pool token-major (plane q of slot s at (s*Q + q)*R), destination
    pool with slots padded to 3R: strides differ from R and from each other."""
    g = wl.Geometry(2, 2, 8, 128, "bf16")
    Q, R = g.planes, g.row_bytes
    case = wl.random_case(88, geom=g, max_reqs=4, max_len=60, src_page=16, dst_page=1)
    rng = np.random.default_rng(88)
    src_tm = rng.integers(0, 256, case.src.num_slots * Q * R, dtype=np.uint8)
    dst_pad = rng.integers(0, 256, (Q, case.dst.num_slots, 3 * R), dtype=np.uint8)
    src_d, dst_d = d(src_tm), d(dst_pad)
    lay, reqs = layout_of(g), requests(case)
    src = kvx.Pool([src_d.data_ptr() + q * R for q in range(Q)], case.src.num_pages,
                   case.src.page_size, slot_stride=Q * R, keep=src_d)
    dst = kvx.Pool([dst_d[q].data_ptr() for q in range(Q)], case.dst.num_pages,
                   case.dst.page_size, slot_stride=3 * R, keep=dst_d)
    say("token_major gather_scatter")
    kvx.gather_scatter(lay, src, table(case.src), reqs, dst, table(case.dst))
    torch.cuda.synchronize()
    exp = dst_pad.copy()
    oracle.gather_scatter([src_tm[q * R:] for q in range(Q)], Q * R, case.src.page_size,
                          case.src.num_pages, case.src.pg_off, case.src.ids, R, case.tok_off,
                          [exp[q].reshape(-1) for q in range(Q)], 3 * R, case.dst.page_size,
                          case.dst.num_pages, case.dst.pg_off, case.dst.ids)
    assert_bytes_equal(dst_d.cpu().numpy(), exp, "token-major gather_scatter")


# ------------------------------------------------------------------ permutes --

PERMS = [
    # (Q, H, D, dtype, s_cap, seq)
    (4, 4, 128, "f16", 300, 300),     # head rows of 256 B (the Qwen2.5-7B permute shape)
    (3, 4, 128, "f16", 300, 173),     # s_cap > seq: rebuild leaves s >= seq alone
    (2, 1, 128, "bf16", 100, 100),    # H = 1: a plain copy
    (2, 8, 64, "bf16", 64, 1),        # seq = 1
    (2, 3, 24, "bf16", 77, 50),       # head rows of 48 B
    (2, 2, 8, "f16", 500, 499),       # head rows of 16 B
    (2, 4, 512, "bf16", 40, 33),      # head rows of 1 KiB (wide copy)
    (2, 2, 1024, "bf16", 20, 20),     # head rows of 2 KiB (wide copy)
    (2, 100, 128, "f16", 10, 7),      # many heads
    (160, 2, 8, "bf16", 9, 9),        # Q > 128: plane ranges
    (2, 4, 128, "f16", 16, 0),        # seq = 0: nothing moves
    (2, 8, 128, "bf16", 100, 77),     # token rows of 2 KiB, ragged last chunk
    (2, 16, 128, "bf16", 50, 45),     # token rows of 4 KiB
    (1, 32, 128, "bf16", 9, 5),       # token rows of 8 KiB
    (2, 64, 128, "bf16", 9, 9),       # token rows of 16 KiB (one token per chunk)
    (3, 12, 128, "bf16", 40, 40),     # token rows of 3 KiB: head-row kernel
    # launches above 64 MiB each way: one token row per wave
    (72, 4, 128, "f16", 1200, 1111),  # token rows of 1 KiB (s_cap > seq; DRAM-page order
                                      # in 4 blocks of 256 tokens, the last 87 in order)
    (60, 4, 128, "bf16", 1280, 1280), # 1 KiB rows: 5 whole DRAM-page blocks
    (20, 8, 128, "bf16", 2000, 2000), # token rows of 2 KiB
    (6, 16, 128, "bf16", 3100, 2999), # token rows of 4 KiB
]


@pytest.mark.parametrize("case", PERMS, ids=lambda c: "Q{}_H{}_D{}_{}_cap{}_seq{}".format(*c))
def test_permutes(case):
    Q, H, D, dtype, s_cap, seq = case
    eb = wl.ELEM_BYTES[dtype]
    Db = D * eb
    lay = kvx.Layout(Q, 1, H, D, dtype)
    rng = np.random.default_rng(Q * 1000 + H * 10 + seq)
    hf_h = rng.integers(0, 256, (Q, H * s_cap * Db), dtype=np.uint8)
    out_guard = 64
    out_pre = rng.integers(0, 256, Q * seq * H * Db + out_guard, dtype=np.uint8)
    tgt_h = rng.integers(0, 256, (Q, H * s_cap * Db), dtype=np.uint8)
    flat_in = rng.integers(0, 256, Q * seq * H * Db, dtype=np.uint8)
    hf_d, out_d, tgt_d, flat_d = d(hf_h), d(out_pre), d(tgt_h), d(flat_in)
    out_c, tgt_c = d(out_pre), d(tgt_h)
    say(f"extract Q={Q} H={H} Db={Db} s_cap={s_cap} seq={seq}")
    kvx.extract_permute(lay, hf_d, s_cap, seq, out_d)
    say("rebuild")
    kvx.rebuild_permute(lay, flat_d, seq, tgt_d, s_cap)
    say("extract and rebuild, cached outputs")
    kvx.extract_permute(lay, hf_d, s_cap, seq, out_c, cached_out=True)
    kvx.rebuild_permute(lay, flat_d, seq, tgt_c, s_cap, cached_out=True)
    torch.cuda.synchronize()
    exp_out = out_pre.copy()
    oracle.extract_permute([hf_h[q] for q in range(Q)], H, Db, s_cap, seq, exp_out)
    exp_tgt = tgt_h.copy()
    oracle.rebuild_permute(flat_in, H, Db, seq, [exp_tgt[q] for q in range(Q)], s_cap)
    assert_bytes_equal(out_d.cpu().numpy(), exp_out, "extract")
    assert_bytes_equal(tgt_d.cpu().numpy(), exp_tgt, "rebuild")
    assert_bytes_equal(out_c.cpu().numpy(), exp_out, "extract, cached output")
    assert_bytes_equal(tgt_c.cpu().numpy(), exp_tgt, "rebuild, cached output")


def test_device_fill_matches_host_hash():
    """The generators' device fill writes SplitMix64 words, as the host does."""
    from workloads import device as wdev
    t = torch.empty(3 * 1000 * 48, dtype=torch.uint8, device=DEV)
    say("fill_hash")
    wdev.fill_hash(t, 1234567, ctr0=0)
    torch.cuda.synchronize()
    assert_bytes_equal(t.cpu().numpy(), wl.hash_fill_host(1234567, t.numel()), "fill_hash")
    w = t[:40].cpu().numpy().view("<u8")
    assert int(w[0]) == 6457827717110365317


@pytest.mark.parametrize("K,R", [(1, 2048), (2, 2048), (4, 2048), (4, 1152), (1, 48), (2, 4096)])
def test_row_pattern_moves_the_rows_it_names(K, R):
    """The measurement helper wl_row_pattern (a table-free row mover used only
    to time access patterns) touches exactly the rows its slot map names:
    random to random copies slot f(q, t) of each plane to the same slot,
    random to contiguous and contiguous to random follow the same map, and
    every other byte stays as it was."""
    from workloads import device as wdev
    Q, T, S, st = 3, 8, 32, 2
    rng = np.random.default_rng(K)
    src_h = rng.integers(0, 256, (Q, S, R), dtype=np.uint8)
    dst_h = rng.integers(0, 256, (Q, S, R), dtype=np.uint8)
    slot = [[((t + st * T) * 40503 + q * 977) % S for t in range(T)] for q in range(Q)]
    sink = torch.zeros(2048, dtype=torch.int32, device=DEV)
    for mode in (15, 7, 11):
        a, b = torch.from_numpy(src_h).to(DEV), torch.from_numpy(dst_h).to(DEV)
        say(f"row_pattern K={K} R={R} mode={mode}")
        wdev.row_pattern(a, b, sink, Q, T, S, K, st, mode, row_bytes=R)
        torch.cuda.synchronize()
        exp = dst_h.copy()
        flat_exp, flat_src = exp.reshape(-1, R), src_h.reshape(-1, R)
        for q in range(Q):
            for t in range(T):
                s_row = q * S + slot[q][t] if mode & 4 else q * T + t
                d_row = q * S + slot[q][t] if mode & 8 else q * T + t
                flat_exp[d_row] = flat_src[s_row]
        assert_bytes_equal(b.cpu().numpy(), exp, f"row_pattern mode {mode}")
        assert_bytes_equal(a.cpu().numpy(), src_h, "row_pattern source untouched")
