"""GPU parity of the head-sliced gather-scatter (P and D with different
tensor-parallel sizes, NHD and HND blocks) against the CPU oracle, byte for
byte over the whole destination pool."""
import numpy as np
import pytest
import torch

import oracle
import scatter_kvx_gather_amd as kvx
import workloads as wl
from tests.gpu_util import DEV, assert_bytes_equal, d, requests, say, table
from workloads import device as wdev

pytestmark = pytest.mark.gpu

# (src kv_heads, dst kv_heads, slice width, src head0, dst head0, head_dim)
SLICES = [
    (8, 4, 4, 4, 0, 128),     # P TP=1 -> D TP=2, rank 1
    (4, 8, 4, 0, 4, 128),     # P TP=2 rank 0 -> D TP=1: merge into heads 4..7
    (8, 8, 8, 0, 0, 128),     # whole row (layout conversion when layouts differ)
    (2, 8, 2, 0, 6, 64),      # P TP=4 -> D TP=1
    (4, 2, 2, 2, 0, 128),     # P TP=2 -> D TP=4
    (3, 5, 2, 1, 3, 16),      # odd head counts
    (100, 100, 100, 0, 0, 8), # more heads than one chunk holds
    (1, 1, 1, 0, 0, 512),     # one 1 KiB head
]
LAYOUTS = [(0, 0), (1, 1), (0, 1), (1, 0)]     # (src HND?, dst HND?)


def run_heads(case, sH, dH, nh, sh0, dh0, D, shnd, dhnd, seed):
    Q = case.geom.planes
    Db = D * 2
    rng = np.random.default_rng(seed)
    src_h = rng.integers(0, 256, (Q, case.src.num_slots * sH * Db), dtype=np.uint8)
    dst_h = rng.integers(0, 256, (Q, case.dst.num_slots * dH * Db), dtype=np.uint8)
    src_d, dst_d = d(src_h), d(dst_h)
    lay = kvx.Layout(case.geom.num_layers, case.geom.num_kv, nh, D, "bf16")
    src = kvx.Pool(src_d, case.src.num_pages, case.src.page_size, slot_stride=sH * Db)
    dst = kvx.Pool(dst_d, case.dst.num_pages, case.dst.page_size, slot_stride=dH * Db)
    skipped = torch.zeros(1, dtype=torch.int64, device=DEV)
    say(case.name, f"heads src(H={sH} h0={sh0} hnd={shnd}) dst(H={dH} h0={dh0} hnd={dhnd}) "
        f"nh={nh} D={D} T={case.total_tokens} pages {case.src.page_size}/{case.dst.page_size}")
    kvx.gather_scatter_heads(lay, src, table(case.src), kvx.Heads(sH, sh0, "hnd" if shnd else "nhd"),
                             requests(case), dst, table(case.dst),
                             kvx.Heads(dH, dh0, "hnd" if dhnd else "nhd"), skipped)
    torch.cuda.synchronize()
    exp = dst_h.copy()
    n = oracle.gather_scatter_heads(
        [src_h[q] for q in range(Q)], sH * Db, case.src.page_size, case.src.num_pages,
        case.src.pg_off, case.src.ids, (sH, sh0, shnd), Db, nh, case.tok_off,
        [exp[q] for q in range(Q)], dH * Db, case.dst.page_size, case.dst.num_pages,
        case.dst.pg_off, case.dst.ids, (dH, dh0, dhnd))
    assert_bytes_equal(dst_d.cpu().numpy(), exp, case.name)
    assert int(skipped.item()) == n


@pytest.mark.parametrize("li", range(len(LAYOUTS)))
@pytest.mark.parametrize("si", range(len(SLICES)))
def test_heads(si, li):
    sH, dH, nh, sh0, dh0, D = SLICES[si]
    shnd, dhnd = LAYOUTS[li]
    pages = [(16, 16), (1, 16), (16, 1), (3, 2)][(si + li) % 4]
    case = wl.random_case(7000 + 10 * si + li, geom=wl.Geometry(2, 2, nh, D), max_reqs=4,
                          max_len=90 if D <= 128 else 30, src_page=pages[0], dst_page=pages[1])
    run_heads(case, sH, dH, nh, sh0, dh0, D, shnd, dhnd, 10 * si + li)


@pytest.mark.parametrize("seed", range(4))
def test_heads_out_of_range(seed):
    sH, dH, nh, sh0, dh0, D = SLICES[seed]
    case = wl.random_case(7100 + seed, geom=wl.Geometry(1, 2, nh, D), max_reqs=5, max_len=60,
                          oor_frac=0.2)
    run_heads(case, sH, dH, nh, sh0, dh0, D, seed % 2, (seed // 2) % 2, 100 + seed)


@pytest.mark.parametrize("seed", range(8))
def test_heads_table_index_faults(seed):
    """Page-table offsets outside the page-id array or into another request's
    list, on both sides of a head-sliced copy, every layout pair."""
    sH, dH, nh, sh0, dh0, D = SLICES[seed % 6]
    case = wl.random_case(7300 + seed, geom=wl.Geometry(1, 2, nh, D), max_reqs=6, max_len=50,
                          oor_frac=0.1 if seed % 2 else 0.0, index_faults=True)
    run_heads(case, sH, dH, nh, sh0, dh0, D, seed % 2, (seed // 2) % 2, 200 + seed)


@pytest.mark.parametrize("li", range(len(LAYOUTS)))
def test_heads_offsets_at_the_ends_of_int64(li):
    """Page lists starting at the ends of the int64 range beside ordinary
    ones, on both sides of a head-sliced copy (pages of 8 tokens of 128-byte
    heads on both sides, so HND to HND takes the page-run kernel): the index
    runs past 2**63 - 1 or starts at -2**63, and those tokens are skipped,
    not wrapped."""
    i64max, i64min = (1 << 63) - 1, -(1 << 63)
    lens = [5, 20, 20, 3]
    ids = np.array([3, 0, 5, 1, 4, 2, 7, 6], np.int32)
    src = wl.Side(8, 8, np.array([0, i64max - 1, i64min, 3, 8], np.int64), ids)
    dst = wl.Side(8, 8, np.array([4, i64min + 1, i64max, 0, 8], np.int64), ids[::-1].copy())
    case = wl.PagedCase(f"heads_ends{li}", wl.Geometry(1, 2, 4, 64), wl.csr_from_lengths(lens),
                        src, dst, 0, 0, 0)
    shnd, dhnd = LAYOUTS[li]
    run_heads(case, 8, 4, 4, 4, 0, 64, shnd, dhnd, 300 + li)


# Batches beyond the 64-request window of the request lookup, with empty
# requests: (requests, fraction empty, page size, src HND?, dst HND?).  HND on
# both sides with one page size <= 64 takes the page-run kernel.
MANY_REQS = [
    (70, 0.2, 4, 1, 1), (70, 0.2, 4, 0, 1),
    (5000, 0.5, 4, 1, 1), (5000, 0.5, 4, 0, 0), (5000, 0.9, 1, 1, 1), (5000, 0.9, 1, 1, 0),
]


@pytest.mark.parametrize("mi", range(len(MANY_REQS)))
def test_heads_many_requests(mi):
    nreq, zf, B, shnd, dhnd = MANY_REQS[mi]
    rng = np.random.default_rng(5 + mi)
    lens = np.where(rng.random(nreq) < zf, 0, rng.integers(1, 12, nreq))
    lens[-1] = max(int(lens[-1]), 1)
    pages = [-(-int(n) // B) for n in lens]
    P = sum(pages) + 3
    perm_s, perm_d = rng.permutation(P), rng.permutation(P)
    offs = np.concatenate([[0], np.cumsum(pages)])
    ls = np.split(perm_s[:offs[-1]], offs[1:-1])
    ld = np.split(perm_d[:offs[-1]], offs[1:-1])
    case = wl.PagedCase(f"heads_{nreq}req", wl.Geometry(1, 2, 2, 128), wl.csr_from_lengths(lens),
                        wl.side_from_page_lists(ls, P, B), wl.side_from_page_lists(ld, P, B),
                        0, 0, 0)
    run_heads(case, 4, 2, 2, 2, 0, 128, shnd, dhnd, 5 + mi)


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
def test_hetero_tp_full_size(layout):
    """The full-size workload: P TP=1 (8 heads, page 16) -> two D ranks at
    TP=2 (4 heads each), with HND blocks (the page-run kernel) or NHD blocks
    (the row kernel on shifted plane bases).  Every plane of every rank
    compared with the oracle, one plane at a time through pinned host
    buffers; every plane also checked on the device: written heads equal
    their source heads and the rest of each destination pool is unchanged."""
    hnd = layout == "hnd"
    case = wl.hetero_tp_case()
    Q, D, B = case.geom.planes, 128, 16
    Db = D * 2
    Ps, Pd = case.src.num_pages, case.dst.num_pages
    say("hetero_tp fill")
    # int16 views of the bf16 payload: every comparison below is bitwise (the
    # hash fill holds NaN patterns, which a floating-point compare rejects)
    src = torch.empty((Q, Ps, 8, B, D) if hnd else (Q, Ps, B, 8, D), dtype=torch.int16,
                      device=DEV)
    wdev.fill_hash(src, case.value_seed)
    lay = kvx.Layout(36, 2, 4, D, "bf16")
    reqs, st, dt = requests(case), table(case.src), table(case.dst)
    # slot maps (whole pages laid out, truncated to each request's length)
    def slots(side):
        out = []
        for r in range(case.num_reqs):
            pg = side.ids[side.pg_off[r]:side.pg_off[r + 1]].astype(np.int64)
            out.append((pg[:, None] * B + np.arange(B)[None, :]).reshape(-1)[:case.lengths[r]])
        return np.concatenate(out)
    ss, ds = slots(case.src), slots(case.dst)
    for rank in range(2):
        dst = torch.empty((Q, Pd, 4, B, D) if hnd else (Q, Pd, B, 4, D), dtype=torch.int16,
                          device=DEV)
        wdev.fill_hash(dst, case.sentinel_seed + rank)
        before = dst.clone()
        skipped = torch.zeros(1, dtype=torch.int64, device=DEV)
        say(f"hetero_tp {layout} rank {rank}")
        kvx.gather_scatter_heads(lay, kvx.Pool(src, Ps, B, slot_stride=8 * Db), st,
                                 kvx.Heads(8, 4 * rank, layout), reqs,
                                 kvx.Pool(dst, Pd, B, slot_stride=4 * Db), dt,
                                 kvx.Heads(4, 0, layout), skipped)
        torch.cuda.synchronize()
        assert int(skipped.item()) == 0
        s_pg, s_row = torch.from_numpy(ss // B).to(DEV), torch.from_numpy(ss % B).to(DEV)
        d_pg, d_row = torch.from_numpy(ds // B).to(DEV), torch.from_numpy(ds % B).to(DEV)
        touched = torch.zeros((Pd, B), dtype=torch.bool, device=DEV)
        touched[d_pg, d_row] = True
        for q in range(Q):
            if hnd:
                got = dst[q][d_pg, :, d_row]                  # [tokens, 4, D]
                want = src[q][s_pg, 4 * rank:4 * rank + 4, s_row]
            else:
                got = dst[q][d_pg, d_row]
                want = src[q][s_pg, s_row, 4 * rank:4 * rank + 4]
            assert torch.equal(got, want), (rank, q)
            keep = ~touched
            dq, bq = (dst[q].permute(0, 2, 1, 3), before[q].permute(0, 2, 1, 3)) if hnd else \
                (dst[q], before[q])
            assert torch.equal(dq[keep], bq[keep])
        say(f"hetero_tp {layout} rank {rank}: oracle on all {Q} planes")
        pin_src = torch.empty(src[0].numel(), dtype=torch.int16, pin_memory=True)
        pin_exp = torch.empty(dst[0].numel(), dtype=torch.int16, pin_memory=True)
        pin_got = torch.empty(dst[0].numel(), dtype=torch.int16, pin_memory=True)
        for q in range(Q):
            pin_src.copy_(src[q].reshape(-1))
            pin_exp.copy_(before[q].reshape(-1))
            pin_got.copy_(dst[q].reshape(-1))
            exp = pin_exp.numpy().view(np.uint8)
            n = oracle.gather_scatter_heads([pin_src.numpy().view(np.uint8)], 8 * Db, B, Ps,
                                            case.src.pg_off, case.src.ids,
                                            (8, 4 * rank, int(hnd)), Db, 4, case.tok_off, [exp],
                                            4 * Db, B, Pd, case.dst.pg_off, case.dst.ids,
                                            (4, 0, int(hnd)), 16)
            assert n == 0
            assert_bytes_equal(pin_got.numpy().view(np.uint8), exp, f"rank {rank} plane {q}")
        del dst, before


# HND on both sides with one page size B <= 64: the page-run kernel (a chunk
# is B tokens x a few heads).  (B, head_dim, src heads, dst heads, slice width,
# src head0, dst head0): 1, 2, 4 and 8 vectors per lane per head, an odd slice
# width (last head of a chunk alone), more heads than one chunk holds, and
# blocks of batch tokens that straddle requests.
PAGE_RUNS = [
    (4, 128, 8, 4, 4, 4, 0),
    (8, 128, 4, 8, 3, 1, 5),
    (16, 128, 8, 4, 4, 0, 0),
    (32, 128, 2, 2, 2, 0, 0),
    (8, 64, 16, 16, 11, 5, 2),
    (64, 64, 3, 3, 1, 2, 0),
    (64, 8, 12, 9, 9, 3, 0),
    (1, 512, 4, 2, 2, 2, 0),
    (2, 512, 5, 7, 5, 0, 2),
    (8, 512, 2, 2, 1, 1, 1),
    (16, 256, 4, 4, 3, 1, 0),
]


@pytest.mark.parametrize("oor", [0.0, 0.15])
@pytest.mark.parametrize("pi", range(len(PAGE_RUNS)))
def test_heads_hnd_page_runs(pi, oor):
    B, D, sH, dH, nh, sh0, dh0 = PAGE_RUNS[pi]
    case = wl.random_case(7200 + 10 * pi + int(oor > 0), geom=wl.Geometry(2, 2, nh, D),
                          max_reqs=6, max_len=4 * B + 37, src_page=B, dst_page=B,
                          oor_frac=oor)
    run_heads(case, sH, dH, nh, sh0, dh0, D, 1, 1, 200 + pi)
