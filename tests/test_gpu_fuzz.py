"""Randomized GPU parity against the oracle: geometries with rows of 16 B to
4 KiB in every element size, pages drawn from {1, 2, 16, 32} on each side,
1 to 64 requests with empty ones (and 65 to 5000 in a second set), some page
ids out of range, random-bit payloads (NaN patterns included),
sentinel-filled destinations and guard bytes after the staging; token-major
pools; pools whose blocks hold several planes' pages; launches of 65-160 MiB each way with rows of 1-16 KiB; head-sliced
copies and permutes; page-table offsets that read outside their request's
list; more than 128 planes; large launches over aligned pools, where the
DRAM-page orders apply.  Every case is compared byte for byte over the whole
destination, and the skip counters must agree.  KVX_FUZZ_SCALE=k multiplies
the number of cases of each family (a longer campaign)."""
import os

import numpy as np
import pytest

import workloads as wl
from tests.test_gpu_parity import (big_case, run_paged_case, run_paged_case_blocks,
                                   run_paged_case_token_major)

pytestmark = pytest.mark.gpu

DTYPES = ["fp8", "f16", "bf16", "f32"]
SCALE = max(1, int(os.environ.get("KVX_FUZZ_SCALE", "1")))


def seeds(n):
    return range(n * SCALE)


def random_geometry(rng):
    while True:
        dt = DTYPES[int(rng.integers(len(DTYPES)))]
        H = int(rng.choice([1, 2, 3, 4, 8, 12, 16]))
        D = int(rng.choice([8, 16, 24, 64, 128]))
        g = wl.Geometry(int(rng.integers(1, 4)), int(rng.integers(1, 3)), H, D, dt)
        if g.row_bytes % 16 == 0 and 16 <= g.row_bytes <= 4096:
            return g


@pytest.mark.parametrize("seed", seeds(40))
def test_fuzz_paged_ops(seed):
    rng = np.random.default_rng(88000 + seed)
    g = random_geometry(rng)
    nreq = int(rng.integers(1, 65))
    lens = rng.integers(0, 40 if nreq > 16 else 120, size=nreq)
    lens[rng.random(nreq) < 0.15] = 0
    if lens.sum() == 0:
        lens[0] = 1
    sp, dp = (int(rng.choice([1, 2, 16, 32])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.0, 0.05]))
    case = big_case(f"fuzz{seed}", g, list(lens), sp, dp, 88000 + seed, oor)
    run_paged_case(case, 88000 + seed)


@pytest.mark.parametrize("seed", seeds(16))
def test_fuzz_paged_many_requests(seed):
    # 65 to 5000 requests: the guessed-window lookup and the 64-way search,
    # with empty requests at a random rate
    rng = np.random.default_rng(89000 + seed)
    g = random_geometry(rng)
    nreq = int(rng.integers(65, 5001))
    zf = float(rng.choice([0.0, 0.2, 0.6, 0.9]))
    lens = np.where(rng.random(nreq) < zf, 0, rng.integers(1, int(rng.integers(2, 12)), nreq))
    while lens.sum() * g.planes * g.row_bytes > (192 << 20):     # bound the host work
        lens //= 2
    if lens.sum() == 0:
        lens[0] = 1
    sp, dp = (int(rng.choice([1, 2, 16, 32])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.0, 0.05]))
    case = big_case(f"fuzzmany{seed}", g, list(lens), sp, dp, 89000 + seed, oor)
    run_paged_case(case, 89000 + seed)


@pytest.mark.parametrize("seed", seeds(24))
def test_fuzz_table_index_faults(seed):
    # page-table offsets that send lookups below 0, past the page-id array or
    # into another request's list, in random geometries, with and without
    # out-of-range ids; a third of the cases with up to 200 requests
    rng = np.random.default_rng(87000 + seed)
    g = random_geometry(rng)
    many = seed % 3 == 2
    case = wl.random_case(87000 + seed, geom=g, max_reqs=int(rng.integers(70, 200)) if many
                          else int(rng.integers(1, 9)), max_len=4 if many else 60,
                          src_page=int(rng.choice([1, 2, 3, 16])),
                          dst_page=int(rng.choice([1, 2, 3, 16])),
                          oor_frac=float(rng.choice([0.0, 0.1])), index_faults=True)
    run_paged_case(case, 87000 + seed)


@pytest.mark.parametrize("seed", seeds(8))
def test_fuzz_many_planes(seed):
    # more than 128 planes: each call runs as launches over plane ranges of
    # 128, with short and long requests (both chunk orders of a gather)
    rng = np.random.default_rng(86000 + seed)
    dt = DTYPES[int(rng.integers(len(DTYPES)))]
    elem = {"fp8": 1, "f16": 2, "bf16": 2, "f32": 4}[dt]
    H = int(rng.choice([1, 2, 4]))
    R = int(rng.choice([64, 256, 1024, 2048]))                # row bytes
    g = wl.Geometry(int(rng.integers(65, 131)), 2, H, R // (H * elem), dt)
    nreq = int(rng.choice([1, 5, 70]))
    lens = rng.integers(0, 3 if seed % 2 else 40, size=nreq)
    while lens.sum() * g.planes * R > (96 << 20):           # bound the host work
        lens //= 2
    lens[-1] = max(int(lens[-1]), 1)
    sp, dp = (int(rng.choice([1, 2, 16])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.05]))
    assert g.planes > 128 and g.row_bytes % 16 == 0
    case = big_case(f"fuzzq{seed}", g, list(lens), sp, dp, 86000 + seed, oor)
    run_paged_case(case, 86000 + seed)


@pytest.mark.parametrize("seed", seeds(16))
def test_fuzz_block_pools(seed):
    # blocks holding several planes' pages: [blocks][num_kv][B][R] per layer
    # on the source side, [blocks][planes][B][R] on the destination side
    rng = np.random.default_rng(95000 + seed)
    g = random_geometry(rng)
    nreq = int(rng.choice([1, 3, 17, 64, 65, 300]))
    lens = rng.integers(0, 60 if nreq > 16 else 200, size=nreq)
    lens[rng.random(nreq) < 0.15] = 0
    if lens.sum() == 0:
        lens[0] = 1
    sp, dp = (int(rng.choice([1, 2, 16, 32])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.0, 0.05]))
    case = big_case(f"fuzzblk{seed}", g, list(lens), sp, dp, 95000 + seed, oor)
    run_paged_case_blocks(case, 95000 + seed)


@pytest.mark.parametrize("seed", seeds(6))
def test_fuzz_large_launches(seed):
    # 65-160 MiB each way: launches that move one row per wave (two 1 KiB
    # rows, one 2 KiB row, or 2 KiB pieces of a 4-16 KiB row), 1-400
    # requests, layer-major or token-major pools
    rng = np.random.default_rng(94000 + seed)
    R = int(rng.choice([1024, 2048, 4096, 8192, 16384]))
    g = wl.Geometry(int(rng.integers(1, 5)), 2, R // 256, 128, "bf16")
    T = (int(rng.integers(65, 161)) << 20) // (g.planes * R) + 1
    nreq = int(rng.choice([1, 5, 64, 65, 400]))
    cuts = np.sort(rng.integers(0, T + 1, nreq - 1))
    lens = np.diff(np.concatenate([[0], cuts, [T]]))
    if rng.random() < 0.3:                      # empty requests; the last takes their tokens
        emptied = rng.random(nreq) < 0.2
        emptied[-1] = False
        lens[-1] += int(lens[emptied].sum())
        lens[emptied] = 0
    sp, dp = (int(rng.choice([1, 2, 16])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.0, 0.02]))
    case = big_case(f"fuzzlarge{seed}", g, list(lens), sp, dp, 94000 + seed, oor)
    assert case.total_tokens * g.planes * R > 64 << 20
    if rng.random() < 0.3:
        run_paged_case_token_major(case, 94000 + seed)
    else:
        run_paged_case(case, 94000 + seed)


@pytest.mark.parametrize("seed", seeds(4))
def test_fuzz_dram_page_order(seed):
    # 65-160 MiB each way over pools and staging aligned to 128 KiB, so that
    # the DRAM-page orders apply: pages of 16-128 rows of 1-16 KiB (rows
    # paired inside pages of 64 KiB or more, pieces of 4-16 KiB rows paired),
    # or blocks holding a layer's K and V pages together (planes paired);
    # 1-400 requests with ragged lengths, empty ones and out-of-range ids
    rng = np.random.default_rng(95000 + seed)
    R = int(rng.choice([1024, 2048, 4096, 8192, 16384]))
    g = wl.Geometry(int(rng.integers(2, 9)), 2, R // 256, 128, "bf16")
    T = (int(rng.integers(65, 161)) << 20) // (g.planes * R) + 1
    nreq = int(rng.choice([1, 5, 64, 65, 400]))
    cuts = np.sort(rng.integers(0, T + 1, nreq - 1))
    lens = np.diff(np.concatenate([[0], cuts, [T]]))
    if rng.random() < 0.3:
        emptied = rng.random(nreq) < 0.2
        emptied[-1] = False
        lens[-1] += int(lens[emptied].sum())
        lens[emptied] = 0
    sp, dp = (int(rng.choice([1, 16, 32, 64, 128])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.0, 0.02]))
    case = big_case(f"fuzzdram{seed}", g, list(lens), sp, dp, 95000 + seed, oor)
    assert case.total_tokens * g.planes * R > 64 << 20
    if rng.random() < 0.3:
        run_paged_case_blocks(case, 95000 + seed, align=128 << 10)
    else:
        run_paged_case(case, 95000 + seed, align=128 << 10)


@pytest.mark.parametrize("seed", seeds(16))
def test_fuzz_token_major_pools(seed):
    # both pools token-major (token-major chunk order), 1 to 300 requests
    rng = np.random.default_rng(93000 + seed)
    g = random_geometry(rng)
    nreq = int(rng.choice([1, 3, 17, 64, 65, 300]))
    lens = rng.integers(0, 60 if nreq > 16 else 200, size=nreq)
    lens[rng.random(nreq) < 0.15] = 0
    if lens.sum() == 0:
        lens[0] = 1
    sp, dp = (int(rng.choice([1, 2, 16, 32])) for _ in range(2))
    oor = float(rng.choice([0.0, 0.0, 0.05]))
    case = big_case(f"fuzztm{seed}", g, list(lens), sp, dp, 93000 + seed, oor)
    run_paged_case_token_major(case, 93000 + seed)


@pytest.mark.parametrize("seed", seeds(24))
def test_fuzz_head_slices(seed):
    from tests.test_gpu_heads import run_heads
    rng = np.random.default_rng(91000 + seed)
    D = int(rng.choice([8, 16, 64, 128, 256]))
    sH, dH = int(rng.integers(1, 13)), int(rng.integers(1, 13))
    nh = int(rng.integers(1, min(sH, dH) + 1))
    sh0, dh0 = int(rng.integers(0, sH - nh + 1)), int(rng.integers(0, dH - nh + 1))
    shnd, dhnd = int(rng.integers(2)), int(rng.integers(2))
    page = [int(rng.choice([1, 2, 4, 16, 32, 64])) for _ in range(2)]
    if shnd and dhnd and rng.random() < 0.5:
        page[1] = page[0]                       # the page-run kernel's case
    case = wl.random_case(91000 + seed, geom=wl.Geometry(int(rng.integers(1, 3)), 2, nh, D),
                          max_reqs=int(rng.integers(1, 9)), max_len=int(rng.integers(1, 150)),
                          src_page=page[0], dst_page=page[1],
                          oor_frac=float(rng.choice([0.0, 0.1])))
    run_heads(case, sH, dH, nh, sh0, dh0, D, shnd, dhnd, 91000 + seed)


@pytest.mark.parametrize("seed", seeds(24))
def test_fuzz_permutes(seed):
    from tests.test_gpu_parity import test_permutes
    rng = np.random.default_rng(92000 + seed)
    dt = DTYPES[int(rng.integers(len(DTYPES)))]
    eb = wl.ELEM_BYTES[dt]
    while True:
        D = int(rng.choice([8, 16, 32, 64, 128, 256]))
        if (D * eb) % 16 == 0:
            break
    H = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    seq = int(rng.integers(0, 300))
    s_cap = seq + int(rng.choice([0, 0, 1, 37]))
    Q = int(rng.choice([1, 2, 3, 7, 130]))
    if Q * H * max(s_cap, 1) * D * eb > (64 << 20):
        seq = s_cap = 8
    test_permutes((Q, H, D, dt, s_cap, seq))
