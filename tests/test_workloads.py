"""Seeded input generators: determinism and the structural properties each
workload promises (CPU only)."""
import numpy as np
import pytest

import workloads as wl


def test_splitmix64_known_answers():
    # first outputs of SplitMix64 from state 1234567 (the public test vector of
    # Vigna's splitmix64.c)
    got = wl.splitmix64(1234567, np.arange(5, dtype=np.uint64))
    assert [int(x) for x in got] == [6457827717110365317, 3203168211198807973,
                                     9817491932198370423, 4593380528125082431,
                                     16408922859458223821]


def test_hash_rows_match_dense_fill():
    Q, S, R = 3, 17, 48
    dense = wl.hash_fill_host(99, Q * S * R).reshape(Q, S, R)
    slots = np.array([16, 0, 5, 5])
    for q in range(Q):
        assert np.array_equal(wl.hash_rows_host(99, q, slots, R, S), dense[q, slots])


def test_workloads_deterministic():
    for make in (wl.qwen15b_128tok_page1, wl.kv144k_2048tok_page1, wl.kv144k_64req_page16):
        assert make().table_sha256() == make().table_sha256()
    assert wl.kv144k_2048tok_page1(0).table_sha256() != wl.kv144k_2048tok_page1(1).table_sha256()


def test_qwen15b_128tok_shape():
    c = wl.qwen15b_128tok_page1()
    assert c.geom.row_bytes == 512 and c.geom.token_bytes == 28 * 1024
    assert c.total_tokens == 128 and c.src.num_slots == 1024 == c.dst.num_slots
    assert len(set(c.src.ids)) == 128 and len(set(c.dst.ids)) == 128
    assert c.payload_bytes() == 3670016


def test_kv144k_2048tok_rotation_disjoint():
    seen_s, seen_d = set(), set()
    for k in range(16):
        c = wl.kv144k_2048tok_page1(k)
        assert c.payload_bytes() == 288 * 2 ** 20
        s, d = set(c.src.ids.tolist()), set(c.dst.ids.tolist())
        assert len(s) == len(d) == 2048
        assert not (s & seen_s) and not (d & seen_d)
        seen_s |= s
        seen_d |= d
    assert seen_s == set(range(32768))


def test_kv144k_32req_fragmented_pool():
    c = wl.kv144k_32req_fragmented()
    assert c.num_reqs == 32
    assert (c.lengths >= 1024).all() and (c.lengths <= 2048).all()
    ids = c.src.ids.astype(np.int64)
    assert len(np.unique(ids)) == ids.size            # every token has its own slot
    assert ids.min() >= 0 and ids.max() < 131072
    runs = sum(1 + np.count_nonzero(np.diff(ids[c.src.pg_off[r]:c.src.pg_off[r + 1]]) != 1)
               for r in range(c.num_reqs))
    assert c.total_tokens / runs < 1.5                  # rows are scattered, not runs


def test_churn_is_a_permutation():
    rng = np.random.default_rng(5)
    free = wl.churned_free_list(rng, 4096, cycles=500, max_alloc=300)
    assert np.array_equal(np.sort(free), np.arange(4096))


def test_kv144k_64req_page16_blocks():
    c = wl.kv144k_64req_page16()
    assert c.num_reqs == 64 and c.src.page_size == 16 and c.src.num_pages == 16384
    assert (np.diff(c.src.pg_off) == 128).all() and (np.diff(c.dst.pg_off) == 128).all()
    tails = c.lengths - 127 * 16
    assert tails.min() >= 1 and tails.max() <= 16
    assert len(np.unique(c.src.ids)) == 8192 and len(np.unique(c.dst.ids)) == 8192
    assert c.src.num_slots * c.geom.token_bytes == 36 * 2 ** 30


@pytest.mark.parametrize("seed", range(5))
def test_random_case_destinations_distinct(seed):
    c = wl.random_case(seed, oor_frac=0.0)
    assert (np.diff(c.tok_off) >= 0).all()
    d = c.dst
    assert len(np.unique(d.ids)) == d.ids.size
    for side in (c.src, d):
        pages = np.diff(side.pg_off)
        assert (pages * side.page_size >= c.lengths).all()


def test_qwen7b_permute_sizes():
    assert wl.qwen7b_permute(1024).payload_bytes() == 56 * 2 ** 20
    assert wl.qwen7b_permute(8192).payload_bytes() == 448 * 2 ** 20
