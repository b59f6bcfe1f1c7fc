"""GPU parity on the five workloads at full size, in the launch configuration
bench.py times (default grid).  Every destination byte is compared with the
oracle on host copies of the same inputs.  The 2 x 36 GiB block pools of the
last workload are compared one 512 MiB plane at a time (all 72 planes,
through pinned host buffers), and every plane is also checked on the device
for two properties that hold at any size: each written row equals its
source row, and every other row still holds its prefill."""
import numpy as np
import pytest
import torch

import oracle
import scatter_kvx_gather_amd as kvx
import workloads as wl
from tests.gpu_util import (DEV, assert_bytes_equal, d, host_planes, layout_of,
                            oracle_gather, oracle_gather_scatter, oracle_scatter, requests, say,
                            table)
from workloads import device as wdev

pytestmark = pytest.mark.gpu
NT = 16   # oracle threads (the machine's CPU share)


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def hash_pool(Q, slots, R, seed):
    t = torch.empty((Q, slots, R), dtype=torch.uint8, device=DEV)
    wdev.fill_hash(t, seed)
    return t


def check_fill_sample(pool_d, seed, rng, nrows=64):
    """Sampled rows of a device hash fill equal the host hash of the same rows."""
    Q, S, R = pool_d.shape
    for q in rng.choice(Q, 3, replace=False):
        slots = rng.choice(S, nrows, replace=False)
        got = pool_d[int(q)][torch.from_numpy(slots).to(DEV)].cpu().numpy()
        assert_bytes_equal(got, wl.hash_rows_host(seed, int(q), slots, R, S), "fill sample")


def test_qwen15b_128tok_gather_then_scatter():
    case = wl.qwen15b_128tok_page1()
    g = case.geom
    Q, R, S = g.planes, g.row_bytes, case.src.num_slots
    shape = (Q, S, g.kv_heads, g.head_dim)
    src_h = wl.uniform_f16(case.value_seed, shape).view(np.uint8).reshape(Q, S, R)
    dst_h = wl.uniform_f16(case.sentinel_seed, shape).view(np.uint8).reshape(Q, S, R)
    lay, reqs = layout_of(g), requests(case)
    src_d, dst_d = d(src_h), d(dst_h)
    staging = torch.zeros(case.total_tokens * Q * R, dtype=torch.uint8, device=DEV)
    say("qwen15b_128tok_page1 gather")
    kvx.gather(lay, kvx.Pool(src_d, S), table(case.src), reqs, staging)
    say("qwen15b_128tok_page1 scatter")
    kvx.scatter(lay, staging, reqs, kvx.Pool(dst_d, S), table(case.dst))
    torch.cuda.synchronize()
    exp_st = np.zeros(case.total_tokens * Q * R, np.uint8)
    oracle_gather(case, src_h, exp_st)
    exp_dst = dst_h.copy()
    oracle_scatter(case, exp_st, exp_dst)
    assert exp_st.nbytes == oracle.kv_bytes(128, 28, 2, 128, 2) == int(3.5 * 2 ** 20)
    assert_bytes_equal(staging.cpu().numpy(), exp_st, "qwen15b_128tok_page1 staging")
    assert_bytes_equal(dst_d.cpu().numpy(), exp_dst, "qwen15b_128tok_page1 destination pool")


def test_kv144k_2048tok_all_three_paged_ops():
    case = wl.kv144k_2048tok_page1(0)
    g = case.geom
    Q, R, S = g.planes, g.row_bytes, case.src.num_slots
    rng = np.random.default_rng(2)
    say("kv144k_2048tok_page1 fill")
    a_d = hash_pool(Q, S, R, case.value_seed)
    b_d = hash_pool(Q, S, R, case.sentinel_seed)
    c_d = hash_pool(Q, S, R, case.sentinel_seed)
    check_fill_sample(a_d, case.value_seed, rng)
    check_fill_sample(b_d, case.sentinel_seed, rng)
    b_before = b_d.cpu().numpy()
    lay, reqs = layout_of(g), requests(case)
    st, dt = table(case.src), table(case.dst)
    staging = torch.zeros(case.total_tokens * Q * R, dtype=torch.uint8, device=DEV)
    skipped = torch.zeros(3, dtype=torch.int64, device=DEV)
    say("kv144k_2048tok_page1 gather_scatter")
    kvx.gather_scatter(lay, kvx.Pool(a_d, S), st, reqs, kvx.Pool(b_d, S), dt, skipped[0:1])
    say("kv144k_2048tok_page1 gather")
    kvx.gather(lay, kvx.Pool(a_d, S), st, reqs, staging, skipped[1:2])
    say("kv144k_2048tok_page1 scatter")
    kvx.scatter(lay, staging, reqs, kvx.Pool(c_d, S), dt, skipped[2:3])
    torch.cuda.synchronize()
    assert skipped.cpu().tolist() == [0, 0, 0]
    a_h = a_d.cpu().numpy()
    exp_st = np.zeros(staging.numel(), np.uint8)
    oracle_gather(case, a_h, exp_st, NT)
    assert_bytes_equal(staging.cpu().numpy(), exp_st, "kv144k_2048tok_page1 gather")
    exp_b = b_before.copy()
    exp_c = b_before
    oracle_gather_scatter(case, a_h, exp_b, NT)
    assert_bytes_equal(b_d.cpu().numpy(), exp_b, "kv144k_2048tok_page1 gather_scatter")
    del exp_b
    oracle_scatter(case, exp_st, exp_c, NT)
    assert_bytes_equal(c_d.cpu().numpy(), exp_c, "kv144k_2048tok_page1 scatter")


def test_kv144k_2048tok_token_major_pools():
    """The 2048-token request with token-major pools (plane q of slot s at
    (s * Q + q) * R, so the rows of a slot in all planes are one 144 KiB run),
    where the paged kernels take token-major chunk order: gather-scatter
    between two such pools, gather, scatter back at another slot set, and
    gather-scatter into a layer-major pool; every destination byte against
    the oracle."""
    case, case2 = wl.kv144k_2048tok_page1(1), wl.kv144k_2048tok_page1(2)
    g = case.geom
    Q, R, S = g.planes, g.row_bytes, case.src.num_slots
    say("kv144k_2048tok_page1 token-major fill")
    a_d = torch.empty((S, Q, R), dtype=torch.uint8, device=DEV)
    b_d = torch.empty((S, Q, R), dtype=torch.uint8, device=DEV)
    c_d = hash_pool(Q, S, R, case.sentinel_seed + 1)
    wdev.fill_hash(a_d, case.value_seed)
    wdev.fill_hash(b_d, case.sentinel_seed)
    b_before = b_d.cpu().numpy().reshape(-1)
    c_before = c_d.cpu().numpy()

    def tm_pool(t):
        p = kvx.Pool([t.data_ptr() + q * R for q in range(Q)], S, 1, slot_stride=Q * R, keep=t)
        return p

    def tm_planes(flat):
        return [flat[q * R:] for q in range(Q)]

    lay, reqs = layout_of(g), requests(case)
    st, dt, dt2 = table(case.src), table(case.dst), table(case2.dst)
    staging = torch.zeros(case.total_tokens * Q * R, dtype=torch.uint8, device=DEV)
    skipped = torch.zeros(4, dtype=torch.int64, device=DEV)
    say("kv144k_2048tok_page1 token-major gather_scatter")
    kvx.gather_scatter(lay, tm_pool(a_d), st, reqs, tm_pool(b_d), dt, skipped[0:1])
    say("kv144k_2048tok_page1 token-major gather")
    kvx.gather(lay, tm_pool(a_d), st, reqs, staging, skipped[1:2])
    say("kv144k_2048tok_page1 token-major scatter")
    kvx.scatter(lay, staging, reqs, tm_pool(b_d), dt2, skipped[2:3])
    say("kv144k_2048tok_page1 token-major -> layer-major gather_scatter")
    kvx.gather_scatter(lay, tm_pool(a_d), st, reqs, kvx.Pool(c_d, S), dt, skipped[3:4])
    torch.cuda.synchronize()
    assert skipped.cpu().tolist() == [0, 0, 0, 0]
    a_h = a_d.cpu().numpy().reshape(-1)
    exp_st = np.zeros(staging.numel(), np.uint8)
    oracle.gather(tm_planes(a_h), Q * R, 1, S, R, case.tok_off, case.src.pg_off, case.src.ids,
                  exp_st, NT)
    assert_bytes_equal(staging.cpu().numpy(), exp_st, "token-major gather")
    exp_b = b_before
    oracle.gather_scatter(tm_planes(a_h), Q * R, 1, S, case.src.pg_off, case.src.ids, R,
                          case.tok_off, tm_planes(exp_b), Q * R, 1, S, case.dst.pg_off,
                          case.dst.ids, NT)
    oracle.scatter(exp_st, R, case.tok_off, case2.dst.pg_off, case2.dst.ids, tm_planes(exp_b),
                   Q * R, 1, S, NT)
    assert_bytes_equal(b_d.cpu().numpy().reshape(-1), exp_b,
                       "token-major gather_scatter, then scatter")
    del exp_b
    exp_c = c_before
    oracle.gather_scatter(tm_planes(a_h), Q * R, 1, S, case.src.pg_off, case.src.ids, R,
                          case.tok_off, host_planes(exp_c), R, 1, S, case.dst.pg_off,
                          case.dst.ids, NT)
    assert_bytes_equal(c_d.cpu().numpy(), exp_c, "token-major -> layer-major gather_scatter")


def test_kv144k_32req_fragmented_gather():
    case = wl.kv144k_32req_fragmented()
    g = case.geom
    Q, R, S = g.planes, g.row_bytes, case.src.num_slots
    say("kv144k_32req_fragmented fill", f"pool {Q * S * R / 2**30:.1f} GiB")
    a_d = hash_pool(Q, S, R, case.value_seed)
    check_fill_sample(a_d, case.value_seed, np.random.default_rng(3))
    n = case.total_tokens * Q * R
    guard = 4096
    staging = torch.empty(n + guard, dtype=torch.uint8, device=DEV)
    wdev.fill_hash(staging, case.sentinel_seed)
    exp = staging.cpu().numpy()
    say("kv144k_32req_fragmented gather", f"{case.num_reqs} requests, {case.total_tokens} tokens")
    kvx.gather(layout_of(g), kvx.Pool(a_d, S), table(case.src), requests(case), staging)
    torch.cuda.synchronize()
    a_h = a_d.cpu().numpy()
    del a_d
    oracle_gather(case, a_h, exp, NT)
    del a_h
    assert_bytes_equal(staging.cpu().numpy(), exp, "kv144k_32req_fragmented staging")


@pytest.mark.parametrize("seq", [1024, 8192])
def test_qwen7b_extract_rebuild(seq):
    case = wl.qwen7b_permute(seq)
    g = case.geom
    Q, H, Dm = g.planes, g.kv_heads, g.head_dim
    Db = g.head_bytes
    lay = layout_of(g)
    hf_h = wl.normal_f16(case.value_seed, (Q, 1, H, seq, Dm))
    tgt_h = wl.normal_f16(case.sentinel_seed, (Q, 1, H, seq, Dm))
    hf_d, tgt_d = d(hf_h), d(tgt_h)
    out_d = torch.empty((Q, seq, H, Dm), dtype=torch.float16, device=DEV)
    say(f"qwen7b_permute seq={seq} extract")
    kvx.extract_permute(lay, hf_d, seq, seq, out_d)
    say(f"qwen7b_permute seq={seq} rebuild")
    kvx.rebuild_permute(lay, out_d, seq, tgt_d, seq)
    torch.cuda.synchronize()
    hf_b = hf_h.view(np.uint8).reshape(Q, -1)
    exp_out = np.zeros(Q * seq * H * Db, np.uint8)
    oracle.extract_permute([hf_b[q] for q in range(Q)], H, Db, seq, seq, exp_out, NT)
    assert_bytes_equal(out_d.cpu().numpy().view(np.uint8).reshape(-1), exp_out, "extract")
    exp_tgt = tgt_h.view(np.uint8).reshape(Q, -1).copy()
    oracle.rebuild_permute(exp_out, H, Db, seq, [exp_tgt[q] for q in range(Q)], seq, NT)
    got_tgt = tgt_d.cpu().numpy()
    assert_bytes_equal(got_tgt.view(np.uint8).reshape(Q, -1), exp_tgt, "rebuild")
    # round trip: rebuild(extract(x)) == x
    assert_bytes_equal(got_tgt.view(np.uint8), hf_h.view(np.uint8), "round trip")


def test_kv144k_64req_page16_block_pools():
    case = wl.kv144k_64req_page16()
    g = case.geom
    Q, R = g.planes, g.row_bytes
    S = case.src.num_slots
    plane_bytes = S * R
    say("kv144k_64req_page16 fill", f"2 x {Q * plane_bytes / 2**30:.0f} GiB")
    a_d = hash_pool(Q, S, R, case.value_seed)
    b_d = hash_pool(Q, S, R, case.sentinel_seed)
    check_fill_sample(a_d, case.value_seed, np.random.default_rng(5))
    skipped = torch.zeros(1, dtype=torch.int64, device=DEV)
    say("kv144k_64req_page16 gather_scatter", f"{case.num_reqs} requests, {case.total_tokens} tokens")
    kvx.gather_scatter(layout_of(g), kvx.Pool(a_d, case.src.num_pages, 16), table(case.src),
                       requests(case), kvx.Pool(b_d, case.dst.num_pages, 16), table(case.dst),
                       skipped)
    torch.cuda.synchronize()
    assert int(skipped.item()) == 0

    # slot maps (whole pages laid out, then each request truncated to its length)
    def slots(side):
        out = []
        for r in range(case.num_reqs):
            pages = side.ids[side.pg_off[r]:side.pg_off[r + 1]].astype(np.int64)
            full = (pages[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
            out.append(full[:case.lengths[r]])
        return np.concatenate(out)
    src_slots, dst_slots = slots(case.src), slots(case.dst)
    untouched = np.ones(S, bool)
    untouched[dst_slots] = False
    src_idx, dst_idx = d(src_slots), d(dst_slots)
    keep_idx = d(np.flatnonzero(untouched))
    scratch = torch.empty((S, R), dtype=torch.uint8, device=DEV)

    # every plane, on the device: written rows equal their source rows, all
    # other rows equal the regenerated prefill
    say("kv144k_64req_page16 device-side checks")
    for q in range(Q):
        wdev.fill_hash(scratch, case.sentinel_seed, ctr0=q * plane_bytes // 8)
        assert torch.equal(b_d[q].index_select(0, dst_idx), a_d[q].index_select(0, src_idx)), q
        assert torch.equal(b_d[q].index_select(0, keep_idx), scratch.index_select(0, keep_idx)), q

    # every plane with the oracle, one plane at a time: host copies of the
    # source plane and of the regenerated prefill, the oracle's gather-scatter
    # into the latter, and the whole destination plane compared
    say(f"kv144k_64req_page16 oracle on all {Q} planes")
    pin_src = torch.empty((S, R), dtype=torch.uint8, pin_memory=True)
    pin_exp = torch.empty((S, R), dtype=torch.uint8, pin_memory=True)
    pin_got = torch.empty((S, R), dtype=torch.uint8, pin_memory=True)
    one = wl.PagedCase(case.name, wl.Geometry(1, 1, g.kv_heads, g.head_dim, g.dtype),
                       case.tok_off, case.src, case.dst, 0, 0, 0)
    for q in range(Q):
        wdev.fill_hash(scratch, case.sentinel_seed, ctr0=q * plane_bytes // 8)
        pin_src.copy_(a_d[q])
        pin_exp.copy_(scratch)
        pin_got.copy_(b_d[q])
        exp = pin_exp.numpy().reshape(1, S, R)
        assert oracle_gather_scatter(one, pin_src.numpy().reshape(1, S, R), exp, NT) == 0
        assert_bytes_equal(pin_got.numpy(), exp[0], f"kv144k_64req_page16 plane {q}")


@pytest.mark.parametrize("page", [1, 16])
def test_mla_single_plane_pools(page):
    """Single-plane MLA pools (27 planes of 1152-byte rows): gather,
    gather-scatter and scatter of a 2048-token request, whole destinations
    compared with the oracle."""
    case = wl.mla_case(page)
    g = case.geom
    Q, R, S = g.planes, g.row_bytes, case.src.num_slots
    say(f"mla page {page} fill")
    a_d = hash_pool(Q, S, R, case.value_seed)
    b_d = hash_pool(Q, S, R, case.sentinel_seed)
    b_before = b_d.cpu().numpy()
    lay, reqs = layout_of(g), requests(case)
    st, dt = table(case.src), table(case.dst)
    staging = torch.zeros(case.total_tokens * Q * R, dtype=torch.uint8, device=DEV)
    c_d = b_d.clone()
    say(f"mla page {page} gather_scatter / gather / scatter")
    kvx.gather_scatter(lay, kvx.Pool(a_d, case.src.num_pages, page), st, reqs,
                       kvx.Pool(b_d, case.dst.num_pages, page), dt)
    kvx.gather(lay, kvx.Pool(a_d, case.src.num_pages, page), st, reqs, staging)
    kvx.scatter(lay, staging, reqs, kvx.Pool(c_d, case.dst.num_pages, page), dt)
    torch.cuda.synchronize()
    a_h = a_d.cpu().numpy()
    exp_st = np.zeros(staging.numel(), np.uint8)
    oracle_gather(case, a_h, exp_st, NT)
    assert exp_st.nbytes == oracle.kv_bytes(2048, 27, 1, 576, 2, num_kv=1)
    assert_bytes_equal(staging.cpu().numpy(), exp_st, "mla gather")
    exp_b = b_before.copy()
    oracle_gather_scatter(case, a_h, exp_b, NT)
    assert_bytes_equal(b_d.cpu().numpy(), exp_b, "mla gather_scatter")
    oracle_scatter(case, exp_st, b_before, NT)
    assert_bytes_equal(c_d.cpu().numpy(), b_before, "mla scatter")
