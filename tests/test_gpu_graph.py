"""kvx calls captured in a HIP graph: every replay, with eager work between
replays, gives the oracle's bytes.  (The calls record only kernel launches --
no memset or copy nodes -- so capture is safe.)"""
import numpy as np
import pytest
import torch

import oracle
import scatter_kvx_gather_amd as kvx
import workloads as wl
from tests.gpu_util import (DEV, assert_bytes_equal, d, layout_of, oracle_gather,
                            oracle_gather_scatter, oracle_scatter, requests, say, table)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cached", [False, True])
def test_graph_replays_match_oracle(cached):
    g = wl.Geometry(2, 2, 8, 128, "bf16")
    case = wl.random_case(4242, geom=g, max_reqs=5, max_len=120, src_page=16, dst_page=1,
                          oor_frac=0.05)
    Q, R = g.planes, g.row_bytes
    rng = np.random.default_rng(42)
    src_h = rng.integers(0, 256, (Q, case.src.num_slots, R), dtype=np.uint8)
    dst_h = rng.integers(0, 256, (Q, case.dst.num_slots, R), dtype=np.uint8)
    n = case.total_tokens * Q * R
    st_h = rng.integers(0, 256, n, dtype=np.uint8)
    H, Dm, seq = g.kv_heads, g.head_dim, 40
    hf_h = rng.integers(0, 256, (Q, H * seq * Dm * 2), dtype=np.uint8)
    flat_h = rng.integers(0, 256, Q * seq * R, dtype=np.uint8)

    src_d = d(src_h)
    dst1, dst2, stage, flat, hf = d(dst_h), d(dst_h), d(st_h), d(flat_h), d(hf_h)
    keep = {k: v.clone() for k, v in dict(dst1=dst1, dst2=dst2, stage=stage, flat=flat,
                                          hf=hf).items()}
    skipped = torch.zeros(2, dtype=torch.int64, device=DEV)
    lay, reqs, st, dt = layout_of(g), requests(case), table(case.src), table(case.dst)
    P_src = kvx.Pool(src_d, case.src.num_pages, case.src.page_size)
    P_d1 = kvx.Pool(dst1, case.dst.num_pages, case.dst.page_size)
    P_d2 = kvx.Pool(dst2, case.dst.num_pages, case.dst.page_size)

    def calls():        # both store policies of the contiguous outputs
        kvx.gather(lay, P_src, st, reqs, stage, skipped[0:1], cached_out=cached)
        kvx.scatter(lay, stage, reqs, P_d1, dt, skipped[1:2])
        kvx.gather_scatter(lay, P_src, st, reqs, P_d2, dt)
        kvx.extract_permute(lay, hf, seq, seq, flat, cached_out=cached)
        kvx.rebuild_permute(lay, flat, seq, hf, seq, cached_out=cached)

    # expected bytes of one pass from the prefills
    exp_st = st_h.copy()
    s0 = oracle_gather(case, src_h, exp_st)
    exp_d1 = dst_h.copy()
    s1 = oracle_scatter(case, exp_st, exp_d1)
    exp_d2 = dst_h.copy()
    oracle_gather_scatter(case, src_h, exp_d2)
    exp_flat = np.zeros_like(flat_h)
    oracle.extract_permute([hf_h[q] for q in range(Q)], H, Dm * 2, seq, seq, exp_flat)
    exp_hf = hf_h.copy()
    oracle.rebuild_permute(exp_flat, H, Dm * 2, seq, [exp_hf[q] for q in range(Q)], seq)

    say("graph capture")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: restore the prefills, clear the counter,
        # run an unrelated eager kvx call
        for k, v in keep.items():
            dict(dst1=dst1, dst2=dst2, stage=stage, flat=flat, hf=hf)[k].copy_(v)
        skipped.zero_()
        kvx.gather(lay, P_src, st, reqs, torch.empty_like(stage))
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert_bytes_equal(stage.cpu().numpy(), exp_st, f"replay {rep} gather")
        assert_bytes_equal(dst1.cpu().numpy(), exp_d1, f"replay {rep} scatter")
        assert_bytes_equal(dst2.cpu().numpy(), exp_d2, f"replay {rep} gather_scatter")
        assert_bytes_equal(flat.cpu().numpy(), exp_flat, f"replay {rep} extract")
        assert_bytes_equal(hf.cpu().numpy(), exp_hf, f"replay {rep} rebuild")
        assert skipped.cpu().tolist() == [s0, s1], rep


def test_graph_replays_full_size_request():
    """The 2048-token, 144 KiB/token request (the one-row-per-wave launches):
    gather-scatter, gather, extract and rebuild captured once and replayed on
    four disjoint requests; every replay's bytes equal the eager calls'."""
    cs = [wl.kv144k_2048tok_page1(k) for k in range(4)]
    g = cs[0].geom
    Q, R, T = g.planes, g.row_bytes, 2048
    from workloads import device as wdev
    A = torch.empty((Q, 32768, R), dtype=torch.uint8, device=DEV)
    wdev.fill_hash(A, cs[0].value_seed)
    B0 = torch.empty_like(A)
    wdev.fill_hash(B0, cs[0].sentinel_seed)
    lay, reqs = layout_of(g), requests(cs[0])
    PA = kvx.Pool(A, 32768)
    H, Db = g.kv_heads, g.head_bytes

    tabs = [(table(c.src), table(c.dst)) for c in cs]   # uploaded before any capture

    def run(k, B, st, hf, fl):
        PB = kvx.Pool(B, 32768)
        kvx.gather_scatter(lay, PA, tabs[k][0], reqs, PB, tabs[k][1])
        kvx.gather(lay, PA, tabs[k][0], reqs, st)
        kvx.rebuild_permute(lay, st, T, hf, T)
        kvx.extract_permute(lay, hf, T, T, fl)

    def buffers():
        return (B0.clone(), torch.empty(T * Q * R, dtype=torch.uint8, device=DEV),
                torch.zeros((Q, H * T * Db), dtype=torch.uint8, device=DEV),
                torch.zeros(T * Q * R, dtype=torch.uint8, device=DEV))

    eager = []
    for k in range(4):
        bufs = buffers()
        say(f"eager request {k}")
        run(k, *bufs)
        torch.cuda.synchronize()
        eager.append(bufs)
    # one graph per request (tables are captured by address), replayed twice
    for k in range(4):
        bufs = buffers()
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        say(f"capture request {k}")
        with torch.cuda.graph(graph, stream=stream):
            run(k, *bufs)
        for rep in range(2):
            say(f"replay request {k} #{rep}")
            graph.replay()
            torch.cuda.synchronize()
            for got, want in zip(bufs, eager[k]):
                assert torch.equal(got, want), (k, rep)
        del graph
