"""The library from several host threads at once: each thread drives its own
stream, pools and tables through gather-scatter, gather and scatter calls
(the ctypes calls release the interpreter lock, so the library is entered
concurrently); every result equals the oracle's.  The calls keep no state
between them, so concurrent callers cannot disturb each other."""
import threading

import numpy as np
import pytest
import torch

import scatter_kvx_gather_amd as kvx
import workloads as wl
from tests.gpu_util import (DEV, assert_bytes_equal, d, layout_of, oracle_gather,
                            oracle_gather_scatter, requests, table)

pytestmark = pytest.mark.gpu


def test_concurrent_callers():
    nthreads, rounds = 4, 25
    jobs = []
    for w in range(nthreads):
        g = wl.Geometry(2, 2, [8, 4, 2, 3][w], 128, "bf16")
        case = wl.random_case(6600 + w, geom=g, max_reqs=6, max_len=90,
                              src_page=[1, 16, 3, 1][w], dst_page=[16, 1, 2, 1][w])
        rng = np.random.default_rng(w)
        Q, R = g.planes, g.row_bytes
        src_h = rng.integers(0, 256, (Q, case.src.num_slots, R), dtype=np.uint8)
        dst_h = rng.integers(0, 256, (Q, case.dst.num_slots, R), dtype=np.uint8)
        jobs.append((g, case, src_h, dst_h))
    results, errors = [None] * nthreads, []

    def worker(w):
        try:
            g, case, src_h, dst_h = jobs[w]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                src, dst = d(src_h), d(dst_h)
                st = torch.zeros(case.total_tokens * g.token_bytes, dtype=torch.uint8,
                                 device=DEV)
                lay, reqs = layout_of(g), requests(case)
                ts, td = table(case.src), table(case.dst)
                ps = kvx.Pool(src, case.src.num_pages, case.src.page_size)
                pd = kvx.Pool(dst, case.dst.num_pages, case.dst.page_size)
                for _ in range(rounds):             # idempotent: the same bytes every round
                    kvx.gather_scatter(lay, ps, ts, reqs, pd, td, stream=stream)
                    kvx.gather(lay, ps, ts, reqs, st, stream=stream)
                stream.synchronize()
                results[w] = (dst.cpu().numpy(), st.cpu().numpy())
        except Exception as e:                     # reported by the main thread
            errors.append((w, e))

    threads = [threading.Thread(target=worker, args=(w,)) for w in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for w in range(nthreads):
        g, case, src_h, dst_h = jobs[w]
        exp_dst = dst_h.copy()
        oracle_gather_scatter(case, src_h, exp_dst)
        exp_st = np.zeros(case.total_tokens * g.token_bytes, np.uint8)
        oracle_gather(case, src_h, exp_st)
        assert_bytes_equal(results[w][0], exp_dst, f"thread {w} gather_scatter")
        assert_bytes_equal(results[w][1], exp_st, f"thread {w} gather")
