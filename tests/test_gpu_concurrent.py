"""The transfer under load: gather-scatter of 144 KiB/token requests on one
stream while a decode-like HBM reader streams a 4 GiB buffer on a second
stream at the same priority (DistServe's pitfall: a transfer measured alone
says nothing about the transfer beside decode).  The reader only loads; the
destination pool is compared byte for byte with the oracle afterwards, and
the events show the two streams' work overlapping in time."""
import numpy as np
import pytest
import torch

import scatter_kvx_gather_amd as kvx
import workloads as wl
from tests.gpu_util import DEV, assert_bytes_equal, layout_of, oracle_gather_scatter, say, table
from workloads import device as wdev

pytestmark = pytest.mark.gpu

_STREAMS = []


def streams():
    """The transfer's and the reader's streams, created once per process and
    one right after the other (default priority), so that they sit on two
    different hardware queues: two streams that share a hardware queue run
    their work one after the other."""
    if not _STREAMS:
        _STREAMS.extend([torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)])
    return _STREAMS


@pytest.mark.parametrize("reader_blocks", [2048, 256])
def test_gather_scatter_beside_a_reader(reader_blocks):
    g = wl.KV144K
    Q, R, S, T, NREQ = g.planes, g.row_bytes, 8192, 1024, 4
    rng = np.random.default_rng(77 + reader_blocks)
    pa, pb = rng.permutation(S), rng.permutation(S)
    cases = [wl.PagedCase(f"beside_reader_{k}", g, wl.csr_from_lengths([T]),
                          wl.side_from_slot_lists([pa[k * T:(k + 1) * T]], S),
                          wl.side_from_slot_lists([pb[k * T:(k + 1) * T]], S), 0, 0, 0)
              for k in range(NREQ)]
    t_stream, r_stream = streams()
    say(f"beside reader ({reader_blocks} workgroups): fill")
    with torch.cuda.stream(t_stream):
        a_d = torch.empty((Q, S, R), dtype=torch.uint8, device=DEV)
        b_d = torch.empty((Q, S, R), dtype=torch.uint8, device=DEV)
        rd = torch.empty(4 * 2 ** 30, dtype=torch.uint8, device=DEV)
    wdev.fill_hash(a_d, 31, stream=t_stream)
    wdev.fill_hash(b_d, 32, stream=t_stream)
    wdev.fill_hash(rd, 33, stream=t_stream)
    sink = torch.zeros(2048, dtype=torch.int64, device=DEV)
    torch.cuda.synchronize()
    b_before = b_d.cpu().numpy()
    lay = layout_of(g)
    reqs = kvx.Requests(torch.tensor([0, T], dtype=torch.int64, device=DEV), T)
    tabs = [(table(c.src), table(c.dst)) for c in cases]
    skipped = torch.zeros(1, dtype=torch.int64, device=DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    say(f"beside reader ({reader_blocks} workgroups): reader and gather-scatter launches")
    ev[0].record(r_stream)
    for _ in range(6):
        wdev.read_stream(rd, sink, blocks=reader_blocks, stream=r_stream)
    ev[1].record(r_stream)
    ev[2].record(t_stream)
    for k in range(NREQ):
        kvx.gather_scatter(lay, kvx.Pool(a_d, S), tabs[k][0], reqs, kvx.Pool(b_d, S), tabs[k][1],
                           skipped, stream=t_stream)
    ev[3].record(t_stream)
    torch.cuda.synchronize()
    assert int(skipped.item()) == 0
    # the reader's launches end after the transfer's start: the two ran together
    reader_start_to_transfer_start = ev[0].elapsed_time(ev[2])
    reader_start_to_reader_end = ev[0].elapsed_time(ev[1])
    say(f"reader {reader_start_to_reader_end:.2f} ms, transfer started at "
        f"{reader_start_to_transfer_start:.2f} ms, took {ev[2].elapsed_time(ev[3]):.2f} ms")
    assert reader_start_to_transfer_start < reader_start_to_reader_end
    a_h = a_d.cpu().numpy()
    exp = b_before
    for c in cases:
        assert oracle_gather_scatter(c, a_h, exp, 16) == 0
    assert_bytes_equal(b_d.cpu().numpy(), exp, f"gather-scatter beside a reader ({reader_blocks})")
