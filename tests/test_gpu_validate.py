"""KVX_VALIDATE=1 (debug mode) on the GPU, in a child process (the flag is
read once per process): valid calls run and match the oracle; a duplicate
destination row, a source and destination that share rows, and staging laid
over the pool it reads, a one-request batch whose tok_off breaks the
contract, a head-sliced copy whose tok_off runs past total_tokens, and a
head-sliced copy that writes a head row it reads are refused with their
status and nothing is written; out-of-range ids stay legal (skipped and
counted)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import torch
import oracle
import scatter_kvx_gather_amd as kvx
import workloads as wl

dev = torch.device("cuda:0")
d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
g = wl.Geometry(1, 2, 2, 128, "bf16")                  # Q = 2, R = 512
Q, R, S = g.planes, g.row_bytes, 64
lay = kvx.Layout(1, 2, 2, 128, "bf16")
rng = np.random.default_rng(5)
src_h = rng.integers(0, 256, (Q, S, R), dtype=np.uint8)
dst_h = rng.integers(0, 256, (Q, S, R), dtype=np.uint8)
tok = np.array([0, 20, 31], np.int64)
pg = np.array([0, 20, 31], np.int64)
sids = rng.permutation(S)[:31].astype(np.int32)
dids = rng.permutation(S)[:31].astype(np.int32)
reqs = kvx.Requests(d(tok), 31)

def expect(status, fn):
    try:
        fn()
    except kvx.KvxError as e:
        assert e.status == status, (e.status, status)
        return
    raise AssertionError(f"expected status {{status}}")

# 1. a valid gather-scatter runs and matches the oracle
A, B = d(src_h), d(dst_h)
kvx.gather_scatter(lay, kvx.Pool(A, S), kvx.Table(d(pg), d(sids)), reqs, kvx.Pool(B, S),
                   kvx.Table(d(pg), d(dids)))
torch.cuda.synchronize()
exp = dst_h.copy()
oracle.gather_scatter([src_h[q].reshape(-1) for q in range(Q)], R, 1, S, pg, sids, R, tok,
                      [exp[q].reshape(-1) for q in range(Q)], R, 1, S, pg, dids)
assert np.array_equal(B.cpu().numpy(), exp)

# 2. two tokens writing one destination row: refused, nothing written
dup = dids.copy(); dup[30] = dup[3]
before = B.clone()
expect(8, lambda: kvx.gather_scatter(lay, kvx.Pool(A, S), kvx.Table(d(pg), d(sids)), reqs,
                                     kvx.Pool(B, S), kvx.Table(d(pg), d(dup))))
torch.cuda.synchronize()
assert torch.equal(B, before)

# 3. one pool as source and destination, a written row also read: refused
shared = np.setdiff1d(np.arange(S), sids)[:31].astype(np.int32)   # rows the source leaves alone
shared[7] = sids[12]                                               # ... but one
before = A.clone()
expect(9, lambda: kvx.gather_scatter(lay, kvx.Pool(A, S), kvx.Table(d(pg), d(sids)), reqs,
                                     kvx.Pool(A, S), kvx.Table(d(pg), d(shared))))
torch.cuda.synchronize()
assert torch.equal(A, before)

# 4. staging laid over the pool a gather reads: refused
over = A.view(-1)[:31 * Q * R]
expect(9, lambda: kvx.gather(lay, kvx.Pool(A, S), kvx.Table(d(pg), d(sids)), reqs, over))
torch.cuda.synchronize()
assert torch.equal(A, before)

# 5. head-sliced copy with a duplicate destination row: refused
one = kvx.Layout(1, 2, 1, 128, "bf16")
before = B.clone()
expect(8, lambda: kvx.gather_scatter_heads(
    one, kvx.Pool(A, S, slot_stride=R), kvx.Table(d(pg), d(sids)), kvx.Heads(2, 1, "hnd"),
    reqs, kvx.Pool(B, S, slot_stride=R), kvx.Table(d(pg), d(dup)), kvx.Heads(2, 0, "nhd")))
torch.cuda.synchronize()
assert torch.equal(B, before)

# 6. an out-of-range source id is legal: that token is skipped and counted
oor = sids.copy(); oor[4] = S + 9
skipped = torch.zeros(1, dtype=torch.int64, device=dev)
kvx.gather_scatter(lay, kvx.Pool(A, S), kvx.Table(d(pg), d(oor)), reqs, kvx.Pool(B, S),
                   kvx.Table(d(pg), d(dids)), skipped)
torch.cuda.synchronize()
assert int(skipped.item()) == Q, int(skipped.item())

# 7. a one-request batch whose tok_off breaks the contract (the kernels take
#    {{0, total_tokens}} for one request without reading it): refused
one_req = kvx.Requests(d(np.array([0, 20], np.int64)), 31)
before = B.clone()
expect(2, lambda: kvx.gather_scatter(lay, kvx.Pool(A, S), kvx.Table(d(pg[[0, 2]]), d(sids)),
                                     one_req, kvx.Pool(B, S), kvx.Table(d(pg[[0, 2]]), d(dids))))
torch.cuda.synchronize()
assert torch.equal(B, before)

# 8. a head-sliced copy whose tok_off runs past total_tokens: refused before
#    the host checker indexes its per-token arrays by it
bad_end = kvx.Requests(d(np.array([0, 31 + 9], np.int64)), 31)
before = B.clone()
expect(2, lambda: kvx.gather_scatter_heads(
    one, kvx.Pool(A, S, slot_stride=R), kvx.Table(d(pg[[0, 2]]), d(sids)), kvx.Heads(2, 1, "hnd"),
    bad_end, kvx.Pool(B, S, slot_stride=R), kvx.Table(d(pg[[0, 2]]), d(dids)),
    kvx.Heads(2, 0, "nhd")))
torch.cuda.synchronize()
assert torch.equal(B, before)

# 9. a head-sliced copy inside one pool whose written head row is a head row
#    it reads (token 7 writes head 1 of page sids[12], token 12 reads it): refused
before = A.clone()
expect(9, lambda: kvx.gather_scatter_heads(
    one, kvx.Pool(A, S, slot_stride=R), kvx.Table(d(pg), d(sids)), kvx.Heads(2, 1, "hnd"),
    reqs, kvx.Pool(A, S, slot_stride=R), kvx.Table(d(pg), d(shared)), kvx.Heads(2, 1, "nhd")))
torch.cuda.synchronize()
assert torch.equal(A, before)
print("validate ok", flush=True)
"""


def test_validate_mode_refuses_broken_preconditions():
    env = dict(os.environ, KVX_VALIDATE="1")
    p = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True,
                       text=True, timeout=180, env=env, cwd=ROOT)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "validate ok" in p.stdout
    assert "KVX_VALIDATE: KVX_E_DUPLICATE" in p.stderr      # the refusals are reported
    assert "KVX_VALIDATE: KVX_E_OVERLAP" in p.stderr
    assert "KVX_VALIDATE: KVX_E_SHAPE" in p.stderr
