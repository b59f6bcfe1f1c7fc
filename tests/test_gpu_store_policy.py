"""The store policy of contiguous outputs reaches the kernel choice: with
KVX_LOG=1 (read once per process, so in a child) every gather, extract and
rebuild launch reports nontemporal stores by default and cached stores with
KVX_OUT_CACHED, scatter and gather-scatter always nontemporal; both policies
write the same bytes.  A gather takes token-major chunk order exactly when
its requests average at most 64 KiB of rows per plane, and launches too
small to give every compute unit an 8 KiB chunk take smaller chunks."""
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
import scatter_kvx_gather_amd as kvx

dev = torch.device("cuda:0")
d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
rng = np.random.default_rng(3)
for (L, H, Db, T, nreq) in [(2, 8, 128, 300, 3), (1, 16, 256, 5000, 70), (1, 3, 48, 90, 2)]:
    lay = kvx.Layout(L, 2, H, Db // 2, "bf16")
    Q, R, S = 2 * L, H * Db, T + 17
    tok = np.linspace(0, T, nreq + 1).astype(np.int64)
    reqs = kvx.Requests(d(tok), T)
    ids = rng.permutation(S)[:T].astype(np.int32)
    A = d(rng.integers(0, 256, (Q, S, R), dtype=np.uint8))
    B = d(rng.integers(0, 256, (Q, S, R), dtype=np.uint8))
    tab = kvx.Table(d(tok), d(ids))
    outs = []
    for cached in (False, True):
        st = torch.zeros(Q * T * R, dtype=torch.uint8, device=dev)
        hf = torch.zeros((Q, H * T * Db), dtype=torch.uint8, device=dev)
        fl = torch.zeros_like(st)
        print(f"case L={{L}} H={{H}} Db={{Db}} T={{T}} cached={{cached}}", file=sys.stderr, flush=True)
        kvx.gather(lay, kvx.Pool(A, S), tab, reqs, st, cached_out=cached)
        kvx.rebuild_permute(lay, st, T, hf, T, cached_out=cached)
        kvx.extract_permute(lay, hf, T, T, fl, cached_out=cached)
        kvx.scatter(lay, fl, reqs, kvx.Pool(B, S), tab)
        torch.cuda.synchronize()
        outs.append((st.clone(), hf.clone(), fl.clone()))
    assert all(torch.equal(a, b) for a, b in zip(*outs))
    assert torch.equal(outs[0][0], outs[0][2])      # extract of rebuild is the staging
# chunk order of a gather: token-major when its requests average at most
# 64 KiB of rows per plane, plane-major otherwise
lay = kvx.Layout(2, 2, 8, 64, "bf16")                        # Q = 4, R = 1 KiB
A = d(rng.integers(0, 256, (4, 4096, 1024), dtype=np.uint8))
for nreq, T in ((64, 4096), (63, 4096)):                     # 64 KiB, then just above
    tok = np.linspace(0, T, nreq + 1).astype(np.int64)
    st = torch.zeros(4 * T * 1024, dtype=torch.uint8, device=dev)
    print(f"order case nreq={{nreq}} T={{T}}", file=sys.stderr, flush=True)
    kvx.gather(lay, kvx.Pool(A, 4096), kvx.Table(d(tok), d(np.arange(T, dtype=np.int32))),
               kvx.Requests(d(tok), T), st)
tok = np.array([0, 4096], np.int64)                          # one request: plane-major
print("order case nreq=1 T=4096", file=sys.stderr, flush=True)
kvx.gather(lay, kvx.Pool(A, 4096), kvx.Table(d(tok), d(np.arange(4096, dtype=np.int32))),
           kvx.Requests(d(tok), 4096), torch.zeros(4 * 4096 * 1024, dtype=torch.uint8, device=dev))
nreq, T = 16, 4096                                           # 256 tokens = 256 KiB: plane-major
tok = np.linspace(0, T, nreq + 1).astype(np.int64)
print(f"order case nreq={{nreq}} T={{T}}", file=sys.stderr, flush=True)
kvx.gather(lay, kvx.Pool(A, 4096), kvx.Table(d(tok), d(np.arange(T, dtype=np.int32))),
           kvx.Requests(d(tok), T), torch.zeros(4 * T * 1024, dtype=torch.uint8, device=dev))
torch.cuda.synchronize()
print("store policy ok", flush=True)
"""


def test_store_policy_reaches_the_kernels():
    env = dict(os.environ, KVX_LOG="1")
    p = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True,
                       text=True, timeout=180, env=env, cwd=ROOT)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "store policy ok" in p.stdout
    policy = {}
    case = None
    for line in p.stderr.splitlines():
        if line.startswith("case "):
            case = line.split("cached=")[1]
        elif line.startswith("order case "):
            case = None
        elif case is not None and line.startswith("kvx: ") and "stores=" in line:
            op = line.split()[1]
            policy.setdefault((op, case), set()).add(line.rsplit("stores=", 1)[1].strip())
    for op in ("gather", "rebuild", "extract"):
        assert policy[(op, "False")] == {"nontemporal"}, (op, policy)
        assert policy[(op, "True")] == {"cached"}, (op, policy)
    assert policy[("scatter", "False")] == policy[("scatter", "True")] == {"nontemporal"}
    order = {}
    case = None
    for line in p.stderr.splitlines():
        if line.startswith("order case "):
            case = line[len("order case "):]
        elif case and line.startswith("kvx: gather") and "order=" in line:
            order[case] = line.split("order=")[1].split()[0]
    assert order == {"nreq=64 T=4096": "token-major", "nreq=63 T=4096": "plane-major",
                     "nreq=1 T=4096": "plane-major", "nreq=16 T=4096": "plane-major"}, order


SMALL_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import torch
import scatter_kvx_gather_amd as kvx

dev = torch.device("cuda:0")
d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
print("cus", torch.cuda.get_device_properties(0).multi_processor_count, flush=True)
# paged: 16 tokens of 512-byte rows in 56 planes (8 KiB chunks would give 56)
lay = kvx.Layout(28, 2, 2, 128, "f16")
A = torch.zeros((56, 64, 512), dtype=torch.uint8, device=dev)
tok = d(np.array([0, 16], np.int64))
st = torch.zeros(16 * 56 * 512, dtype=torch.uint8, device=dev)
print("case paged", file=sys.stderr, flush=True)
kvx.gather(lay, kvx.Pool(A, 64), kvx.Table(tok, d(np.arange(16, dtype=np.int32))),
           kvx.Requests(tok, 16), st)
# permute: 16 tokens of 1 KiB token rows in 56 planes
lay = kvx.Layout(28, 2, 4, 128, "f16")
hf = torch.zeros((56, 4 * 16 * 256), dtype=torch.uint8, device=dev)
print("case permute", file=sys.stderr, flush=True)
kvx.extract_permute(lay, hf, 16, 16, torch.zeros(56 * 16 * 1024, dtype=torch.uint8, device=dev))
# head-sliced: 8 tokens, heads 4..7 of 8 into 0..3 of 4, HND -> NHD, page 16
lay = kvx.Layout(36, 2, 4, 128, "bf16")
src = torch.zeros((72, 4 * 16 * 8 * 256), dtype=torch.uint8, device=dev)
dst = torch.zeros((72, 4 * 16 * 4 * 256), dtype=torch.uint8, device=dev)
tok = d(np.array([0, 8], np.int64))
pg = d(np.array([0, 1], np.int64))
print("case heads", file=sys.stderr, flush=True)
kvx.gather_scatter_heads(lay, kvx.Pool(src, 4, 16, slot_stride=8 * 256), kvx.Table(pg, d(np.array([2], np.int32))),
                         kvx.Heads(8, 4, "hnd"), kvx.Requests(tok, 8),
                         kvx.Pool(dst, 4, 16, slot_stride=4 * 256), kvx.Table(pg, d(np.array([1], np.int32))),
                         kvx.Heads(4, 0, "nhd"))
torch.cuda.synchronize()
print("small ok", flush=True)
"""


def test_small_launches_fill_the_compute_units():
    """A launch too small to give every compute unit an 8 KiB chunk takes
    smaller chunks: with KVX_LOG=1 a 16-token paged gather of 512-byte rows
    and an 8-token head-sliced copy report at least one chunk per compute
    unit, and a 16-token extract of 1 KiB token rows one row per chunk."""
    env = dict(os.environ, KVX_LOG="1")
    p = subprocess.run([sys.executable, "-c", SMALL_CHILD.format(root=ROOT)], capture_output=True,
                       text=True, timeout=180, env=env, cwd=ROOT)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "small ok" in p.stdout
    cus = int(p.stdout.split("cus", 1)[1].split()[0])
    seen = {}
    case = None
    for line in p.stderr.splitlines():
        if line.startswith("case "):
            case = line.split()[1]
        elif case and line.startswith("kvx: "):
            f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
            seen[case] = f
    assert int(seen["paged"]["chunks"]) >= cus, seen["paged"]
    assert int(seen["heads"]["chunks"]) >= cus, seen["heads"]
    assert seen["permute"]["unit"] == "token-row" and seen["permute"]["U"] == "1", seen["permute"]


DRAM_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import torch
import scatter_kvx_gather_amd as kvx

dev = torch.device("cuda:0")
d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
rng = np.random.default_rng(5)


def pool(Q, S, R, off):
    buf = torch.zeros(Q * S * R + (256 << 10), dtype=torch.uint8, device=dev)
    o = (-buf.data_ptr()) % (128 << 10) + off
    return buf[o:o + Q * S * R].view(Q, S, R)


def paged(L, H, B, T, off, op):
    lay = kvx.Layout(L, 2, H, 128, "bf16")                  # R = H * 256 bytes
    Q, R, P = 2 * L, H * 256, T // B + 4
    tok, pg = d(np.array([0, T], np.int64)), d(np.array([0, T // B], np.int64))
    reqs = kvx.Requests(tok, T)
    A, Bp = pool(Q, P * B, R, off), pool(Q, P * B, R, off)
    ta = kvx.Table(pg, d(rng.permutation(P)[:T // B].astype(np.int32)))
    tb = kvx.Table(pg, d(rng.permutation(P)[:T // B].astype(np.int32)))
    if op == "gather":
        st = torch.zeros(Q * T * R + (256 << 10), dtype=torch.uint8, device=dev)
        o = (-st.data_ptr()) % (128 << 10) + off
        st = st[o:o + Q * T * R]
        kvx.gather(lay, kvx.Pool(A, P, B), ta, reqs, st)
    else:
        kvx.gather_scatter(lay, kvx.Pool(A, P, B), ta, reqs, kvx.Pool(Bp, P, B), tb)
    torch.cuda.synchronize()


def kvblocks(L, B, T, op):
    lay = kvx.Layout(L, 2, 8, 128, "bf16")                  # R = 2 KiB
    Q, R, P = 2 * L, 2048, T // B + 4
    run = B * R

    def kvpool():
        t = pool(1, L * P * 2 * B, R, 0).reshape(-1)        # [L][P][2][B][R], aligned
        return kvx.Pool([t.data_ptr() + (q // 2) * P * 2 * run + (q % 2) * run
                         for q in range(Q)], P, B, slot_stride=R, page_stride=2 * run, keep=t)
    tok, pg = d(np.array([0, T], np.int64)), d(np.array([0, T // B], np.int64))
    reqs = kvx.Requests(tok, T)
    ta = kvx.Table(pg, d(rng.permutation(P)[:T // B].astype(np.int32)))
    tb = kvx.Table(pg, d(rng.permutation(P)[:T // B].astype(np.int32)))
    if op == "gather":
        st = torch.zeros(Q * T * R, dtype=torch.uint8, device=dev)
        kvx.gather(lay, kvpool(), ta, reqs, st)
    else:
        kvx.gather_scatter(lay, kvpool(), ta, reqs, kvpool(), tb)
    torch.cuda.synchronize()


for name, L, B, T, op in (("kv_gs", 36, 16, 640, "gather_scatter"),
                          ("kv_gather", 36, 16, 640, "gather")):
    print(f"case {{name}}", file=sys.stderr, flush=True)
    kvblocks(L, B, T, op)
# permutes above one round: 4 heads of 256 B take the DRAM-page order, 8 do not
for name, L, H, seq in (("perm4", 28, 4, 1280), ("perm8", 36, 8, 640)):
    lay = kvx.Layout(L, 2, H, 128, "bf16")
    hf = torch.zeros((2 * L, H * seq * 256), dtype=torch.uint8, device=dev)
    print(f"case {{name}}", file=sys.stderr, flush=True)
    kvx.extract_permute(lay, hf, seq, seq,
                        torch.zeros(2 * L * seq * H * 256, dtype=torch.uint8, device=dev))
torch.cuda.synchronize()
# token-major pools (a slot's 72 rows of 2 KiB one run): planes 16 apart pair
lay = kvx.Layout(36, 2, 8, 128, "bf16")
S, T = 1024, 640
tmA = torch.zeros(S * 72 * 2048, dtype=torch.uint8, device=dev)
tmB = torch.zeros_like(tmA)
tmpool = lambda t: kvx.Pool([t.data_ptr() + q * 2048 for q in range(72)], S, 1,
                            slot_stride=72 * 2048, keep=t)
tok = d(np.array([0, T], np.int64))
print("case tm_gs", file=sys.stderr, flush=True)
kvx.gather_scatter(lay, tmpool(tmA), kvx.Table(tok, d(rng.permutation(S)[:T].astype(np.int32))),
                   kvx.Requests(tok, T), tmpool(tmB),
                   kvx.Table(tok, d(rng.permutation(S)[:T].astype(np.int32))))
torch.cuda.synchronize()
for name, L, H, B, T, off, op in (("large64", 36, 8, 64, 640, 0, "gather_scatter"),
                                   ("large1", 36, 8, 1, 640, 0, "gather"),
                                   ("large1gs", 36, 8, 1, 640, 0, "gather_scatter"),
                                   ("large32", 36, 8, 32, 640, 0, "gather"),
                                   ("large1k", 28, 4, 64, 1280, 0, "gather"),
                                   ("large16", 36, 8, 16, 640, 0, "gather"),
                                   ("misaligned", 36, 8, 64, 640, 2048, "gather"),
                                   ("small64", 2, 8, 64, 640, 0, "gather"),
                                   ("pieces16", 8, 16, 16, 1280, 0, "gather_scatter")):
    print(f"case {{name}}", file=sys.stderr, flush=True)
    paged(L, H, B, T, off, op)
print("dram ok", flush=True)
"""


def test_dram_page_order_reaches_the_kernels():
    """With KVX_LOG=1: a plane-major launch above one round of resident
    waves pairs the rows that share DRAM pages (2 KiB rows one per wave, 1 KiB
    rows two per wave) when a pool's pages hold runs of at least 64 KiB of a
    plane and its planes are aligned, or when a gather's or scatter's staging
    is aligned (then at any page size); not pool to pool with pages of
    32 KiB or less, with planes and staging off the 64 KiB grid, or in a
    launch of 8 KiB chunks.  Pools whose blocks hold a layer's K and V pages
    together pair the two planes in a gather-scatter, and token-major pools
    pair a token's planes 32 KiB apart.  Permutes of 4-head 1 KiB token rows
    take the DRAM-page order of their token rows; of 8-head rows not."""
    env = dict(os.environ, KVX_LOG="1")
    p = subprocess.run([sys.executable, "-c", DRAM_CHILD.format(root=ROOT)], capture_output=True,
                       text=True, timeout=180, env=env, cwd=ROOT)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "dram ok" in p.stdout
    assert "pieces/row=2" in p.stderr
    seen, case = {}, None
    for line in p.stderr.splitlines():
        if line.startswith("case "):
            case = line.split()[1]
        elif case and line.startswith("kvx: "):
            seen[case] = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
    expect = {"large64": ("1", "2"), "large1": ("1", "2"), "large1gs": ("1", "0"),
              "large32": ("1", "2"), "large1k": ("2", "2"), "large16": ("1", "2"),
              "misaligned": ("1", "0"), "small64": ("4", "0"), "pieces16": ("1", "2")}
    for case, (U, grp) in expect.items():
        f = seen[case]
        assert f["order"] == "plane-major" and f["U"] == U and f["dram_group"] == grp, (case, f)
    # K and V pages of one block (32 KiB each): a gather-scatter pairs the
    # planes, a gather pairs its staging rows instead
    f = seen["kv_gs"]
    assert f["order"] == "plane-pairs" and f["dram_group"] == "0", f
    f = seen["kv_gather"]
    assert f["order"] == "plane-major" and f["dram_group"] == "2", f
    # token-major pools: a token's planes 16 apart (32 KiB) pair
    assert seen["tm_gs"]["order"] == "token-major-pairs", seen["tm_gs"]
    assert seen["perm4"]["U"] == "1" and seen["perm4"]["order"] == "dram-pages", seen["perm4"]
    assert seen["perm8"]["U"] == "1" and seen["perm8"]["order"] == "natural", seen["perm8"]
