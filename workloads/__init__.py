"""Seeded synthetic inputs for the paged-KV path.

Shared by ``tests/``, ``bench.py`` and ``__graft_entry__.smoke()``; imported by
both sides of every parity check, so it holds none of the method's arithmetic:
it only draws slot / page tables and fills buffers with reproducible bytes.  It
never imports the HIP binding or the oracle.

Value recipe (the copy is bitwise, so values only have to be reproducible and
bit-diverse):

* Hash fill.  8-byte word ``i`` of a dense buffer filled with seed ``k`` holds
  ``splitmix64_i(k)``: output ``i`` (0-based) of the SplitMix64 generator
  started at state ``k`` (Steele, Lea & Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014; Vigna's public-domain splitmix64.c), i.e.
  ``mix(k + (i + 1) * 0x9E3779B97F4A7C15)``.  It is counter-based, so any row
  of a 36 GiB pool can be recomputed on the host, and ``devfill.hip`` computes
  the same words on the device.  Every 16-bit pattern occurs, NaNs included.
* fp16 configurations draw float32 values with numpy's PCG64 and round them to
  float16 (round to nearest even), as their workload descriptions state.

Table recipes (one function per workload; seeds are fixed per workload and
recorded with a SHA-256 of the tables) are documented on each function.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional, Sequence

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


# ------------------------------------------------------------------ values --

def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """Output ``counters[j]`` (0-based) of SplitMix64 started at ``seed``."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (counters.astype(np.uint64) + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def hash_fill_host(seed: int, nbytes: int, ctr0: int = 0) -> np.ndarray:
    """Host copy of a hash-filled buffer of ``nbytes`` (multiple of 8) as uint8."""
    if nbytes % 8:
        raise ValueError("hash fill works in 8-byte words")
    words = splitmix64(seed, np.arange(ctr0, ctr0 + nbytes // 8, dtype=np.uint64))
    return words.astype("<u8").view(np.uint8)


def hash_rows_host(seed: int, plane: int, slots: np.ndarray, row_bytes: int,
                   num_slots: int) -> np.ndarray:
    """Rows ``slots`` of plane ``plane`` of a dense hash-filled [Q][num_slots][R]
    pool, as a [len(slots), R] uint8 array (R a multiple of 8)."""
    wpr = row_bytes // 8
    slots = np.asarray(slots, dtype=np.uint64)
    base = (np.uint64(plane) * np.uint64(num_slots) + slots) * np.uint64(wpr)
    ctr = base[:, None] + np.arange(wpr, dtype=np.uint64)[None, :]
    return splitmix64(seed, ctr).astype("<u8").view(np.uint8).reshape(len(slots), row_bytes)


def uniform_f16(seed: int, shape) -> np.ndarray:
    """Uniform [0, 1) float32 values rounded to float16."""
    return np.random.default_rng(seed).random(shape, dtype=np.float32).astype(np.float16)


def normal_f16(seed: int, shape) -> np.ndarray:
    """Standard normal float32 values rounded to float16."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32).astype(np.float16)


# ---------------------------------------------------------------- geometry --

ELEM_BYTES = {"f16": 2, "bf16": 2, "fp8": 1, "f32": 4}


@dataclasses.dataclass(frozen=True)
class Geometry:
    """Row shape of a KV pool: Q = layers x num_kv planes of [slots, H, D]."""
    num_layers: int
    num_kv: int
    kv_heads: int
    head_dim: int
    dtype: str = "bf16"

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def planes(self) -> int:
        return self.num_layers * self.num_kv

    @property
    def row_bytes(self) -> int:
        return self.kv_heads * self.head_dim * self.elem_bytes

    @property
    def head_bytes(self) -> int:
        return self.head_dim * self.elem_bytes

    @property
    def token_bytes(self) -> int:
        return self.planes * self.row_bytes


@dataclasses.dataclass
class Side:
    """Where a batch's tokens live in one pool: CSR page table + paging."""
    num_pages: int
    page_size: int
    pg_off: np.ndarray      # int64 [num_reqs + 1]
    ids: np.ndarray         # int32 page ids

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size


@dataclasses.dataclass
class PagedCase:
    """One paged workload: geometry, the token CSR and per-pool page tables."""
    name: str
    geom: Geometry
    tok_off: np.ndarray                 # int64 [num_reqs + 1]
    src: Side
    dst: Optional[Side]
    value_seed: int
    sentinel_seed: int
    table_seed: int
    values: str = "hash"                # "hash" | "uniform_f16"

    @property
    def num_reqs(self) -> int:
        return len(self.tok_off) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.tok_off[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.tok_off)

    def payload_bytes(self) -> int:
        """Bytes moved one way (rows x row size), excluding tables."""
        return self.total_tokens * self.geom.token_bytes

    def table_sha256(self) -> str:
        parts = [self.tok_off, self.src.pg_off, self.src.ids]
        if self.dst is not None:
            parts += [self.dst.pg_off, self.dst.ids]
        return table_sha256(*parts)


def table_sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def csr_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


def side_from_slot_lists(slot_lists: Sequence[np.ndarray], num_slots: int) -> Side:
    """Page-size-1 side whose page ids are the given slot lists, request by request."""
    lens = [len(s) for s in slot_lists]
    ids = (np.concatenate([np.asarray(s, dtype=np.int32) for s in slot_lists])
           if slot_lists else np.zeros(0, np.int32))
    return Side(num_pages=num_slots, page_size=1, pg_off=csr_from_lengths(lens),
                ids=ids.astype(np.int32))


def side_from_page_lists(page_lists: Sequence[np.ndarray], num_pages: int,
                         page_size: int) -> Side:
    lens = [len(p) for p in page_lists]
    ids = (np.concatenate([np.asarray(p, dtype=np.int32) for p in page_lists])
           if page_lists else np.zeros(0, np.int32))
    return Side(num_pages=num_pages, page_size=page_size, pg_off=csr_from_lengths(lens),
                ids=ids.astype(np.int32))


# --------------------------------------------------------------- workloads --

QWEN15B = Geometry(28, 2, 2, 128, "f16")      # 28 KiB per token
KV144K = Geometry(36, 2, 8, 128, "bf16")      # 144 KiB per token, 2 KiB rows
QWEN7B = Geometry(28, 2, 4, 128, "f16")       # 56 KiB per token


def qwen15b_128tok_page1() -> PagedCase:
    """Qwen2.5-1.5B-shaped KV (fp16, 28 layers x {K,V} x 2 heads x 128): one
    128-token request whose slots are a seeded random 128-subset of a 1024-slot
    token-paged pool; the scatter target is an independent 128-subset of a
    second 1024-slot pool.  Values uniform [0, 1) in fp16."""
    rng = np.random.default_rng(1001)
    src = rng.choice(1024, 128, replace=False)
    dst = rng.choice(1024, 128, replace=False)
    return PagedCase("qwen1.5b_128tok_page1", QWEN15B, csr_from_lengths([128]),
                     side_from_slot_lists([src], 1024), side_from_slot_lists([dst], 1024),
                     value_seed=2001, sentinel_seed=3001, table_seed=1001, values="uniform_f16")


def kv144k_2048tok_page1(request: int = 0, num_requests_in_pool: int = 16) -> PagedCase:
    """One 2048-token request at 144 KiB/token (36 layers x {K,V} x 8 heads x
    128, bf16, 288 MiB): source slots are a slice of a seeded permutation of a
    32768-slot token-paged pool, destination slots a slice of an independent
    permutation of a second 32768-slot pool.  ``request`` picks one of 16
    disjoint slices (used to rotate requests between timed launches)."""
    if not 0 <= request < num_requests_in_pool:
        raise ValueError("request index out of range")
    rng = np.random.default_rng(1002)
    perm_a = rng.permutation(32768)
    perm_b = rng.permutation(32768)
    sl = slice(2048 * request, 2048 * (request + 1))
    return PagedCase(f"kv144k_2048tok_page1_req{request}", KV144K, csr_from_lengths([2048]),
                     side_from_slot_lists([perm_a[sl]], 32768),
                     side_from_slot_lists([perm_b[sl]], 32768),
                     value_seed=2002, sentinel_seed=3002, table_seed=1002)


def churned_free_list(rng: np.random.Generator, num_slots: int, cycles: int = 10000,
                      max_alloc: int = 2048) -> np.ndarray:
    """Free-list order after seeded allocate/free churn (FIFO list).

    Starts as 0..N-1.  Each cycle draws k ~ U{1..max_alloc}; if an allocation
    is live and (fewer than k slots are free, or a fair coin says so) a
    uniformly chosen live allocation is freed and its slots are appended in
    shuffled order; otherwise k slots are taken from the head.  At the end all
    live allocations are freed in random order, each shuffled.
    """
    ring = np.arange(num_slots, dtype=np.int64)
    head, count = 0, num_slots
    live: List[np.ndarray] = []

    def take(k):
        nonlocal head, count
        idx = (head + np.arange(k)) % num_slots
        out = ring[idx].copy()
        head = (head + k) % num_slots
        count -= k
        return out

    def give(a):
        nonlocal count
        idx = (head + count + np.arange(len(a))) % num_slots
        ring[idx] = a
        count += len(a)

    for _ in range(cycles):
        k = int(rng.integers(1, max_alloc + 1))
        if live and (count < k or rng.random() < 0.5):
            a = live.pop(int(rng.integers(len(live))))
            give(rng.permutation(a))
        else:
            live.append(take(k))
    for i in rng.permutation(len(live)):
        give(rng.permutation(live[i]))
    return take(count)


def kv144k_32req_fragmented(num_slots: int = 131072, num_reqs: int = 32) -> PagedCase:
    """Fragmented layer-major pool (one [slots, 8, 128] bf16 tensor per layer
    per K/V, 36 layers, 2 KiB rows): 32 requests with lengths U{1024..2048},
    slots allocated in order from a free list shuffled by 10k seeded
    allocate/free cycles.  One batched gather of all requests into staging."""
    rng = np.random.default_rng(1003)
    free = churned_free_list(rng, num_slots)
    lens = rng.integers(1024, 2049, size=num_reqs)
    slots, pos = [], 0
    for n in lens:
        slots.append(free[pos:pos + n])
        pos += int(n)
    return PagedCase("kv144k_32req_fragmented_page1", KV144K, csr_from_lengths(lens),
                     side_from_slot_lists(slots, num_slots), None,
                     value_seed=2003, sentinel_seed=3003, table_seed=1003)


@dataclasses.dataclass
class PermuteCase:
    """HF DynamicCache-shaped planes [1, H, s_cap, D] and the extract length."""
    name: str
    geom: Geometry
    s_cap: int
    seq: int
    value_seed: int
    sentinel_seed: int

    def payload_bytes(self) -> int:
        return self.geom.planes * self.seq * self.geom.row_bytes


def qwen7b_permute(seq: int = 1024) -> PermuteCase:
    """Qwen2.5-7B shape (28 layers x {K,V}, 4 heads, 128, fp16): HF layout
    [1, heads, seq, dim] <-> [seq, heads, dim], seq in {1024, 8192}, values
    normal(0, 1) rounded to fp16."""
    if seq not in (1024, 8192):
        raise ValueError("seq is 1024 or 8192")
    return PermuteCase(f"qwen7b_permute_seq{seq}", QWEN7B, seq, seq,
                       value_seed=2004 + seq, sentinel_seed=3004 + seq)


def kv144k_64req_page16(num_reqs: int = 64, num_blocks: int = 16384, page_size: int = 16) -> PagedCase:
    """vLLM-style block pools, page 16, bf16, 144 KiB/token, 16384 blocks of 16
    tokens (262144 token slots, 36 GiB) per pool: 64 requests of 2032 + f
    tokens, f ~ U{1..16} (so 128 pages each, the last partly filled); block
    tables are the first 8192 entries of a seeded permutation of the block ids,
    64 x 128, independently for source and destination.  One gather-scatter."""
    rng = np.random.default_rng(1005)
    pages_per_req = 128
    fill = rng.integers(1, page_size + 1, size=num_reqs)
    lens = (pages_per_req - 1) * page_size + fill
    src_perm = rng.permutation(num_blocks)[: num_reqs * pages_per_req]
    dst_perm = rng.permutation(num_blocks)[: num_reqs * pages_per_req]
    src = side_from_page_lists(np.split(src_perm, num_reqs), num_blocks, page_size)
    dst = side_from_page_lists(np.split(dst_perm, num_reqs), num_blocks, page_size)
    return PagedCase("kv144k_64req_page16", KV144K, csr_from_lengths(lens), src, dst,
                     value_seed=2005, sentinel_seed=3005, table_seed=1005)


MLA_LITE = Geometry(27, 1, 1, 576, "bf16")   # one 576-element latent+rope row per layer


def mla_case(page_size: int = 1, request: int = 0, tokens: int = 2048,
             num_slots: int = 32768) -> PagedCase:
    """Single-plane (MLA) pools, DeepSeek-V2-Lite-sized rows: 27 layers, one
    576-element bf16 vector per token and layer (1152-byte rows, 30.4 KiB per
    token).  One request of ``tokens`` tokens; its source and destination
    pages are slice ``request`` (of 16 disjoint ones) of independent seeded
    permutations of pools of ``num_slots`` token slots."""
    rng = np.random.default_rng(1007 + page_size)
    pages = num_slots // page_size
    need = -(-tokens // page_size)
    if not 0 <= request < pages // need:
        raise ValueError("request index out of range")
    sl = slice(need * request, need * (request + 1))
    src = side_from_page_lists([rng.permutation(pages)[sl]], pages, page_size)
    dst = side_from_page_lists([rng.permutation(pages)[sl]], pages, page_size)
    return PagedCase(f"mla27x576_{tokens}tok_page{page_size}", MLA_LITE,
                     csr_from_lengths([tokens]), src, dst,
                     value_seed=2007, sentinel_seed=3007, table_seed=1007 + page_size)


def hetero_tp_case(num_reqs: int = 16, num_blocks: int = 4096, page_size: int = 16) -> PagedCase:
    """P and D with different tensor-parallel sizes: 36 layers x {K,V},
    head_dim 128, bf16, 8 KV heads in total; P runs TP=1 (8 heads per token
    row) and D runs TP=2 (4 heads per row per rank).  Block pools of 4096
    HND blocks of 16 tokens; 16 requests of 2032 + U{1..16} tokens with block
    tables drawn from seeded permutations.  The geometry's kv_heads is the
    slice width moved per call (4: one D rank's share)."""
    rng = np.random.default_rng(1006)
    pages_per_req = 128
    fill = rng.integers(1, page_size + 1, size=num_reqs)
    lens = (pages_per_req - 1) * page_size + fill
    src_perm = rng.permutation(num_blocks)[: num_reqs * pages_per_req]
    dst_perm = rng.permutation(num_blocks)[: num_reqs * pages_per_req]
    src = side_from_page_lists(np.split(src_perm, num_reqs), num_blocks, page_size)
    dst = side_from_page_lists(np.split(dst_perm, num_reqs), num_blocks, page_size)
    return PagedCase("kv144k_16req_page16_hnd_tp1_to_tp2", Geometry(36, 2, 4, 128, "bf16"),
                     csr_from_lengths(lens), src, dst,
                     value_seed=2006, sentinel_seed=3006, table_seed=1006)


def random_case(seed: int, geom: Optional[Geometry] = None, max_reqs: int = 6,
                max_len: int = 70, src_page: Optional[int] = None,
                dst_page: Optional[int] = None, oor_frac: float = 0.0,
                slack_pages: int = 7, index_faults: bool = False) -> PagedCase:
    """Small random paged case for fuzzing: ragged requests (empty ones
    included), page sizes drawn from {1, 2, 3, 4, 16}, distinct destination
    pages, source pages drawn with replacement, and optionally a fraction of
    page ids made out of range (negative or >= num_pages).

    ``index_faults``: page-table offsets that send some lookups outside the
    page-id array or into another request's list, with the destination's
    written rows still distinct.  Source side: one request's list starts
    1-3 entries early (negative indices for request 0, else the previous
    request's last entries), one request (of three or more) starts past the
    end of the array, and the array loses its last 1-2 entries.  Destination
    side: request 0's list starts 1-3 entries early (its first pages'
    lookups fall below 0, later ones reuse its own earlier entries) and the
    array loses its last 1-2 entries (the last pages' lookups run past it)."""
    rng = np.random.default_rng(seed)
    if geom is None:
        geom = Geometry(int(rng.integers(1, 4)), int(rng.choice([1, 2])),
                        int(rng.choice([1, 2, 3, 4])), int(rng.choice([8, 16, 64])), "bf16")
    nreq = int(rng.integers(1, max_reqs + 1))
    lens = rng.integers(0, max_len + 1, size=nreq)
    if nreq > 1:
        lens[rng.integers(nreq)] = 0
    bs = int(src_page or rng.choice([1, 2, 3, 4, 16]))
    bd = int(dst_page or rng.choice([1, 2, 3, 4, 16]))
    pages_s = [-(-int(n) // bs) for n in lens]
    pages_d = [-(-int(n) // bd) for n in lens]
    ns = sum(pages_s) + slack_pages
    nd = sum(pages_d) + slack_pages
    src_lists = [rng.integers(0, ns, size=p) for p in pages_s]
    dperm = rng.permutation(nd)
    dst_lists, pos = [], 0
    for p in pages_d:
        dst_lists.append(dperm[pos:pos + p])
        pos += p
    src = side_from_page_lists(src_lists, ns, bs)
    dst = side_from_page_lists(dst_lists, nd, bd)
    for side in (src, dst):
        if oor_frac > 0 and side.ids.size:
            m = rng.random(side.ids.size) < oor_frac
            bad = np.where(rng.random(side.ids.size) < 0.5, -1 - rng.integers(0, 5, side.ids.size),
                           side.num_pages + rng.integers(0, 5, side.ids.size))
            side.ids = np.where(m, bad, side.ids).astype(np.int32)
    if index_faults:
        _index_faults(rng, src, source=True)
        _index_faults(rng, dst, source=False)
    return PagedCase(f"random_{seed}", geom, csr_from_lengths(lens), src, dst,
                     value_seed=5000 + seed, sentinel_seed=6000 + seed, table_seed=seed)


def _index_faults(rng: np.random.Generator, side: Side, source: bool) -> None:
    """Move page-table offsets as random_case's ``index_faults`` describes."""
    nreq = len(side.pg_off) - 1
    pg = side.pg_off.copy()
    if source and nreq >= 1:
        pg[int(rng.integers(nreq))] -= int(rng.integers(1, 4))
        if nreq >= 3:
            pg[int(rng.integers(nreq))] = side.ids.size + int(rng.integers(0, 3))
    elif nreq >= 1:
        pg[0] -= int(rng.integers(1, 4))
    cut = int(rng.integers(1, 3))
    side.ids = side.ids[:max(0, side.ids.size - cut)].copy()
    side.pg_off = pg
