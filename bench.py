#!/usr/bin/env python3
"""Benchmark of the paged-KV data-movement path on one MI355X.

Workload: one 2048-token request at 144 KiB per token (36 layers x {K,V} x 8
KV heads x 128, bf16; 288 MiB), in token-paged pools of 32768 slots (4.5 GiB
each), two pools in the one GPU's HBM, slots a seeded random subset of each
pool.  A step is one pass of the whole path:

  gather_scatter  pool A -> pool B directly ("P writes D's pages")
  gather          pool A -> contiguous staging [plane][token][H][D]
  rebuild         staging -> HF cache tensors [1, H, seq, D] per plane
  extract         HF cache tensors -> a second staging buffer
  scatter         second staging -> pool B

Each op moves 288 MiB in and 288 MiB out (603,979,776 bytes read + written).
Steps rotate over 16 disjoint requests of the pools, and the staging and HF
buffers the ops hand to each other are double-buffered: rebuild reads the
staging the previous step's gather wrote, extract the HF tensors the
previous step's rebuild wrote, scatter the staging the previous step's
extract wrote (the rows gathered three steps earlier).  About 1.4 GB is
written between producing a buffer and reading it back, so no op finds its
input in the 256 MiB Infinity Cache: every byte counted is an HBM byte.
Inputs are resident in HBM before the timed region.

Printed (one JSON line on stdout): step throughput in GB/s (read + write,
decimal), its fraction of the 8 TB/s HBM peak, ms per 288 MiB request for the
gather-scatter, per-op times from HIP events recorded on the launch stream,
each op timed alone (per launch, rotated inputs, nothing reading its output)
with its fraction of peak against the 70% bar, a contiguous-copy ceiling of
equal bytes, the roofline of the dominant kernel, and the CPU oracle timed
on the host on a bounded sample of the same steps.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --all-configs         (every op on every workload, beside a plain
                                         copy of equal bytes and the oracle on a sample)
  python bench.py --concurrent          (the transfer under a decode-like HBM reader)
  python bench.py --cu-split            (the two on complementary CU-masked streams)
  python bench.py --comparators         (per-block runtime copies, DMA copy of staging)
  python bench.py --patterns            (the request's row patterns moved without tables)
  python bench.py --dram-pages          (equal-density slot placements: rows sharing DRAM pages)
  python bench.py --sizes               (one request of 16 .. 8192 tokens: latency to bandwidth)
  python bench.py --batches             (49152 tokens in 1 .. 49152 requests: request lookup)
  python bench.py --row-sizes           (rows of 256 B .. 16 KiB at ~256 MiB each way)
  python bench.py --pmc-pass            (short run for rocprofv3 --pmc)
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --pmc-out OUT
  python bench.py --summarize-trace TRACE_DIR OUT TITLE COMMAND
  python bench.py --counter-commands    (rocprofv3 commands of the memory/wave counter passes)
  python bench.py --summarize-counters OUT TITLE
  python bench.py --summarize-json LOG OUT TITLE COMMAND   (f3 / f4 JSON lines -> markdown)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged KV gather GB/s (read+write) & % HBM peak; ms per 288 MiB request"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, 8 TB/s
NREQ = 16                         # disjoint 2048-token requests per pool
OPS = ["gather_scatter", "gather", "rebuild", "extract", "scatter"]
KERNEL_SOURCES = ["scatter_kvx_gather_amd/csrc/kvx_kernels.hpp",
                  "scatter_kvx_gather_amd/csrc/kvx.hip"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "kv144k_2048tok_page1_hbm_traffic.md")
COPY_CALIB_BYTES = 4 * 32768 * 2048     # four 64 MiB planes


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def code_of(text: str) -> str:
    """C++ source with comments and whitespace removed: what the compiler
    sees, so an edit to a comment does not count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


def kernel_source_sha256(sources=None) -> str:
    """SHA-256 over the code (comments and whitespace removed) of the kernel
    sources; `sources` maps a path in KERNEL_SOURCES to its text (default:
    read the files)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if sources is not None:
            text = sources[rel]
        else:
            with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
                text = f.read()
        h.update(code_of(text).encode())
    return h.hexdigest()


def read_traffic():
    """Per-launch HBM bytes of the dominant kernel from the committed counter
    summary, or None when it is missing or the kernel changed since."""
    if not os.path.exists(PMC_SUMMARY):
        return None, None
    vals = {}
    with open(PMC_SUMMARY) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_sha256():
        return None, vals.get("kernel")
    try:
        return int(vals["traffic_bytes_per_launch"]), vals.get("kernel")
    except (KeyError, ValueError):
        return None, vals.get("kernel")


# ------------------------------------------------------------------ setup --

class Workload:
    """The 2048-token, 144 KiB/token request in two token-paged pools.  With
    the default 32768-slot pools (4.5 GiB each) it is the bench workload
    (16 disjoint requests); smaller pools (the translation-counter runs) hold
    slots // 2048 disjoint requests drawn from seeded permutations."""

    def __init__(self, torch, kvx, wl, wdev, dev, stream, slots=32768):
        self.torch = torch
        g = wl.KV144K
        self.geom = g
        self.Q, self.R, self.S = g.planes, g.row_bytes, slots
        self.T = 2048
        if slots == 32768:
            self.cases = [wl.kv144k_2048tok_page1(k) for k in range(NREQ)]
        else:
            import numpy as np
            rng = np.random.default_rng(1002 + slots)
            pa, pb = rng.permutation(slots), rng.permutation(slots)
            self.cases = [wl.PagedCase(f"kv144k_2048tok_page1_{slots}slots_req{k}", g,
                                       wl.csr_from_lengths([2048]),
                                       wl.side_from_slot_lists([pa[2048 * k:2048 * (k + 1)]],
                                                               slots),
                                       wl.side_from_slot_lists([pb[2048 * k:2048 * (k + 1)]],
                                                               slots),
                                       2002, 3002, 1002 + slots)
                          for k in range(slots // 2048)]
        self.nreq = len(self.cases)
        c0 = self.cases[0]
        Q, R, S, T = self.Q, self.R, self.S, self.T
        with torch.cuda.stream(stream):
            self.A = torch.empty((Q, S, R), dtype=torch.uint8, device=dev)
            self.B = torch.empty((Q, S, R), dtype=torch.uint8, device=dev)
            wdev.fill_hash(self.A, c0.value_seed, stream=stream)
            wdev.fill_hash(self.B, c0.sentinel_seed, stream=stream)
            # double-buffered hand-offs: gather -> S1[i % 2] -> rebuild (next
            # step) -> HF[.] -> extract (next step) -> S2[.] -> scatter (next step)
            self.S1s = [torch.zeros(T * Q * R, dtype=torch.uint8, device=dev) for _ in range(2)]
            self.S2s = [torch.zeros(T * Q * R, dtype=torch.uint8, device=dev) for _ in range(2)]
            self.HFs = [torch.zeros((Q, g.kv_heads * T * g.head_bytes), dtype=torch.uint8,
                                    device=dev) for _ in range(2)]
            self.S1, self.S2, self.HF = self.S1s[0], self.S2s[0], self.HFs[0]

            def d(a):
                return torch.from_numpy(a).to(dev)
            self.reqs = kvx.Requests(d(c0.tok_off), T)
            self.src_tabs = [kvx.Table(d(c.src.pg_off), d(c.src.ids)) for c in self.cases]
            self.dst_tabs = [kvx.Table(d(c.dst.pg_off), d(c.dst.ids)) for c in self.cases]
        self.lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
        self.PA = kvx.Pool(self.A, S)
        self.PB = kvx.Pool(self.B, S)
        self.op_bytes = 2 * T * Q * R               # read + write per op
        self.seeds = {"tables": c0.table_seed, "source_values": c0.value_seed,
                      "destination_values": c0.sentinel_seed}
        self.tables_sha256 = hashlib.sha256(
            "".join(c.table_sha256() for c in self.cases).encode()).hexdigest()
        # page tables the kernels read per step (not in the payload bytes):
        # tok_off once per paged op, pg_off + page ids once per pool side
        # (gather-scatter two sides, gather and scatter one each)
        side = c0.src.pg_off.nbytes + c0.src.ids.size * 4
        self.table_bytes_per_step = 3 * c0.tok_off.nbytes + 4 * side
        self.kvx = kvx

    def requests_of(self, i):
        """Requests of step i: gather-scatter k_gs, gather k_g, and the
        request whose rows the scatter writes back, k_sc -- the one gathered
        three steps earlier (its rows reach the scatter through rebuild,
        extract and the double buffers).  k_gs is even and k_sc odd, so the
        two writes into pool B never share a row."""
        n = self.nreq
        return (2 * i) % n, (2 * i + 1) % n, (2 * i - 5) % n

    def step(self, i, stream, ev=None, marks=(0, 1, 2, 3, 4, 5)):
        """One pass of the path; event ev[j] is recorded before op j (after the
        last op for j = 5) for every j in marks."""
        kvx, lay = self.kvx, self.lay
        k_gs, k_g, k_sc = self.requests_of(i)
        cur, prev = i % 2, (i - 1) % 2
        T = self.T

        def mark(j):
            if ev is not None and j in marks:
                ev[j].record(stream)
        mark(0)
        kvx.gather_scatter(lay, self.PA, self.src_tabs[k_gs], self.reqs, self.PB,
                           self.dst_tabs[k_gs], stream=stream)
        mark(1)
        kvx.gather(lay, self.PA, self.src_tabs[k_g], self.reqs, self.S1s[cur], stream=stream)
        mark(2)
        kvx.rebuild_permute(lay, self.S1s[prev], T, self.HFs[cur], T, stream=stream)
        mark(3)
        kvx.extract_permute(lay, self.HFs[prev], T, T, self.S2s[cur], stream=stream)
        mark(4)
        kvx.scatter(lay, self.S2s[prev], self.reqs, self.PB, self.dst_tabs[k_sc], stream=stream)
        mark(5)

    def isolated(self, op, k, stream):
        """Launch k of `op` timed alone: rotated requests, inputs read from
        buffers written long before (four staging buffers, two HF sets), and
        nothing reads the output."""
        kvx, lay, T = self.kvx, self.lay, self.T
        stages = self.S1s + self.S2s
        n = self.nreq
        if op == "gather_scatter":
            kvx.gather_scatter(lay, self.PA, self.src_tabs[k % n], self.reqs, self.PB,
                               self.dst_tabs[k % n], stream=stream)
        elif op == "gather":
            kvx.gather(lay, self.PA, self.src_tabs[k % n], self.reqs, self.S1s[k % 2],
                       stream=stream)
        elif op == "rebuild":
            kvx.rebuild_permute(lay, stages[k % 4], T, self.HFs[k % 2], T, stream=stream)
        elif op == "extract":
            kvx.extract_permute(lay, self.HFs[k % 2], T, T, stages[(k + 1) % 4], stream=stream)
        elif op == "scatter":
            kvx.scatter(lay, stages[k % 4], self.reqs, self.PB, self.dst_tabs[k % n],
                        stream=stream)


def settle_steps(torch, wk, stream, block=8, max_s=2.0, tol=0.03):
    """Setup, before the warmup steps: untimed steps in blocks of `block`
    until two blocks in a row take the same GPU time per step (within
    `tol`) and the host enqueues a block faster than the GPU runs it, or
    `max_s` seconds have passed.  Measured: a bench process started after
    another had used the GPU ran its first ~40 steps with the GPU idle
    between kernels (2.1-2.3 ms per step of 0.53 ms of kernels; the kernels
    themselves at their usual times); a measurement of K steps after W = 5
    warmup steps fell inside that phase.  Returns the steps run and the
    per-block times."""
    import time as _t
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = _t.perf_counter()
    blocks, prev, i = [], None, 0
    while True:
        torch.cuda.synchronize()
        h0 = _t.perf_counter()
        e0.record(stream)
        for _ in range(block):
            wk.step(i, stream)
            i += 1
        e1.record(stream)
        host = (_t.perf_counter() - h0) * 1e3 / block
        torch.cuda.synchronize()
        gpu = e0.elapsed_time(e1) / block
        blocks.append((round(gpu, 4), round(host, 4)))
        if prev is not None and abs(gpu - prev) <= tol * prev and host < gpu:
            break
        if _t.perf_counter() - t0 > max_s:
            break
        prev = gpu
    log(f"settle: {i} steps in {_t.perf_counter() - t0:.2f} s, ms/step per block "
        f"(gpu, host): {blocks}")
    return {"steps": i, "seconds": round(_t.perf_counter() - t0, 3),
            "blocks_gpu_host_ms_per_step": blocks}


def time_isolated(torch, wk, stream, n=24, warm=8):
    """Each op alone, two ways, after `warm` launches: n launches back to back
    between two HIP events on the launch stream (the sustained rate of a
    stream of such calls: ms per launch, GB/s, fraction of the HBM peak), and
    n launches with events around each one (one launch from start to end,
    its ramp-up and drain included: median ms and fraction)."""
    out = {}
    ev = torch.cuda.Event
    for op in OPS:
        for k in range(warm):
            wk.isolated(op, k, stream)
        e0, e1 = ev(enable_timing=True), ev(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(n):
            wk.isolated(op, warm + k, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        sustained = e0.elapsed_time(e1) / n
        evs = [(ev(enable_timing=True), ev(enable_timing=True)) for _ in range(n)]
        for k, (a, b) in enumerate(evs):
            a.record(stream)
            wk.isolated(op, warm + n + k, stream)
            b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        med = ms[len(ms) // 2]
        gbps = wk.op_bytes / (sustained * 1e-3) / 1e9
        one = wk.op_bytes / (med * 1e-3) / 1e9
        out[op] = {"ms_per_launch": round(sustained, 5), "GBps": round(gbps, 1),
                   "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                   "single_launch_ms_median": round(med, 5),
                   "single_launch_frac_hbm_peak": round(one / HBM_PEAK_GBPS, 4),
                   "launches": n}
    return out


# -------------------------------------------------------------- cpu side --

def cpu_share():
    """Cores this process may use: the affinity mask, capped by a cgroup CPU
    quota when one is set (cgroup v2 cpu.max, else v1 cfs quota / period)."""
    import math
    nproc = os.cpu_count() or 1
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
            if q != "max":
                quota = int(q) / int(period)
    except (OSError, ValueError):
        try:
            with open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us") as f:
                q = int(f.read())
            with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
                period = int(f.read())
            if q > 0:
                quota = q / period
        except (OSError, ValueError):
            pass
    cg = math.ceil(quota) if quota else None
    usable = min(aff, cg) if cg else aff
    return {"nproc": nproc, "affinity": aff, "cgroup_cpus": cg, "usable": max(1, usable)}


def cpu_baseline(wk, budget_s, parity_step=None):
    """Time the oracle on host copies of the same pools and requests, running
    the same step as the GPU (same ops, requests and double buffers) at one
    thread and at every usable core.  With parity_step j (>= 3, the last step
    run on the GPU before this call), first check that step's results
    bitwise against the oracle: the gather-scatter's and the scatter's
    destination rows of pool B equal the source rows of pool A, the gather's
    staging equals the oracle's gather, and extract(rebuild(.)) returned the
    staging gathered two steps earlier."""
    import numpy as np

    import oracle
    Q, R, S, T = wk.Q, wk.R, wk.S, wk.T
    g = wk.geom
    log("cpu baseline: reading pools back to host")
    A_h = wk.A.cpu().numpy()
    B_h = wk.B.cpu().numpy()
    S1 = [np.zeros(T * Q * R, np.uint8) for _ in range(2)]
    S2 = [np.zeros(T * Q * R, np.uint8) for _ in range(2)]
    HF = [np.zeros((Q, g.kv_heads * T * g.head_bytes), np.uint8) for _ in range(2)]
    A_planes = [A_h[q].reshape(-1) for q in range(Q)]
    B_planes = [B_h[q].reshape(-1) for q in range(Q)]
    HF_planes = [[h[q] for q in range(Q)] for h in HF]
    c0 = wk.cases[0]
    share = cpu_share()
    ncores = share["usable"]
    parity = None
    if parity_step is not None:
        j = parity_step
        k_gs, k_g, k_sc = wk.requests_of(j)
        _, k_g2, _ = wk.requests_of(j - 2)
        S1_dev, S2_dev = wk.S1s[j % 2].cpu().numpy(), wk.S2s[j % 2].cpu().numpy()

        def rows(planes, side):
            out = np.zeros(T * Q * R, np.uint8)
            oracle.gather(planes, R, 1, S, R, c0.tok_off, side.pg_off, side.ids, out, ncores)
            return out
        cs = wk.cases
        parity = {
            "step": j,
            "gather_scatter_rows_equal_source_rows":
                bool(np.array_equal(rows(B_planes, cs[k_gs].dst), rows(A_planes, cs[k_gs].src))),
            "gather_equals_oracle": bool(np.array_equal(S1_dev, rows(A_planes, cs[k_g].src))),
            "extract_of_rebuild_equals_staging_of_two_steps_before":
                bool(np.array_equal(S2_dev, rows(A_planes, cs[k_g2].src))),
            "scatter_rows_equal_source_rows":
                bool(np.array_equal(rows(B_planes, cs[k_sc].dst), rows(A_planes, cs[k_sc].src))),
        }
        log(f"parity of step {j}: {parity}")
        del S1_dev, S2_dev

    def step(i, nt):
        k_gs, k_g, k_sc = wk.requests_of(i)
        a, b, c = wk.cases[k_gs], wk.cases[k_g], wk.cases[k_sc]
        cur, prev = i % 2, (i - 1) % 2
        oracle.gather_scatter(A_planes, R, 1, S, a.src.pg_off, a.src.ids, R, c0.tok_off,
                              B_planes, R, 1, S, a.dst.pg_off, a.dst.ids, nt)
        oracle.gather(A_planes, R, 1, S, R, c0.tok_off, b.src.pg_off, b.src.ids, S1[cur], nt)
        oracle.rebuild_permute(S1[prev], g.kv_heads, g.head_bytes, T, HF_planes[cur], T, nt)
        oracle.extract_permute(HF_planes[prev], g.kv_heads, g.head_bytes, T, T, S2[cur], nt)
        oracle.scatter(S2[prev], R, c0.tok_off, c.dst.pg_off, c.dst.ids, B_planes, R, 1, S, nt)

    out = {}
    for nt in sorted({1, ncores}):
        step(0, nt)                                # pre-fault staging and HF pages
        step(1, nt)
        runs = []
        for _ in range(1 if nt == 1 else 3):       # the threaded rate: median of 3 runs
            steps, t0 = 0, time.perf_counter()
            while True:
                step(steps + 2, nt)
                steps += 1
                el = time.perf_counter() - t0
                if el >= (budget_s if nt == 1 else budget_s / 3) or steps >= 200:
                    break
            runs.append((steps, el))
            log(f"cpu baseline: {nt} thread(s): {steps} steps in {el:.2f} s")
        runs.sort(key=lambda r: r[0] / r[1])
        out[nt] = runs[len(runs) // 2]
    del A_h, B_h
    return out, ncores, parity, share


def host_cpu():
    """Model name and socket count of the host CPU: lscpu's "Model name" and
    "Socket(s)" when lscpu runs, else /proc/cpuinfo's model name and physical
    ids."""
    import subprocess
    model, sockets = None, None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            key, _, val = line.partition(":")
            if key.strip() == "Model name" and model is None:
                model = val.strip()
            elif key.strip() == "Socket(s)":
                try:
                    sockets = int(val.strip())
                except ValueError:
                    pass
    except (OSError, subprocess.SubprocessError):
        pass
    ids = set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "model name" and model is None:
                    model = val.strip()
                elif key == "physical id":
                    ids.add(val.strip())
    except OSError:
        pass
    return model or "unknown", sockets or max(1, len(ids))


# ----------------------------------------------------------------- pmc --

def counter_rows(d):
    """Rows of every rocprofv3 counter_collection.csv under directory d."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for fn in files:
        with open(fn) as f:
            out.extend(csv.DictReader(f))
    return out


def summarize_pmc(fetch_dir, write_dir, out_path):
    """Traffic per launch of the dominant kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads
    for the plain copy kernel of COPY_CALIB_BYTES run in the same process."""
    def per_kernel(d, counter):
        acc = {}
        for r in counter_rows(d):
            if r.get("Counter_Name") != counter:
                continue
            name = r["Kernel_Name"]
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
        return acc

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def pick(acc, key):
        ks = [k for k in acc if key in k]
        if not ks:
            raise SystemExit(f"kernel matching {key!r} not found: {sorted(acc)[:8]}")
        vals = acc[ks[0]]
        return ks[0], sorted(vals)[len(vals) // 2]
    dom = "k_paged<kvx::PoolRef, kvx::PoolRef"
    kname, f_kib = pick(fetch, dom)
    _, w_kib = pick(write, dom)
    _, fc_kib = pick(fetch, "k_copy16")
    _, wc_kib = pick(write, "k_copy16")
    f_scale = (COPY_CALIB_BYTES / 1024.0) / fc_kib
    w_scale = (COPY_CALIB_BYTES / 1024.0) / wc_kib
    fetch_b = f_kib * f_scale * 1024
    write_b = w_kib * w_scale * 1024
    algo = 2 * 2048 * 72 * 2048
    with open(out_path, "w") as f:
        f.write("# HBM traffic per launch, 288 MiB request (kv144k, page 1): the gather-scatter "
                "kernel, then every kernel of the step\n\n")
        f.write("Two `rocprofv3 --pmc` runs of `python bench.py --pmc-pass` (one counter each);\n")
        f.write("median per dispatch, scaled by the plain copy kernel `k_copy16` of\n")
        f.write(f"{COPY_CALIB_BYTES} bytes run in the same process.\n\n")
        f.write("Commands (from the repository root, on an MI355X machine):\n\n")
        f.write("    rocprofv3 --pmc FETCH_SIZE -d rocprof_out/pmc_fetch -o pmc --output-format csv "
                "-- python3 bench.py --pmc-pass\n")
        f.write("    rocprofv3 --pmc WRITE_SIZE -d rocprof_out/pmc_write -o pmc --output-format csv "
                "-- python3 bench.py --pmc-pass\n")
        f.write("    python3 bench.py --summarize-pmc rocprof_out/pmc_fetch rocprof_out/pmc_write "
                "--pmc-out profiles/kv144k_2048tok_page1_hbm_traffic.md\n\n")
        f.write(f"- kernel: `{kname}`\n")
        f.write(f"- fetch_kib_per_dispatch: {f_kib:.1f}\n")
        f.write(f"- write_kib_per_dispatch: {w_kib:.1f}\n")
        f.write(f"- copy_fetch_kib: {fc_kib:.1f}\n")
        f.write(f"- copy_write_kib: {wc_kib:.1f}\n")
        f.write(f"- copy_bytes: {COPY_CALIB_BYTES}\n")
        f.write(f"- fetch_scale: {f_scale:.4f}\n")
        f.write(f"- write_scale: {w_scale:.4f}\n")
        f.write(f"- fetch_bytes_per_launch: {int(fetch_b)}\n")
        f.write(f"- write_bytes_per_launch: {int(write_b)}\n")
        f.write(f"- traffic_bytes_per_launch: {int(fetch_b + write_b)}\n")
        f.write(f"- algorithmic_bytes_per_launch: {algo}\n")
        f.write(f"- traffic_over_algorithmic: {(fetch_b + write_b) / algo:.4f}\n")
        f.write(f"- kernel_source_sha256: {kernel_source_sha256()}\n")
        f.write("- hash_of: the code of " + ", ".join(KERNEL_SOURCES)
                + " with comments and whitespace removed\n")
        # every kernel of the step, from the same two runs
        f.write("\nEvery kernel of the five-op step (same runs and scaling; each moves "
                f"{algo} algorithmic bytes per launch):\n\n")
        f.write("| kernel | fetch bytes | write bytes | traffic / algorithmic |\n")
        f.write("|---|---:|---:|---:|\n")
        for name in sorted(k for k in fetch if "kvx::k_" in k and k in write):
            fv, wv = fetch[name], write[name]
            fb = sorted(fv)[len(fv) // 2] * f_scale * 1024
            wb = sorted(wv)[len(wv) // 2] * w_scale * 1024
            short = name.split("(")[0].replace("void ", "").replace("kvx::", "")
            f.write(f"| `{short}` | {int(fb)} | {int(wb)} | {(fb + wb) / algo:.4f} |\n")
    print(open(out_path).read())


# ------------------------------------------------------ all workloads --

def all_configs(torch, kvx, wl, wdev, dev, stream, reps, cpu=True):
    """Time every op on every workload at full size (one JSON line each),
    beside a plain contiguous copy of the same bytes timed the same way and
    (cpu baseline leg) the oracle on a bounded host sample of the same
    workload."""
    import numpy as np
    import oracle
    nt = min(16, os.cpu_count() or 1)

    def d(a):
        return torch.from_numpy(a).to(dev)

    def host(t):
        """Host uint8 copy of a device tensor (one plane per row)."""
        return t.cpu().view(torch.uint8).numpy().reshape(t.shape[0], -1)

    def cpu_rate(run, nbytes, sample, budget_s=1.0):
        """Oracle GB/s (r+w) of `run` (one op on the host sample moving
        nbytes), repeated for about budget_s after one untimed call."""
        if not cpu:
            return None
        run(0)
        n, t0 = 0, time.perf_counter()
        while True:
            run(n + 1)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 100:
                break
        return {"GBps": round(nbytes * n / el / 1e9, 2), "threads": nt, "sample": sample}

    def lay_of(g):
        return kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)

    def timed(fn, n):
        """GPU time per launch: n launches captured in one graph, replayed, so
        host-side call overhead does not hide short kernels."""
        fn(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(n):
                fn(i + 1)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / n

    copy_rates = {}

    def copy_rate(nbytes, rot):
        """Plain contiguous copy (k_copy16) of nbytes / 2 bytes, graph-timed
        like the ops: `rot` disjoint slices rotated when the op rotates its
        requests (so neither finds its data in the MALL), copies above 4 GiB
        timed at 4 GiB.  GB/s counted r+w."""
        n = min(nbytes // 2, 4 << 30) // 16 * 16
        k = max(1, min(rot, (4 << 30) // max(n, 1)))
        if (n, k) not in copy_rates:
            a = torch.empty(n * k, dtype=torch.uint8, device=dev)
            b = torch.empty(n * k, dtype=torch.uint8, device=dev)
            wdev.fill_hash(a, 9, stream=stream)
            ms = timed(lambda i: wdev.copy_bytes(b[(i % k) * n:], a[(i % k) * n:], n,
                                                 stream=stream), max(8 * k, 32))
            copy_rates[(n, k)] = 2 * n / (ms * 1e-3) / 1e9
            del a, b
            torch.cuda.empty_cache()
        return copy_rates[(n, k)]

    def emit(cfg, op, ms, nbytes, note="", rot=1, oracle_cpu=None):
        gbps = nbytes / (ms * 1e-3) / 1e9
        cp = copy_rate(nbytes, rot)
        line = {"workload": cfg, "op": op, "ms": round(ms, 5),
                "bytes_rw": nbytes, "GBps": round(gbps, 1),
                "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                "plain_copy_GBps": round(cp, 1), "vs_plain_copy": round(gbps / cp, 3),
                "note": note}
        if oracle_cpu is not None:
            line["cpu_oracle"] = oracle_cpu
        print(json.dumps(line), flush=True)

    def pool_of(case, side, seed):
        g = case.geom
        t = torch.empty((g.planes, side.num_slots, g.row_bytes), dtype=torch.uint8, device=dev)
        wdev.fill_hash(t, seed, stream=stream)
        return t

    with torch.cuda.stream(stream):
        # 1: 128 tokens x 28 KiB, page 1, 1024-slot pools (fits in cache)
        c = wl.qwen15b_128tok_page1()
        g = c.geom
        A, B = pool_of(c, c.src, 1), pool_of(c, c.dst, 2)
        st = torch.empty(c.total_tokens * g.token_bytes, dtype=torch.uint8, device=dev)
        reqs = kvx.Requests(d(c.tok_off), c.total_tokens)
        ts, td = kvx.Table(d(c.src.pg_off), d(c.src.ids)), kvx.Table(d(c.dst.pg_off), d(c.dst.ids))
        lay = lay_of(g)
        nb = 2 * c.payload_bytes()
        R = g.row_bytes
        hA, hB = host(A), host(B)
        hst = np.zeros(c.total_tokens * g.token_bytes, np.uint8)
        smp = f"the whole request, {g.planes} planes"
        cpu_g = cpu_rate(lambda i: oracle.gather(list(hA), R, 1, 1024, R, c.tok_off, c.src.pg_off,
                                                 c.src.ids, hst, nt), nb, smp)
        cpu_s = cpu_rate(lambda i: oracle.scatter(hst, R, c.tok_off, c.dst.pg_off, c.dst.ids,
                                                  list(hB), R, 1, 1024, nt), nb, smp)
        emit(c.name, "gather", timed(lambda i: kvx.gather(lay, kvx.Pool(A, 1024), ts, reqs, st,
                                                         stream=stream), reps * 10), nb,
             "3.5 MiB request: launch-latency bound, cache resident", oracle_cpu=cpu_g)
        emit(c.name, "scatter", timed(lambda i: kvx.scatter(lay, st, reqs, kvx.Pool(B, 1024), td,
                                                           stream=stream), reps * 10), nb,
             "launch-latency bound", oracle_cpu=cpu_s)
        del A, B, st
        torch.cuda.empty_cache()

        # 2: the bench request, each op alone, rotating 16 disjoint requests
        cs = [wl.kv144k_2048tok_page1(k) for k in range(NREQ)]
        g = cs[0].geom
        A, B = pool_of(cs[0], cs[0].src, 1), pool_of(cs[0], cs[0].dst, 2)
        st = torch.empty(2048 * g.token_bytes, dtype=torch.uint8, device=dev)
        reqs = kvx.Requests(d(cs[0].tok_off), 2048)
        tabs = [(kvx.Table(d(c.src.pg_off), d(c.src.ids)), kvx.Table(d(c.dst.pg_off),
                                                                      d(c.dst.ids)))
                for c in cs]
        lay = lay_of(g)
        PA, PB = kvx.Pool(A, 32768), kvx.Pool(B, 32768)
        nb = 2 * cs[0].payload_bytes()
        k, R = 8, g.row_bytes
        pa, pb = list(host(A[:k])), list(host(B[:k]))
        hst = np.zeros(2048 * k * R, np.uint8)
        nbk = 2 * 2048 * k * R
        smp = f"{k} of {g.planes} planes, the 16 requests rotated"
        cpu_gs = cpu_rate(lambda i: oracle.gather_scatter(
            pa, R, 1, 32768, cs[i % NREQ].src.pg_off, cs[i % NREQ].src.ids, R, cs[0].tok_off, pb, R,
            1, 32768, cs[i % NREQ].dst.pg_off, cs[i % NREQ].dst.ids, nt), nbk, smp)
        cpu_g = cpu_rate(lambda i: oracle.gather(
            pa, R, 1, 32768, R, cs[0].tok_off, cs[i % NREQ].src.pg_off, cs[i % NREQ].src.ids, hst,
            nt), nbk, smp)
        cpu_s = cpu_rate(lambda i: oracle.scatter(
            hst, R, cs[0].tok_off, cs[i % NREQ].dst.pg_off, cs[i % NREQ].dst.ids, pb, R, 1, 32768,
            nt), nbk, smp)
        del pa, pb, hst
        emit(cs[0].name, "gather_scatter", timed(lambda i: kvx.gather_scatter(
            lay, PA, tabs[i % NREQ][0], reqs, PB, tabs[i % NREQ][1], stream=stream), reps * 4), nb,
             rot=NREQ, oracle_cpu=cpu_gs)
        emit(cs[0].name, "gather", timed(lambda i: kvx.gather(
            lay, PA, tabs[i % NREQ][0], reqs, st, stream=stream), reps * 4), nb, rot=NREQ,
             oracle_cpu=cpu_g)
        emit(cs[0].name, "scatter", timed(lambda i: kvx.scatter(
            lay, st, reqs, PB, tabs[i % NREQ][1], stream=stream), reps * 4), nb, rot=NREQ,
             oracle_cpu=cpu_s)
        del A, B, st, PA, PB
        torch.cuda.empty_cache()

        # 2, token-major pools: plane q of slot s at (s * Q + q) * R, so a
        # slot's rows of all planes are one 144 KiB run (token-major chunk order)
        Q = g.planes
        A = torch.empty((32768, Q, R), dtype=torch.uint8, device=dev)
        B = torch.empty((32768, Q, R), dtype=torch.uint8, device=dev)
        wdev.fill_hash(A, 1, stream=stream)
        wdev.fill_hash(B, 2, stream=stream)
        st = torch.empty(2048 * g.token_bytes, dtype=torch.uint8, device=dev)
        PA = kvx.Pool([A.data_ptr() + q * R for q in range(Q)], 32768, 1, slot_stride=Q * R,
                      keep=A)
        PB = kvx.Pool([B.data_ptr() + q * R for q in range(Q)], 32768, 1, slot_stride=Q * R,
                      keep=B)
        hA, hB = A.cpu().numpy().reshape(-1), B.cpu().numpy().reshape(-1)
        pa, pb = [hA[q * R:] for q in range(k)], [hB[q * R:] for q in range(k)]
        hst = np.zeros(2048 * k * R, np.uint8)
        smp = f"{k} of {Q} planes, the 16 requests rotated"
        cpu_gs = cpu_rate(lambda i: oracle.gather_scatter(
            pa, Q * R, 1, 32768, cs[i % NREQ].src.pg_off, cs[i % NREQ].src.ids, R, cs[0].tok_off,
            pb, Q * R, 1, 32768, cs[i % NREQ].dst.pg_off, cs[i % NREQ].dst.ids, nt), nbk, smp)
        cpu_g = cpu_rate(lambda i: oracle.gather(
            pa, Q * R, 1, 32768, R, cs[0].tok_off, cs[i % NREQ].src.pg_off, cs[i % NREQ].src.ids,
            hst, nt), nbk, smp)
        cpu_s = cpu_rate(lambda i: oracle.scatter(
            hst, R, cs[0].tok_off, cs[i % NREQ].dst.pg_off, cs[i % NREQ].dst.ids, pb, Q * R, 1,
            32768, nt), nbk, smp)
        del pa, pb, hA, hB, hst
        name = "kv144k_2048tok_page1_token_major"
        emit(name, "gather_scatter", timed(lambda i: kvx.gather_scatter(
            lay, PA, tabs[i % NREQ][0], reqs, PB, tabs[i % NREQ][1], stream=stream), reps * 4), nb,
             "token-major pools (a slot's 72 rows contiguous)", rot=NREQ, oracle_cpu=cpu_gs)
        emit(name, "gather", timed(lambda i: kvx.gather(
            lay, PA, tabs[i % NREQ][0], reqs, st, stream=stream), reps * 4), nb,
             "token-major pool", rot=NREQ, oracle_cpu=cpu_g)
        emit(name, "scatter", timed(lambda i: kvx.scatter(
            lay, st, reqs, PB, tabs[i % NREQ][1], stream=stream), reps * 4), nb,
             "token-major pool", rot=NREQ, oracle_cpu=cpu_s)
        del A, B, st, PA, PB
        torch.cuda.empty_cache()

        # 3: 32 fragmented requests, one batched gather
        c = wl.kv144k_32req_fragmented()
        g = c.geom
        A = pool_of(c, c.src, 1)
        st = torch.empty(c.total_tokens * g.token_bytes, dtype=torch.uint8, device=dev)
        reqs = kvx.Requests(d(c.tok_off), c.total_tokens)
        ts = kvx.Table(d(c.src.pg_off), d(c.src.ids))
        k, R = 8, g.row_bytes
        pa = list(host(A[:k]))
        hst = np.zeros(c.total_tokens * k * R, np.uint8)
        cpu_g = cpu_rate(lambda i: oracle.gather(pa, R, 1, c.src.num_slots, R, c.tok_off,
                                                 c.src.pg_off, c.src.ids, hst, nt),
                         2 * c.total_tokens * k * R, f"{k} of {g.planes} planes, all 32 requests")
        del pa, hst
        emit(c.name, "gather", timed(lambda i: kvx.gather(lay_of(g), kvx.Pool(A, c.src.num_slots),
                                                         ts, reqs, st, stream=stream), reps),
             2 * c.payload_bytes(), f"{c.num_reqs} requests, {c.total_tokens} tokens",
             oracle_cpu=cpu_g)
        del A, st
        torch.cuda.empty_cache()

        # 4: HF permutes, seq 1024 and 8192 (two buffer sets alternate)
        for seq in (1024, 8192):
            c = wl.qwen7b_permute(seq)
            g = c.geom
            lay = lay_of(g)
            hf = [torch.empty((g.planes, g.kv_heads * seq * g.head_bytes), dtype=torch.uint8,
                              device=dev) for _ in range(2)]
            fl = [torch.empty(g.planes * seq * g.row_bytes, dtype=torch.uint8, device=dev)
                  for _ in range(2)]
            for t in hf + fl:
                wdev.fill_hash(t, 3, stream=stream)
            nb = 2 * c.payload_bytes()
            k, H, Db = 8, g.kv_heads, g.head_bytes
            hh = list(host(hf[0][:k]))
            hfl = np.zeros(k * seq * g.row_bytes, np.uint8)
            nbk = 2 * k * seq * g.row_bytes
            smp = f"{k} of {g.planes} planes"
            cpu_e = cpu_rate(lambda i: oracle.extract_permute(hh, H, Db, seq, seq, hfl, nt), nbk,
                             smp)
            cpu_r = cpu_rate(lambda i: oracle.rebuild_permute(hfl, H, Db, seq, hh, seq, nt), nbk,
                             smp)
            del hh, hfl
            emit(c.name, "extract", timed(lambda i: kvx.extract_permute(
                lay, hf[i % 2], seq, seq, fl[i % 2], stream=stream), reps * 4), nb, rot=2,
                 oracle_cpu=cpu_e)
            emit(c.name, "rebuild", timed(lambda i: kvx.rebuild_permute(
                lay, fl[i % 2], seq, hf[i % 2], seq, stream=stream), reps * 4), nb, rot=2,
                 oracle_cpu=cpu_r)
            del hf, fl
            torch.cuda.empty_cache()

        # MLA single-plane pools, 1152-byte rows, page 1 and page 16
        for page in (1, 16):
            cs = [wl.mla_case(page, k) for k in range(NREQ)]
            c = cs[0]
            g = c.geom
            A, B = pool_of(c, c.src, 1), pool_of(c, c.dst, 2)
            st = torch.empty(c.total_tokens * g.token_bytes, dtype=torch.uint8, device=dev)
            reqs = kvx.Requests(d(c.tok_off), c.total_tokens)
            tabs = [(kvx.Table(d(x.src.pg_off), d(x.src.ids)),
                     kvx.Table(d(x.dst.pg_off), d(x.dst.ids))) for x in cs]
            lay = lay_of(g)
            PA, PB = kvx.Pool(A, c.src.num_pages, page), kvx.Pool(B, c.dst.num_pages, page)
            nb = 2 * c.payload_bytes()
            R = g.row_bytes
            pa, pb = list(host(A)), list(host(B))
            hst = np.zeros(c.total_tokens * g.token_bytes, np.uint8)
            smp = f"all {g.planes} planes, the 16 requests rotated"
            cpu_gs = cpu_rate(lambda i: oracle.gather_scatter(
                pa, R, page, c.src.num_pages, cs[i % NREQ].src.pg_off, cs[i % NREQ].src.ids, R,
                c.tok_off, pb, R, page, c.dst.num_pages, cs[i % NREQ].dst.pg_off,
                cs[i % NREQ].dst.ids, nt), nb, smp)
            cpu_g = cpu_rate(lambda i: oracle.gather(
                pa, R, page, c.src.num_pages, R, c.tok_off, cs[i % NREQ].src.pg_off,
                cs[i % NREQ].src.ids, hst, nt), nb, smp)
            del pa, pb, hst
            emit(c.name, "gather_scatter", timed(lambda i: kvx.gather_scatter(
                lay, PA, tabs[i % NREQ][0], reqs, PB, tabs[i % NREQ][1], stream=stream),
                reps * 8), nb, "16 disjoint requests rotated", rot=NREQ, oracle_cpu=cpu_gs)
            emit(c.name, "gather", timed(lambda i: kvx.gather(
                lay, PA, tabs[i % NREQ][0], reqs, st, stream=stream), reps * 8), nb,
                 "16 disjoint requests rotated", rot=NREQ, oracle_cpu=cpu_g)
            del A, B, st, PA, PB
            torch.cuda.empty_cache()

        # head-sliced: P at TP=1 (8 heads, HND page 16) -> two D ranks at TP=2
        c = wl.hetero_tp_case()
        D, B = c.geom.head_dim, c.src.page_size
        Db = c.geom.head_bytes
        A = torch.empty((c.geom.planes, c.src.num_pages * B * 8 * Db), dtype=torch.uint8,
                        device=dev)
        Ds = [torch.empty((c.geom.planes, c.dst.num_pages * B * 4 * Db), dtype=torch.uint8,
                          device=dev) for _ in range(2)]
        for t in [A] + Ds:
            wdev.fill_hash(t, 5, stream=stream)
        reqs = kvx.Requests(d(c.tok_off), c.total_tokens)
        ts, td = kvx.Table(d(c.src.pg_off), d(c.src.ids)), kvx.Table(d(c.dst.pg_off), d(c.dst.ids))
        lay = lay_of(c.geom)
        PA = kvx.Pool(A, c.src.num_pages, B, slot_stride=8 * Db)
        PD = [kvx.Pool(t, c.dst.num_pages, B, slot_stride=4 * Db) for t in Ds]
        k = 8
        pa, pd = list(host(A[:k])), list(host(Ds[0][:k]))
        cpu_h = cpu_rate(lambda i: oracle.gather_scatter_heads(
            pa, 8 * Db, B, c.src.num_pages, c.src.pg_off, c.src.ids, (8, 4 * (i % 2), 1), Db, 4,
            c.tok_off, pd, 4 * Db, B, c.dst.num_pages, c.dst.pg_off, c.dst.ids, (4, 0, 1), nt),
            2 * c.total_tokens * k * 4 * Db, f"{k} of {c.geom.planes} planes")
        del pa, pd
        emit(c.name, "gather_scatter_heads", timed(lambda i: kvx.gather_scatter_heads(
            lay, PA, ts, kvx.Heads(8, 4 * (i % 2), "hnd"), reqs, PD[i % 2], td,
            kvx.Heads(4, 0, "hnd"), stream=stream), reps * 2), 2 * c.payload_bytes(),
             f"{c.num_reqs} requests, {c.total_tokens} tokens, 4 of 8 heads per launch", rot=2,
             oracle_cpu=cpu_h)
        del A, Ds, PA, PD
        torch.cuda.empty_cache()

        # 5: 64 requests, page-16 block pools of 36 GiB, one gather-scatter
        c = wl.kv144k_64req_page16()
        g = c.geom
        A, B = pool_of(c, c.src, 1), pool_of(c, c.dst, 2)
        reqs = kvx.Requests(d(c.tok_off), c.total_tokens)
        ts, td = kvx.Table(d(c.src.pg_off), d(c.src.ids)), kvx.Table(d(c.dst.pg_off), d(c.dst.ids))
        k, R = 4, g.row_bytes
        pa, pb = list(host(A[:k])), list(host(B[:k]))
        cpu_gs = cpu_rate(lambda i: oracle.gather_scatter(
            pa, R, 16, c.src.num_pages, c.src.pg_off, c.src.ids, R, c.tok_off, pb, R, 16,
            c.dst.num_pages, c.dst.pg_off, c.dst.ids, nt), 2 * c.total_tokens * k * R,
            f"{k} of {g.planes} planes, all 64 requests")
        del pa, pb
        emit(c.name, "gather_scatter", timed(lambda i: kvx.gather_scatter(
            lay_of(g), kvx.Pool(A, c.src.num_pages, 16), ts, reqs, kvx.Pool(B, c.dst.num_pages, 16),
            td, stream=stream), reps), 2 * c.payload_bytes(),
             f"{c.num_reqs} requests, {c.total_tokens} tokens, page 16", oracle_cpu=cpu_gs)
        del A, B
        torch.cuda.empty_cache()


# ----------------------------------------------- load and comparators --

def concurrent_load(torch, kvx, wl, wdev, dev, reps=32):
    """Gather-scatter of the 2048-token request while a decode-like reader
    streams a 16 GiB buffer on a second stream (both default priority), at
    three reader intensities (workgroups per launch)."""
    wk_stream = torch.cuda.Stream(device=dev)
    rd_stream = torch.cuda.Stream(device=dev)
    wk = Workload(torch, kvx, wl, wdev, dev, wk_stream)
    rd_buf = torch.empty(16 * 2 ** 30, dtype=torch.uint8, device=dev)
    wdev.fill_hash(rd_buf, 9, stream=rd_stream)
    sink = torch.zeros(2048, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def run_gs(n):
        e0, e1 = ev(), ev()
        e0.record(wk_stream)
        for i in range(n):
            k = i % NREQ
            kvx.gather_scatter(wk.lay, wk.PA, wk.src_tabs[k], wk.reqs, wk.PB, wk.dst_tabs[k],
                               stream=wk_stream)
        e1.record(wk_stream)
        return e0, e1

    def run_reader(n, blocks):
        e0, e1 = ev(), ev()
        e0.record(rd_stream)
        for _ in range(n):
            wdev.read_stream(rd_buf, sink, blocks=blocks, stream=rd_stream)
        e1.record(rd_stream)
        return e0, e1

    def gbps(nbytes, e):
        return nbytes / (e[0].elapsed_time(e[1]) * 1e6)

    for _ in range(8):                                   # warm up clocks and caches
        run_gs(4)
    torch.cuda.synchronize()
    eg = run_gs(reps)
    torch.cuda.synchronize()
    result = {"gather_scatter_alone_GBps": round(gbps(wk.op_bytes * reps, eg), 1),
              "readers": []}
    for blocks in (2048, 256, 64):
        er = run_reader(2, blocks)
        torch.cuda.synchronize()
        alone = gbps(rd_buf.numel() * 2, er)
        # enough reader launches to outlast the gather-scatter launches even
        # if those slow down to 0.2 TB/s
        launch_ms = rd_buf.numel() / (alone * 1e6)
        n_rd = int(wk.op_bytes * reps / 0.2e12 * 1e3 / launch_ms) + 2
        er = run_reader(n_rd, blocks)
        eg = run_gs(reps)
        torch.cuda.synchronize()
        result["readers"].append({
            "reader_blocks": blocks,
            "reader_alone_GBps": round(alone, 1),
            "reader_loaded_GBps": round(gbps(rd_buf.numel() * n_rd, er), 1),
            "gather_scatter_loaded_GBps": round(gbps(wk.op_bytes * reps, eg), 1),
            "reader_outlasts_gather_scatter": bool(er[0].elapsed_time(er[1]) >=
                                                   eg[0].elapsed_time(eg[1]))})
    result["note"] = ("reader: 16 GiB per launch, nontemporal 16-byte loads, 256-thread "
                      "workgroups; gather-scatter: the 2048-token, 144 KiB/token request, 16 "
                      "disjoint requests rotated; GB/s counts bytes read + written")
    print(json.dumps(result), flush=True)


def cu_split(torch, kvx, wl, wdev, dev, reps=32):
    """The compute units split between the transfer and a full-intensity
    decode-like reader: each on a stream with its own CU mask
    (hipExtStreamCreateWithCUMask).  Mask bit i selects a CU on XCD i mod 8,
    and a mask that leaves an XCD without CUs is refused ("out of memory":
    workgroups are dealt to every XCD), so both sides take whole groups of 8
    consecutive bits -- one CU on each XCD per group -- the transfer every
    m-th group and the reader the rest.  The pair of streams is created
    before any other stream and destroyed before the next split."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    words = (ncu + 31) // 32

    def masked_stream(cus):
        mask = (ctypes.c_uint32 * words)()
        for c in cus:
            mask[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), words, mask)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask returned {rc}")
        return h, torch.cuda.ExternalStream(h.value, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def gbps(nbytes, e):
        return nbytes / (e[0].elapsed_time(e[1]) * 1e6)

    result = {"splits": []}
    wk = rd_buf = sink = None
    for m in (8, 4, 2):                      # transfer on 1/8, 1/4, 1/2 of the CUs
        t_cus = [c for c in range(ncu) if (c // 8) % m == 0]
        r_cus = [c for c in range(ncu) if (c // 8) % m != 0]
        ht, ts = masked_stream(t_cus)
        hr, rs = masked_stream(r_cus)
        try:
            if wk is None:                   # buffers filled on the first masked stream
                wk = Workload(torch, kvx, wl, wdev, dev, ts)
                rd_buf = torch.empty(16 * 2 ** 30, dtype=torch.uint8, device=dev)
                wdev.fill_hash(rd_buf, 9, stream=ts)
                sink = torch.zeros(2048, dtype=torch.int64, device=dev)
                torch.cuda.synchronize()

            def gs_on(st, n):
                e0, e1 = ev(), ev()
                e0.record(st)
                for i in range(n):
                    k = i % NREQ
                    kvx.gather_scatter(wk.lay, wk.PA, wk.src_tabs[k], wk.reqs, wk.PB,
                                       wk.dst_tabs[k], stream=st)
                e1.record(st)
                return e0, e1

            def rd_on(st, n):
                e0, e1 = ev(), ev()
                e0.record(st)
                for _ in range(n):
                    wdev.read_stream(rd_buf, sink, blocks=2048, stream=st)
                e1.record(st)
                return e0, e1

            gs_on(ts, 8)
            torch.cuda.synchronize()
            eg = gs_on(ts, reps)
            torch.cuda.synchronize()
            g_alone = gbps(wk.op_bytes * reps, eg)
            er = rd_on(rs, 2)
            torch.cuda.synchronize()
            r_alone = gbps(rd_buf.numel() * 2, er)
            # enough reader launches to outlast the transfer at half its rate
            n_rd = int(wk.op_bytes * reps / (0.5 * g_alone) / (rd_buf.numel() / r_alone)) + 2
            er = rd_on(rs, n_rd)
            eg = gs_on(ts, reps)
            torch.cuda.synchronize()
            result["splits"].append({
                "transfer_cus": len(t_cus), "reader_cus": len(r_cus),
                "gather_scatter_alone_GBps": round(g_alone, 1),
                "reader_alone_GBps": round(r_alone, 1),
                "gather_scatter_loaded_GBps": round(gbps(wk.op_bytes * reps, eg), 1),
                "reader_loaded_GBps": round(gbps(rd_buf.numel() * n_rd, er), 1),
                "reader_outlasts_gather_scatter": bool(er[0].elapsed_time(er[1]) >=
                                                       eg[0].elapsed_time(eg[1]))})
            log(f"cu split {len(t_cus)}/{len(r_cus)}: {result['splits'][-1]}")
        finally:
            torch.cuda.synchronize()
            hip.hipStreamDestroy(ht)
            hip.hipStreamDestroy(hr)
    result["note"] = ("transfer: gather-scatter of the 2048-token, 144 KiB/token request, 16 "
                      "disjoint requests rotated; reader: 16 GiB per launch, nontemporal "
                      "16-byte loads, 2048 workgroups of 256 threads; each on its own CU "
                      "mask; GB/s counts bytes read + written")
    print(json.dumps(result), flush=True)


def graph_timed(torch, stream, fn, n):
    """Milliseconds per call of fn(i), i = 1..n, captured in one graph on
    `stream` and replayed once after a warm replay (fn(0) runs eagerly
    first)."""
    fn(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(n):
            fn(i + 1)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):        # replay runs on the current stream
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def request_sizes(torch, kvx, wl, wdev, dev, stream):
    """Gather-scatter and gather of one request of n tokens at 144 KiB/token
    (page-1 pools of 65536 slots, slots from seeded permutations, 8 disjoint
    requests rotated), n from 16 to 8192, graph-timed, beside a plain
    contiguous copy of the same bytes: where per-launch latency gives way to
    bandwidth."""
    import numpy as np
    g = wl.KV144K
    Q, R, NS = g.planes, g.row_bytes, 65536
    rng = np.random.default_rng(1010)
    pa, pb = rng.permutation(NS), rng.permutation(NS)
    A = torch.empty((Q, NS, R), dtype=torch.uint8, device=dev)
    B = torch.empty_like(A)
    wdev.fill_hash(A, 1, stream=stream)
    wdev.fill_hash(B, 2, stream=stream)
    lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
    PA, PB = kvx.Pool(A, NS), kvx.Pool(B, NS)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    for n in (16, 64, 256, 1024, 2048, 4096, 8192):
        reqs = kvx.Requests(d(np.array([0, n], np.int64)), n)
        pg = d(np.array([0, n], np.int64))
        tabs = [(kvx.Table(pg, d(pa[k * n:(k + 1) * n].astype(np.int32))),
                 kvx.Table(pg, d(pb[k * n:(k + 1) * n].astype(np.int32)))) for k in range(8)]
        st = torch.empty(n * Q * R, dtype=torch.uint8, device=dev)
        cp = torch.empty_like(st)
        reps = 64 if n <= 1024 else 16
        nb = 2 * n * Q * R
        line = {"tokens": n, "bytes_rw": nb}
        for op, fn in (("gather_scatter", lambda i: kvx.gather_scatter(
                           lay, PA, tabs[i % 8][0], reqs, PB, tabs[i % 8][1], stream=stream)),
                       ("gather", lambda i: kvx.gather(lay, PA, tabs[i % 8][0], reqs, st,
                                                       stream=stream)),
                       ("plain_copy", lambda i: wdev.copy_bytes(cp, st, st.numel(),
                                                                stream=stream))):
            ms = graph_timed(torch, stream, fn, reps)
            line[op] = {"us": round(ms * 1e3, 2), "GBps": round(nb / (ms * 1e6), 1)}
        print(json.dumps(line), flush=True)
        del st, cp


def batch_sizes(torch, kvx, wl, wdev, dev, stream):
    """Gather and gather-scatter of 49152 tokens at 144 KiB/token (page-1
    pools of 65536 slots, slots from seeded permutations) split into 1 to
    49152 requests: equal lengths, and at 1024 and 4096 requests exponential
    lengths with empty requests among them.  Graph-timed.  Batches above 64
    requests take the kernels with the 64-way request search."""
    import numpy as np
    g = wl.KV144K
    Q, R, NS, T = g.planes, g.row_bytes, 65536, 49152
    rng = np.random.default_rng(2020)
    pa, pb = rng.permutation(NS)[:T], rng.permutation(NS)[:T]
    A = torch.empty((Q, NS, R), dtype=torch.uint8, device=dev)
    B = torch.empty_like(A)
    wdev.fill_hash(A, 1, stream=stream)
    wdev.fill_hash(B, 2, stream=stream)
    st = torch.empty(T * Q * R, dtype=torch.uint8, device=dev)
    lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
    PA, PB = kvx.Pool(A, NS), kvx.Pool(B, NS)
    nb = 2 * T * Q * R

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def exp_lengths(n):
        w = rng.exponential(1.0, n) * (rng.random(n) > 0.1)
        w[-1] = max(w[-1], 1.0)
        lens = np.floor(w / w.sum() * T).astype(np.int64)
        lens[-1] += T - lens.sum()
        return lens

    cases = [(n, "equal") for n in (1, 16, 64, 65, 256, 1024, 4096, 16384, 49152)]
    cases += [(1024, "exponential"), (4096, "exponential")]
    for n, mix in cases:
        if mix == "equal":
            lens = np.full(n, T // n, np.int64)
            lens[:T - lens.sum()] += 1
        else:
            lens = exp_lengths(n)
        tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        reqs = kvx.Requests(d(tok), T)
        ts = kvx.Table(d(tok), d(pa.astype(np.int32)))
        td = kvx.Table(d(tok), d(pb.astype(np.int32)))
        line = {"requests": n, "lengths": mix, "tokens": T, "bytes_rw": nb,
                "empty": int((lens == 0).sum())}
        for op, fn in (("gather", lambda i: kvx.gather(lay, PA, ts, reqs, st, stream=stream)),
                       ("gather_scatter", lambda i: kvx.gather_scatter(lay, PA, ts, reqs, PB, td,
                                                                       stream=stream))):
            ms = graph_timed(torch, stream, fn, 8)
            line[op] = {"us": round(ms * 1e3, 1), "GBps": round(nb / (ms * 1e6), 1)}
        print(json.dumps(line), flush=True)
    del A, B, st


def row_sizes(torch, kvx, wl, wdev, dev, stream):
    """Gather-scatter, gather and scatter of about 256 MiB each way at page 1
    (random slots from seeded permutations, one request, four disjoint tables
    rotated so that no launch finds its rows in the 256 MiB MALL) for rows of
    256 B to 16 KiB: the flat, row-loop and wide copies, each beside a plain
    contiguous copy of the same bytes.  Graph-timed."""
    import numpy as np
    target = 256 << 20
    # (layers, kv_heads, head_dim, dtype): rows of H * D * 2 bytes, 2 planes a layer
    shapes = [(28, 1, 128, "bf16"), (28, 2, 128, "bf16"), (28, 4, 128, "bf16"),
              (27, 1, 576, "bf16"), (28, 6, 128, "bf16"), (36, 8, 128, "bf16"),
              (16, 16, 128, "bf16"), (8, 32, 128, "bf16"), (4, 64, 128, "bf16")]
    for L, H, D, dt in shapes:
        g = wl.Geometry(L, 2 if D != 576 else 1, H, D, dt)
        Q, R = g.planes, g.row_bytes
        T = max(64, target // (Q * R))
        NS = 4 * T + 64
        A = torch.empty((Q, NS, R), dtype=torch.uint8, device=dev)
        B = torch.empty_like(A)
        wdev.fill_hash(A, 1, stream=stream)
        wdev.fill_hash(B, 2, stream=stream)
        st = torch.empty(T * Q * R, dtype=torch.uint8, device=dev)
        cp = torch.empty_like(st)
        rng = np.random.default_rng(3030 + R)
        tok = np.array([0, T], np.int64)

        def d(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        reqs = kvx.Requests(d(tok), T)
        ps, pd = rng.permutation(NS), rng.permutation(NS)
        tabs = [(kvx.Table(d(tok), d(ps[k * T:(k + 1) * T].astype(np.int32))),
                 kvx.Table(d(tok), d(pd[k * T:(k + 1) * T].astype(np.int32)))) for k in range(4)]
        lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
        PA, PB = kvx.Pool(A, NS), kvx.Pool(B, NS)
        nb = 2 * T * Q * R
        line = {"row_bytes": R, "planes": Q, "tokens": T, "bytes_rw": nb}
        for op, fn in (("gather_scatter", lambda i: kvx.gather_scatter(
                           lay, PA, tabs[i % 4][0], reqs, PB, tabs[i % 4][1], stream=stream)),
                       ("gather", lambda i: kvx.gather(lay, PA, tabs[i % 4][0], reqs, st,
                                                       stream=stream)),
                       ("scatter", lambda i: kvx.scatter(lay, st, reqs, PB, tabs[i % 4][1],
                                                         stream=stream)),
                       ("plain_copy", lambda i: wdev.copy_bytes(cp, st, st.numel(),
                                                                stream=stream))):
            ms = graph_timed(torch, stream, fn, 8)
            line[op] = {"us": round(ms * 1e3, 1), "GBps": round(nb / (ms * 1e6), 1)}
        print(json.dumps(line), flush=True)
        del A, B, st, cp, PA, PB
        torch.cuda.empty_cache()


# (name, mode bits of wdev.row_pattern): the access patterns of the paged ops
# on the 2048-token request's 72 x 2048 rows of 2 KiB, with no table read
PATTERNS = [("random source -> random destination (gather-scatter)", 15),
            ("random source -> contiguous (gather)", 7),
            ("contiguous -> random destination (scatter)", 11),
            ("contiguous -> contiguous (plain copy)", 3),
            ("random reads only", 5), ("random writes only", 10),
            ("contiguous reads only", 1), ("contiguous writes only", 2)]


def _pattern_rates(torch, wdev, A, B, Q, T, S, R, patterns, stream, rounds, n):
    """Median GB/s (r+w) of each (pattern, rows per wave) of wl_row_pattern."""
    sink = torch.zeros(2048, dtype=torch.int32, device=A.device)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    res = {}
    for _ in range(rounds):
        for name, mode in patterns:
            nbytes = Q * T * R * ((mode & 1) + ((mode >> 1) & 1))
            for K in (1, 2, 4):
                for i in range(4):
                    wdev.row_pattern(A, B, sink, Q, T, S, K, i % (S // T), mode, stream, R)
                ev[0].record(stream)
                for i in range(n):
                    wdev.row_pattern(A, B, sink, Q, T, S, K, i % (S // T), mode, stream, R)
                ev[1].record(stream)
                torch.cuda.synchronize()
                ms = ev[0].elapsed_time(ev[1]) / n
                res.setdefault((name, K), []).append(nbytes / (ms * 1e-3) / 1e9)
    rows = []
    for name, mode in patterns:
        row = {"pattern": name, "mode": mode}
        for K in (1, 2, 4):
            v = sorted(res[(name, K)])
            row[f"rows_per_wave_{K}_GBps"] = round(v[len(v) // 2], 1)
        rows.append(row)
        log(f"  {name:55s} " + "  ".join(f"{row[f'rows_per_wave_{K}_GBps']:7.1f}" for K in (1, 2, 4)))
    return rows


def row_patterns(torch, kvx, wl, wdev, dev, stream, rounds=3, n=32):
    """The 2048-token request's access patterns moved by a table-free kernel
    (wl_row_pattern: each row's slot a bijective hash of its token, 16
    disjoint slot sets rotated, in the same two 4.5 GiB pools), 1, 2 and 4
    rows per wave, beside the library's ops timed alone in the same process:
    what the patterns cost by themselves, against what the paged kernels with
    their table reads achieve.  Then the same for the MLA request (27 planes
    of 1152-byte rows, 2048 tokens, 32768-slot page-1 pools)."""
    wk = Workload(torch, kvx, wl, wdev, dev, stream)
    Q, T, S = wk.Q, wk.T, wk.S
    torch.cuda.synchronize()
    pats = _pattern_rates(torch, wdev, wk.A, wk.B, Q, T, S, wk.R, PATTERNS, stream, rounds, n)
    iso = time_isolated(torch, wk, stream)
    del wk
    torch.cuda.empty_cache()
    # MLA: the library's gather-scatter, gather and scatter of 16 disjoint
    # requests rotated, and the same rows without tables
    cs = [wl.mla_case(1, k) for k in range(NREQ)]
    c, g = cs[0], cs[0].geom
    Qm, Rm, Sm = g.planes, g.row_bytes, c.src.num_slots
    A = torch.zeros((Qm, Sm, Rm), dtype=torch.uint8, device=dev)
    B = torch.zeros((Qm, Sm, Rm), dtype=torch.uint8, device=dev)
    d = lambda a: torch.from_numpy(a).to(dev)
    reqs = kvx.Requests(d(c.tok_off), c.total_tokens)
    tabs = [(kvx.Table(d(x.src.pg_off), d(x.src.ids)), kvx.Table(d(x.dst.pg_off), d(x.dst.ids)))
            for x in cs]
    lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
    PA, PB = kvx.Pool(A, c.src.num_pages), kvx.Pool(B, c.dst.num_pages)
    st = torch.empty(c.total_tokens * g.token_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    mla_ops = {
        "gather_scatter": lambda i: kvx.gather_scatter(lay, PA, tabs[i % NREQ][0], reqs, PB,
                                                       tabs[i % NREQ][1], stream=stream),
        "gather": lambda i: kvx.gather(lay, PA, tabs[i % NREQ][0], reqs, st, stream=stream),
        "scatter": lambda i: kvx.scatter(lay, st, reqs, PB, tabs[i % NREQ][1], stream=stream)}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    mla_lib = {}
    for _ in range(rounds):
        for op, fn in mla_ops.items():
            for i in range(4):
                fn(i)
            ev[0].record(stream)
            for i in range(n):
                fn(i)
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / n
            mla_lib.setdefault(op, []).append(2 * c.payload_bytes() / (ms * 1e-3) / 1e9)
    mla_lib = {op: round(sorted(v)[len(v) // 2], 1) for op, v in mla_lib.items()}
    log(f"  MLA library ops: {mla_lib}")
    mla_pats = _pattern_rates(torch, wdev, A, B, Qm, c.total_tokens, Sm, Rm, PATTERNS[:3] +
                              PATTERNS[4:6], stream, rounds, n)
    out = {"row_patterns": pats,
           "library_ops_alone_GBps": {op: iso[op]["GBps"] for op in OPS},
           "mla_row_patterns": mla_pats, "library_mla_ops_GBps": mla_lib,
           "note": "rates count bytes read + written; a pattern launch moves the request's "
                   "rows: 72 x 2048 of 2 KiB (302 MB each way it reads or writes), or for "
                   "MLA 27 x 2048 of 1152 bytes (64 MB each way); the library's ops are "
                   "launched back to back on rotated requests, nothing reading their output"}
    print(json.dumps(out), flush=True)


# ------------------------------------------------------- DRAM-page probe --
#
# HBM serves a row fastest when other rows on the same DRAM page arrive with
# it.  The probe keeps the 2048-token request's size and density (2048 of the
# 32768 slots of each page-1 pool, 2 KiB rows) and varies only where the
# slots lie: in pairs at a fixed distance, the partner a fixed number of
# tokens later, on one side or both, or as runs of B slots (pages of a
# block-paged pool written as page-1 tables) in their natural token order or
# with the rows 32 KiB apart made adjacent.

DRAM_SEG = 32 << 10        # bytes between rows that share a DRAM page (probe result)


def dram_page_sets(kind, arg, rng, slots=32768, tokens=2048, nsets=8, row_bytes=2048):
    """`nsets` pairwise disjoint slot lists of `tokens` entries each (one per
    rotated request), every slot in [0, slots):
      ("random", None)         a seeded permutation cut into pieces;
      ("sorted", None)         the same, each list sorted;
      ("pairs", (dist, gap))   slot pairs (s, s + dist) with s % (2 dist) < dist,
                               the partner `gap` tokens after its start;
      ("pages", (B, grouped))  runs of B slots at B-aligned starts; with
                               `grouped` the run's rows DRAM_SEG bytes apart are
                               consecutive in token order."""
    import numpy as np
    if kind in ("random", "sorted"):
        p = rng.permutation(slots)
        sets = [p[k * tokens:(k + 1) * tokens] for k in range(nsets)]
        return [np.sort(s) if kind == "sorted" else s for s in sets]
    if kind == "pairs":
        dist, gap = arg
        s = np.arange(slots)
        cand = s[(s % (2 * dist) < dist) & (s + dist < slots)]
        rng.shuffle(cand)
        half = tokens // 2
        out = []
        for k in range(nsets):
            st = cand[k * half:(k + 1) * half]
            ids = np.empty(tokens, np.int64)
            for b in range(0, half, gap):
                blk = st[b:b + gap]
                ids[2 * b:2 * b + len(blk)] = blk
                ids[2 * b + len(blk):2 * b + 2 * len(blk)] = blk + dist
            out.append(ids)
        return out
    if kind == "pages":
        B, grouped = arg
        per = tokens // B
        pages = rng.permutation(slots // B)
        within = np.arange(B)
        g = DRAM_SEG // row_bytes
        if grouped and B >= 2 * g and B % g == 0:
            within = within.reshape(B // g, g).T.reshape(-1)
        return [(pages[k * per:(k + 1) * per, None] * B + within[None, :]).reshape(-1)
                for k in range(nsets)]
    raise ValueError(kind)


# (label, source sets, destination sets)
DRAM_PAGE_DESIGNS = (
    [("random slots (the workload's tables)", ("random", None), ("random", None)),
     ("sorted slots", ("sorted", None), ("sorted", None))]
    + [(f"pairs {d * 2} KiB apart, adjacent tokens", ("pairs", (d, 1)), ("pairs", (d, 1)))
       for d in (4, 8, 12, 16, 24, 32, 48, 64)]
    + [(f"pairs 64 KiB apart, partner {j} tokens later", ("pairs", (32, j)),
        ("pairs", (32, j))) for j in (2, 4, 8, 16, 64, 1024)]
    + [("pairs 64 KiB apart in the source only", ("pairs", (32, 1)), ("random", None)),
       ("pairs 64 KiB apart in the destination only", ("random", None), ("pairs", (32, 1)))]
    + [(f"runs of {B} slots ({B * 2} KiB), {'grouped' if g else 'natural'} order",
        ("pages", (B, g)), ("pages", (B, g))) for B in (16, 32, 64) for g in (False, True)
       if B > 16 or not g])


def dram_pages(torch, kvx, wl, wdev, dev, stream, rounds=3, n=24):
    """Gather-scatter, gather and scatter of the 2048-token request over
    slot placements of equal density (DRAM_PAGE_DESIGNS), graph-timed, the
    designs alternating round by round in one process on the same two
    4.5 GiB pools; 8 disjoint requests rotated per design."""
    import numpy as np
    g = wl.KV144K
    Q, R, NS, T, NSETS = g.planes, g.row_bytes, 32768, 2048, 8
    A = torch.empty((Q, NS, R), dtype=torch.uint8, device=dev)
    Bt = torch.empty_like(A)
    wdev.fill_hash(A, 1, stream=stream)
    wdev.fill_hash(Bt, 2, stream=stream)
    st = torch.empty(T * Q * R, dtype=torch.uint8, device=dev)
    lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
    PA, PB = kvx.Pool(A, NS), kvx.Pool(Bt, NS)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tok = d(np.array([0, T], np.int64))
    reqs = kvx.Requests(tok, T)
    tabs = []
    for i, (label, sk, dk) in enumerate(DRAM_PAGE_DESIGNS):
        ss = dram_page_sets(*sk, np.random.default_rng(5100 + i), NS, T, NSETS, R)
        ds = dram_page_sets(*dk, np.random.default_rng(5900 + i), NS, T, NSETS, R)
        for x in ss + ds:
            if len(np.unique(x)) != T or x.min() < 0 or x.max() >= NS:
                raise AssertionError(f"{label}: bad slot list")
        tabs.append(([kvx.Table(tok, d(x.astype(np.int32))) for x in ss],
                      [kvx.Table(tok, d(x.astype(np.int32))) for x in ds]))
    torch.cuda.synchronize()
    nb = 2 * T * Q * R
    res = [{"gather_scatter": [], "gather": [], "scatter": []} for _ in DRAM_PAGE_DESIGNS]
    for rnd in range(rounds):
        for i, (sT, dT) in enumerate(tabs):
            fns = {"gather_scatter": lambda k: kvx.gather_scatter(
                       lay, PA, sT[k % NSETS], reqs, PB, dT[k % NSETS], stream=stream),
                   "gather": lambda k: kvx.gather(lay, PA, sT[k % NSETS], reqs, st,
                                                  stream=stream),
                   "scatter": lambda k: kvx.scatter(lay, st, reqs, PB, dT[k % NSETS],
                                                    stream=stream)}
            for op, fn in fns.items():
                res[i][op].append(nb / (graph_timed(torch, stream, fn, n) * 1e-3) / 1e9)
        log(f"dram-pages round {rnd + 1}/{rounds} done")
    rows = []
    for (label, sk, dk), r in zip(DRAM_PAGE_DESIGNS, res):
        row = {"design": label}
        for op, v in r.items():
            row[f"{op}_GBps"] = round(sorted(v)[len(v) // 2], 1)
        rows.append(row)
        log(f"  {label:55s} {row['gather_scatter_GBps']:7.1f} {row['gather_GBps']:7.1f} "
            f"{row['scatter_GBps']:7.1f}")
    # the same request in block pools (page_size B, random pages), where the
    # library pairs the rows that share DRAM pages once a page holds 64 KiB
    blocks = {B: {"gather_scatter": [], "gather": [], "scatter": []} for B in (16, 32, 64, 128)}
    btabs = {}
    for B in blocks:
        P, npg = NS // B, T // B
        rng = np.random.default_rng(6100 + B)
        ps, pd = rng.permutation(P), rng.permutation(P)
        pg = d(np.array([0, npg], np.int64))
        btabs[B] = (kvx.Pool(A, P, B), kvx.Pool(Bt, P, B),
                    [kvx.Table(pg, d(ps[k * npg:(k + 1) * npg].astype(np.int32)))
                     for k in range(NSETS)],
                    [kvx.Table(pg, d(pd[k * npg:(k + 1) * npg].astype(np.int32)))
                     for k in range(NSETS)])
    for rnd in range(rounds):
        for B, (pa, pb, sT, dT) in btabs.items():
            fns = {"gather_scatter": lambda k: kvx.gather_scatter(
                       lay, pa, sT[k % NSETS], reqs, pb, dT[k % NSETS], stream=stream),
                   "gather": lambda k: kvx.gather(lay, pa, sT[k % NSETS], reqs, st,
                                                  stream=stream),
                   "scatter": lambda k: kvx.scatter(lay, st, reqs, pb, dT[k % NSETS],
                                                    stream=stream)}
            for op, fn in fns.items():
                blocks[B][op].append(nb / (graph_timed(torch, stream, fn, n) * 1e-3) / 1e9)
    # the same bytes as pools whose blocks hold a layer's K and V pages
    # together ([L][blocks][2][B][R]; page stride 2 B R): from pages of
    # 32 KiB the library pairs the two planes of a token
    kvb = {B: {"gather_scatter": [], "gather": [], "scatter": []} for B in (8, 16, 32)}
    kvtabs = {}
    for B in kvb:
        nblk, npg, run = NS // B, T // B, B * R

        def kvpool(t, nblk=nblk, run=run, B=B):
            return kvx.Pool([t.data_ptr() + (q // 2) * nblk * 2 * run + (q % 2) * run
                             for q in range(Q)], nblk, B, slot_stride=R, page_stride=2 * run,
                            keep=t)
        rng = np.random.default_rng(6300 + B)
        ps, pd = rng.permutation(nblk), rng.permutation(nblk)
        pg = d(np.array([0, npg], np.int64))
        kvtabs[B] = (kvpool(A), kvpool(Bt),
                     [kvx.Table(pg, d(ps[k * npg:(k + 1) * npg].astype(np.int32)))
                      for k in range(NSETS)],
                     [kvx.Table(pg, d(pd[k * npg:(k + 1) * npg].astype(np.int32)))
                      for k in range(NSETS)])
    for rnd in range(rounds):
        for B, (pa, pb, sT, dT) in kvtabs.items():
            fns = {"gather_scatter": lambda k: kvx.gather_scatter(
                       lay, pa, sT[k % NSETS], reqs, pb, dT[k % NSETS], stream=stream),
                   "gather": lambda k: kvx.gather(lay, pa, sT[k % NSETS], reqs, st,
                                                  stream=stream),
                   "scatter": lambda k: kvx.scatter(lay, st, reqs, pb, dT[k % NSETS],
                                                    stream=stream)}
            for op, fn in fns.items():
                kvb[B][op].append(nb / (graph_timed(torch, stream, fn, n) * 1e-3) / 1e9)
    kvrows = []
    for B, r in kvb.items():
        row = {"page_size": B, "page_KiB": B * R // 1024, "planes_paired": B * R >= DRAM_SEG}
        for op, v in r.items():
            row[f"{op}_GBps"] = round(sorted(v)[len(v) // 2], 1)
        kvrows.append(row)
        log(f"  K/V block pool, page {B:3d}: {row['gather_scatter_GBps']:7.1f} "
            f"{row['gather_GBps']:7.1f} {row['scatter_GBps']:7.1f}")
    brows = []
    for B, r in blocks.items():
        row = {"page_size": B, "page_KiB": B * R // 1024,
               "paired": B * R >= 2 * DRAM_SEG}
        for op, v in r.items():
            row[f"{op}_GBps"] = round(sorted(v)[len(v) // 2], 1)
        brows.append(row)
        log(f"  block pool, page {B:3d}: {row['gather_scatter_GBps']:7.1f} "
            f"{row['gather_GBps']:7.1f} {row['scatter_GBps']:7.1f}")
    pa = pb = fns = None                      # the loops' last pools
    del A, Bt, st, PA, PB, tabs, btabs, kvtabs, pa, pb, fns
    torch.cuda.empty_cache()
    orders_64req = dram_pages_batch_orders(torch, kvx, wl, wdev, dev, stream, rounds)
    print(json.dumps({"dram_pages": rows, "block_pools": brows, "kv_block_pools": kvrows,
                      "kv144k_64req_page16_orders": orders_64req,
                      "note": "one request of 2048 tokens x 72 planes of 2 KiB rows (288 MiB "
                              "each way) in page-1 pools of 32768 slots (4.5 GiB each); every "
                              "design uses 2048 of the 32768 slots per request, only their "
                              "placement differs; 8 disjoint requests rotated, 24 launches per "
                              "graph, median of 3 rounds"}), flush=True)


def dram_pages_batch_orders(torch, kvx, wl, wdev, dev, stream, rounds=3, n=4):
    """The kv144k_64req_page16 batch (64 requests, page 16, two 36 GiB pools; half of each
    pool's pages in use) written as one page-1 request over the same source
    and destination slots, its tokens in batch order or sorted by destination
    slot, by destination DRAM page (the rows of one 128 KiB block's pages
    together) or by source DRAM page.  A gather-scatter's result does not
    depend on the order; graph-timed gather-scatter GB/s per order."""
    import numpy as np
    case = wl.kv144k_64req_page16()
    g = case.geom
    Q, R, B = g.planes, g.row_bytes, case.src.page_size
    NS, T = case.src.num_pages * B, case.total_tokens
    src_slot = np.empty(T, np.int64)
    dst_slot = np.empty(T, np.int64)
    for r in range(case.num_reqs):
        a, b = int(case.tok_off[r]), int(case.tok_off[r + 1])
        t = np.arange(b - a)
        src_slot[a:b] = case.src.ids[case.src.pg_off[r] + t // B].astype(np.int64) * B + t % B
        dst_slot[a:b] = case.dst.ids[case.dst.pg_off[r] + t // B].astype(np.int64) * B + t % B
    seg = DRAM_SEG // R                       # rows per 32 KiB

    def page_key(x):                          # 128 KiB block, row within segment, segment
        return (x // (4 * seg)) * (4 * seg) + (x % seg) * 4 + (x % (4 * seg)) // seg
    orders = {"batch order": np.arange(T),
              "sorted by destination slot": np.argsort(dst_slot, kind="stable"),
              "sorted by destination DRAM page": np.argsort(page_key(dst_slot), kind="stable"),
              "sorted by source DRAM page": np.argsort(page_key(src_slot), kind="stable")}
    A = torch.empty((Q, NS, R), dtype=torch.uint8, device=dev)
    Bt = torch.empty_like(A)
    wdev.fill_hash(A, 1, stream=stream)
    wdev.fill_hash(Bt, 2, stream=stream)
    lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)
    PA, PB = kvx.Pool(A, NS), kvx.Pool(Bt, NS)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tok = d(np.array([0, T], np.int64))
    reqs = kvx.Requests(tok, T)
    tabs = {k: (kvx.Table(tok, d(src_slot[o].astype(np.int32))),
                kvx.Table(tok, d(dst_slot[o].astype(np.int32)))) for k, o in orders.items()}
    torch.cuda.synchronize()
    nb = 2 * T * Q * R
    res = {k: [] for k in orders}
    for rnd in range(rounds):
        for k, (sT, dT) in tabs.items():
            ms = graph_timed(torch, stream, lambda i: kvx.gather_scatter(
                lay, PA, sT, reqs, PB, dT, stream=stream), n)
            res[k].append(nb / (ms * 1e-3) / 1e9)
        log(f"dram-pages kv144k_64req_page16 orders round {rnd + 1}/{rounds} done")
    out = [{"order": k, "gather_scatter_GBps": round(sorted(v)[len(v) // 2], 1)}
           for k, v in res.items()]
    for r in out:
        log(f"  kv144k_64req_page16, {r['order']:35s} {r['gather_scatter_GBps']:7.1f}")
    del A, Bt, PA, PB
    torch.cuda.empty_cache()
    return out


def comparators(torch, kvx, wl, wdev, dev):
    """The same 2048-token request moved by per-block runtime copies."""
    import ctypes
    import numpy as np
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    hip.hipMemcpyAsync.restype = ctypes.c_int
    d2d = 3                                        # hipMemcpyDeviceToDevice
    stream = torch.cuda.Stream(device=dev)
    wk = Workload(torch, kvx, wl, wdev, dev, stream)
    sh = stream.cuda_stream
    Q, R, S = wk.Q, wk.R, wk.S
    a0, b0 = wk.A.data_ptr(), wk.B.data_ptr()
    plane = S * R
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def per_block(case, runs):
        """One hipMemcpyAsync per run of consecutive slots (per (token, plane)
        block when runs are single slots)."""
        s_ids = case.src.ids.astype(np.int64)
        d_ids = case.dst.ids.astype(np.int64)
        if runs:
            brk = np.flatnonzero((np.diff(s_ids) != 1) | (np.diff(d_ids) != 1)) + 1
            starts = np.concatenate([[0], brk])
            lens = np.diff(np.concatenate([starts, [len(s_ids)]]))
        else:
            starts = np.arange(len(s_ids))
            lens = np.ones(len(s_ids), np.int64)
        calls = 0
        e0, e1 = ev(), ev()
        t0 = time.perf_counter()
        e0.record(stream)
        for q in range(Q):
            for st, n in zip(starts.tolist(), lens.tolist()):
                rc = hip.hipMemcpyAsync(b0 + q * plane + int(d_ids[st]) * R,
                                        a0 + q * plane + int(s_ids[st]) * R, n * R, d2d, sh)
                if rc != 0:
                    raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
                calls += 1
        e1.record(stream)
        torch.cuda.synchronize()
        return calls, e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3

    out = {}
    rnd = wl.kv144k_2048tok_page1(3)
    calls, ms, wall = per_block(rnd, runs=False)
    out["per_block_random"] = {"calls": calls, "ms": round(ms, 2), "wall_ms": round(wall, 2),
                               "GBps": round(wk.op_bytes / (ms * 1e6), 1)}
    fresh = wl.PagedCase("fresh", wl.KV144K, wl.csr_from_lengths([2048]),
                         wl.side_from_slot_lists([np.arange(4096, 6144)], S),
                         wl.side_from_slot_lists([np.arange(8192, 10240)], S), 0, 0, 0)
    calls, ms, wall = per_block(fresh, runs=True)
    out["per_run_fresh_pool"] = {"calls": calls, "ms": round(ms, 3), "wall_ms": round(wall, 2),
                                 "GBps": round(wk.op_bytes / (ms * 1e6), 1)}
    calls, ms, wall = per_block(rnd, runs=True)
    out["per_run_random"] = {"calls": calls, "ms": round(ms, 2)}
    # the runtime's contiguous copy of a 288 MiB staging buffer
    e0, e1 = ev(), ev()
    e0.record(stream)
    for k in range(8):
        rc = hip.hipMemcpyAsync(wk.S2.data_ptr(), wk.S1.data_ptr(), wk.S1.numel(), d2d, sh)
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 8
    out["runtime_copy_of_staging"] = {"ms": round(ms, 4),
                                      "GBps": round(2 * wk.S1.numel() / (ms * 1e6), 1)}
    # the same copy on the DMA engines (hipMemcpyDeviceToDeviceNoCU: no
    # compute units), the engine a cross-GPU staging copy would use
    e0, e1 = ev(), ev()
    e0.record(stream)
    rc = 0
    for k in range(4):
        rc = hip.hipMemcpyAsync(wk.S2.data_ptr(), wk.S1.data_ptr(), wk.S1.numel(), 1024, sh)
        if rc != 0:
            break
    e1.record(stream)
    torch.cuda.synchronize()
    if rc == 0:
        ms = e0.elapsed_time(e1) / 4
        out["dma_copy_of_staging"] = {"ms": round(ms, 4),
                                      "GBps": round(2 * wk.S1.numel() / (ms * 1e6), 1)}
    else:
        out["dma_copy_of_staging"] = {"error": f"hipMemcpyAsync returned {rc}"}
    for k in range(32):                                  # clocks back up after the idle copies
        kvx.gather_scatter(wk.lay, wk.PA, wk.src_tabs[k % NREQ], wk.reqs, wk.PB,
                           wk.dst_tabs[k % NREQ], stream=stream)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for k in range(8):
        kvx.gather_scatter(wk.lay, wk.PA, wk.src_tabs[k], wk.reqs, wk.PB, wk.dst_tabs[k],
                           stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 8
    out["kvx_gather_scatter"] = {"ms": round(ms, 4), "GBps": round(wk.op_bytes / (ms * 1e6), 1)}
    print(json.dumps(out), flush=True)


# TCC channels summed by the *_sum counters on MI355X: 16 per XCD x 8 XCDs;
# TCP and TA instances summed by *_sum counters: one per compute unit
TCC_CHANNELS = 128
CU_COUNT = 256

# Per-kernel memory-side, translation and wave metrics from the counter passes
# that --summarize-counters reads (each pass a separate rocprofv3 --pmc run of
# `bench.py --pmc-pass`): (column, formula over per-dispatch medians).
COUNTER_METRICS = [
    ("EA read latency (TCC cycles)", lambda m: m["TCC_EA0_RDREQ_LEVEL_sum"] / m["TCC_EA0_RDREQ_sum"]),
    ("EA write latency (TCC cycles)", lambda m: m["TCC_EA0_WRREQ_LEVEL_sum"] / m["TCC_EA0_WRREQ_sum"]),
    ("EA reads in flight", lambda m: m["TCC_EA0_RDREQ_LEVEL_sum"] / (m["TCC_CYCLE_sum"] / TCC_CHANNELS)),
    ("EA writes in flight", lambda m: m["TCC_EA0_WRREQ_LEVEL_sum"] / (m["TCC_CYCLE_sum"] / TCC_CHANNELS)),
    ("EA write-stall cycles / TCC cycles", lambda m: m["TCC_EA0_WRREQ_STALL_sum"] / m["TCC_CYCLE_sum"]),
    ("EA read DRAM-credit-stall cycles / TCC cycles",
     lambda m: m["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"] / m["TCC_CYCLE_sum"]),
    ("TCC busy", lambda m: m["TCC_BUSY_sum"] / m["TCC_CYCLE_sum"]),
    ("TCC tag-stall cycles / TCC cycles", lambda m: m["TCC_TAG_STALL_sum"] / m["TCC_CYCLE_sum"]),
    ("TCP->TCC read latency", lambda m: m["TCP_TCC_READ_REQ_LATENCY_sum"] / m["TCP_TCC_READ_REQ_sum"]),
    ("TCP->TCC write latency", lambda m: m["TCP_TCC_WRITE_REQ_LATENCY_sum"] / m["TCP_TCC_WRITE_REQ_sum"]),
    ("UTCL1 requests", lambda m: m["TCP_UTCL1_REQUEST_sum"]),
    ("UTCL1 translation misses", lambda m: m["TCP_UTCL1_TRANSLATION_MISS_sum"]),
    ("UTCL1 miss rate", lambda m: m["TCP_UTCL1_TRANSLATION_MISS_sum"] / m["TCP_UTCL1_REQUEST_sum"]),
    ("UTCL1 misses under a miss", lambda m: m["TCP_UTCL1_TRANSLATION_MISS_UNDER_MISS_sum"]),
    ("UTCL1 stalls: UTCL2 out of credits (per CU cycle)",
     lambda m: m["TCP_UTCL1_STALL_UTCL2_REQ_OUT_OF_CREDITS_sum"] / (CU_COUNT * m["GRBM_GUI_ACTIVE"])),
    ("UTCL1 stalls: in-flight max (per CU cycle)",
     lambda m: m["TCP_UTCL1_STALL_INFLIGHT_MAX_sum"] / (CU_COUNT * m["GRBM_GUI_ACTIVE"])),
    ("UTCL2 busy / GPU-active cycles", lambda m: m["GRBM_UTCL2_BUSY"] / m["GRBM_GUI_ACTIVE"]),
    ("TCP pending-stall cycles (per CU cycle)",
     lambda m: m["TCP_PENDING_STALL_CYCLES_sum"] / (CU_COUNT * m["GRBM_GUI_ACTIVE"])),
    ("TA address stalled by TC (per CU cycle)",
     lambda m: m["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / (CU_COUNT * m["GRBM_GUI_ACTIVE"])),
    ("TA data stalled by TC (per CU cycle)",
     lambda m: m["TA_DATA_STALLED_BY_TC_CYCLES_sum"] / (CU_COUNT * m["GRBM_GUI_ACTIVE"])),
    ("VMEM instruction latency (SQ cycles)", lambda m: m["VmemLatency"]),
    ("SMEM instruction latency (SQ cycles)", lambda m: m["SmemLatency"]),
    ("waves", lambda m: m["SQ_WAVES"]),
    ("wave life (cycles)", lambda m: 4 * m["SQ_WAVE_CYCLES"] / m["SQ_WAVES"]),
    ("wave time waiting", lambda m: m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]),
    ("waves resident (avg)", lambda m: 4 * m["SQ_WAVE_CYCLES"] / (m["TCC_CYCLE_sum"] / TCC_CHANNELS)),
]


# The counter passes (one rocprofv3 run each: at most 4 TCC, 4 TCP, 2 TA,
# 2 GRBM and 8 SQ counters per run) and the command that makes each.
COUNTER_PASSES = {
    "ea_level": "TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum TCC_EA0_WRREQ_LEVEL_sum "
                "TCC_EA0_WRREQ_sum",
    "stalls": "TCC_EA0_WRREQ_STALL_sum TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum "
              "TCC_TOO_MANY_EA_WRREQS_STALL_sum TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum",
    "tcp_latency": "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum "
                   "TCP_TCC_WRITE_REQ_LATENCY_sum TCP_TCC_WRITE_REQ_sum",
    "busy": "TCC_CYCLE_sum TCC_BUSY_sum TCC_TAG_STALL_sum GRBM_GUI_ACTIVE",
    "sq": "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY "
          "SQ_ACTIVE_INST_VMEM SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR",
    "utcl1": "TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_TRANSLATION_HIT_sum TCP_UTCL1_REQUEST_sum "
             "TCP_UTCL1_STALL_UTCL2_REQ_OUT_OF_CREDITS_sum GRBM_UTCL2_BUSY GRBM_GUI_ACTIVE",
    "vmem_latency": "VmemLatency SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR",
    "smem_latency": "SmemLatency",
    "tcp_stalls": "TCP_PENDING_STALL_CYCLES_sum TCP_UTCL1_TRANSLATION_MISS_UNDER_MISS_sum "
                  "TCP_UTCL1_STALL_INFLIGHT_MAX_sum TCP_TCR_TCP_STALL_CYCLES_sum "
                  "TA_ADDR_STALLED_BY_TC_CYCLES_sum TA_DATA_STALLED_BY_TC_CYCLES_sum "
                  "GRBM_GUI_ACTIVE",
}

# Workloads a counter pass can run (bench.py --pmc-pass --pmc-workload W):
# the bench step on the 4.5 GiB pools, the same step on 1 GiB pools (8192
# slots: the translation comparison), and the MLA single-plane request.
PMC_WORKLOADS = {
    "kv144k": "the five-op step of the 2048-token, 144 KiB/token request, 4.5 GiB pools",
    "kv144k_1gib": "the same step, 1 GiB pools (8192 slots, 4 disjoint requests)",
    "mla": "gather-scatter, gather and scatter of the 2048-token MLA request (27 planes of "
           "1152-byte rows, page 1, 32768-slot pools)",
}


def counter_pass_command(name, tag="kv144k", prefix="rocprof_out/pmcx_"):
    return (f"rocprofv3 --pmc {COUNTER_PASSES[name]} -d {prefix}{tag}_{name} -o pmc "
            f"--output-format csv -- python3 bench.py --pmc-pass --pmc-workload {tag}")


def summarize_counters(out_path, title, tags="kv144k", prefix="rocprof_out/pmcx_"):
    """Markdown table of COUNTER_METRICS per (workload, kernel) from the
    COUNTER_PASSES runs of each workload tag (comma-separated)."""
    tags = [t for t in tags.split(",") if t]
    commands = [counter_pass_command(n, t, prefix) for t in tags for n in COUNTER_PASSES]
    cols = {}
    for t in tags:
        for n in COUNTER_PASSES:
            d = f"{prefix}{t}_{n}"
            if not os.path.isdir(d):
                continue
            for r in counter_rows(d):
                name = r["Kernel_Name"].split("(")[0] if not r["Kernel_Name"].startswith("(") \
                    else r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
                name = name.replace("void ", "").replace("kvx::", "")
                if not name.startswith(("k_paged", "k_permute", "k_copy16")):
                    continue
                key = f"`{name}` ({t})" if len(tags) > 1 else f"`{name}`"
                cols.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    keep = list(cols)
    with open(out_path, "w") as f:
        f.write(f"# {title}\n\n")
        f.write("Per-dispatch medians of hardware counters, one `rocprofv3 --pmc` run per "
                "pass of `python3 bench.py --pmc-pass --pmc-workload W`; workloads: "
                + "; ".join(f"{t}: {PMC_WORKLOADS[t]}" for t in tags)
                + " (each run also launches the plain copy `k_copy16` of 256 MiB).  EA = the "
                "L2's requests to memory; TCC *_sum counters add the "
                f"{TCC_CHANNELS} L2 channels (per-channel cycles = TCC_CYCLE_sum / "
                f"{TCC_CHANNELS}), TCP and TA *_sum counters the {CU_COUNT} compute units "
                "(per-CU shares divide by that and GRBM_GUI_ACTIVE); latencies are "
                "Little's-law averages (requests in flight summed per cycle / requests).\n\n")
        f.write("Commands (from the repository root, on an MI355X machine):\n\n")
        for c in commands:
            f.write(f"    {c}\n")
        f.write(f"    python3 bench.py --summarize-counters {out_path} '{title}' "
                f"{','.join(tags)}\n")
        f.write("\n| metric | " + " | ".join(keep) + " |\n")
        f.write("|---|" + "---:|" * len(keep) + "\n")
        for label, fn in COUNTER_METRICS:
            cells = []
            for k in keep:
                m = {c: sorted(v)[len(v) // 2] for c, v in cols[k].items()}
                try:
                    x = fn(m)
                    cells.append(f"{x:.3f}" if x < 10 else f"{x:,.0f}")
                except (KeyError, ZeroDivisionError):
                    cells.append("-")
            if any(c != "-" for c in cells):
                f.write(f"| {label} | " + " | ".join(cells) + " |\n")
    print(open(out_path).read())


# What the kernels in a bench trace that are not the library's are.
TRACE_NOTES = [
    ("__amd_rocclr_copyBuffer",
     "the HIP runtime's copy kernel: the host readback of the pools and staging "
     "buffers (in pieces of about 1 MiB) for the oracle's parity check and the CPU "
     "baseline, after the timed steps"),
    ("k_fill_hash", "device fill of the pools with seeded SplitMix64 words "
     "(`workloads/devfill.hip`), before any timing"),
    ("k_copy16", "the plain contiguous copy timed beside the ops (reference rate, and "
     "the calibration of the traffic counters)"),
    ("FillFunctor", "torch's zero fill of output buffers at set-up"),
    ("arange", "torch's arange, building the identity page tables of the contiguous-row "
     "gather timed beside the ops"),
]


def summarize_trace(trace_dir, out_path, title, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows.extend(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    with open(out_path, "w") as f:
        f.write(f"# {title}\n\n")
        f.write("Kernel durations from `rocprofv3 --kernel-trace --stats` (microseconds).\n\n")
        f.write("Command (from the repository root, on an MI355X machine):\n\n")
        f.write(f"    {command}\n\n")
        f.write("| kernel | calls | avg us | min us | max us | share % |\n")
        f.write("|---|---:|---:|---:|---:|---:|\n")
        for r in rows:
            name = r["Name"].replace("|", "/")
            if len(name) > 110:
                name = name[:107] + "..."
            f.write(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                    f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                    f"{float(r['Percentage']):.2f} |\n")
        notes = [(key, text) for key, text in TRACE_NOTES
                 if any(key in r["Name"] for r in rows)]
        if notes:
            f.write("\nKernels that are not the library's (`kvx::`):\n\n")
            for key, text in notes:
                f.write(f"* `{key}`: {text}.\n")
    print(open(out_path).read())


COMPARATOR_ROWS = [
    ("per_block_random", "one hipMemcpyAsync per (token, plane) row, random slots"),
    ("per_run_random", "the same, contiguous runs merged (random slots: none to merge)"),
    ("per_run_fresh_pool", "runs merged on a fresh pool (2048 consecutive slots per plane)"),
    ("runtime_copy_of_staging", "runtime copy of the 288 MiB staging buffer (blit kernel)"),
    ("dma_copy_of_staging", "the same copy on the DMA engines (hipMemcpyDeviceToDeviceNoCU)"),
    ("kvx_gather_scatter", "kvx_gather_scatter, random slots, one launch"),
]


def summarize_json(log_path, out_path, title, command):
    """Markdown tables from the JSON lines that --concurrent, --cu-split,
    --comparators, --patterns and --dram-pages print (any of them, in one
    log)."""
    lines = []
    with open(log_path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                try:
                    lines.append(json.loads(line))
                except json.JSONDecodeError:
                    pass
    if not lines:
        raise SystemExit(f"no JSON line in {log_path}")
    with open(out_path, "w") as f:
        f.write(f"# {title}\n\n")
        f.write("GB/s count bytes read + written (decimal).  Made by (from the repository root, "
                "on an MI355X machine):\n\n")
        f.write(f"    {command}\n\n")
        for d in lines:
            if "readers" in d:
                f.write("Gather-scatter of the 2048-token, 144 KiB/token request (16 disjoint "
                        "requests rotated) while a decode-like reader streams a 16 GiB buffer "
                        "on a second stream at the same priority; gather-scatter alone: "
                        f"{d['gather_scatter_alone_GBps']} GB/s.\n\n")
                f.write("| reader workgroups per launch | reader alone | reader under load | "
                        "gather-scatter under load | together | reader outlasts transfer |\n")
                f.write("|---:|---:|---:|---:|---:|---|\n")
                for r in d["readers"]:
                    tog = r["reader_loaded_GBps"] + r["gather_scatter_loaded_GBps"]
                    f.write(f"| {r['reader_blocks']} | {r['reader_alone_GBps']} | "
                            f"{r['reader_loaded_GBps']} | {r['gather_scatter_loaded_GBps']} | "
                            f"{tog:.1f} | {r['reader_outlasts_gather_scatter']} |\n")
                f.write("\n")
            if "splits" in d:
                f.write("The transfer and a full-intensity reader (2048 workgroups) on "
                        "complementary CU masks (hipExtStreamCreateWithCUMask, whole groups "
                        "of 8 CUs, one per XCD).\n\n")
                f.write("| transfer / reader CUs | gather-scatter alone | reader alone | "
                        "gather-scatter under load | reader under load | together |\n")
                f.write("|---|---:|---:|---:|---:|---:|\n")
                for r in d["splits"]:
                    tog = r["reader_loaded_GBps"] + r["gather_scatter_loaded_GBps"]
                    f.write(f"| {r['transfer_cus']} / {r['reader_cus']} | "
                            f"{r['gather_scatter_alone_GBps']} | {r['reader_alone_GBps']} | "
                            f"{r['gather_scatter_loaded_GBps']} | {r['reader_loaded_GBps']} | "
                            f"{tog:.1f} |\n")
                f.write("\n")
            if "kvx_gather_scatter" in d:
                f.write("The 2048-token, 144 KiB/token request (288 MiB each way) moved by "
                        "runtime copies and by one batched launch.\n\n")
                f.write("| method | launches | ms | GB/s |\n|---|---:|---:|---:|\n")
                for key, label in COMPARATOR_ROWS:
                    r = d.get(key)
                    if not r:
                        continue
                    if "error" in r:
                        f.write(f"| {label} | - | {r['error']} | - |\n")
                        continue
                    calls = r.get("calls", 1)
                    gbps = r.get("GBps", round(603979776 / (r["ms"] * 1e6), 1))
                    f.write(f"| {label} | {calls} | {r['ms']} | {gbps} |\n")
                f.write("\n")
            if "row_patterns" in d:
                f.write("The 2048-token request's 72 x 2048 rows of 2 KiB moved by a table-free "
                        "kernel (each row's slot a bijective hash of its token in the same two "
                        "4.5 GiB page-1 pools, 16 disjoint slot sets rotated), by access "
                        "pattern and rows per wave.\n\n")
                f.write("| pattern | 1 row / wave | 2 rows / wave | 4 rows / wave |\n"
                        "|---|---:|---:|---:|\n")
                for r in d["row_patterns"]:
                    f.write(f"| {r['pattern']} | {r['rows_per_wave_1_GBps']} | "
                            f"{r['rows_per_wave_2_GBps']} | {r['rows_per_wave_4_GBps']} |\n")
                f.write("\nThe library's ops on the same request, timed alone in the same "
                        "process (with their page-table reads):\n\n| op | GB/s |\n|---|---:|\n")
                for op, v in d["library_ops_alone_GBps"].items():
                    f.write(f"| {op} | {v} |\n")
                f.write("\n")
            if "dram_pages" in d:
                f.write("The 2048-token request (72 planes of 2 KiB rows, 288 MiB each way) "
                        "with its slots placed differently at the same density: 2048 of the "
                        "32768 slots of each page-1 pool per request.\n\n")
                f.write("| slot placement (source and destination) | gather-scatter | gather | "
                        "scatter |\n|---|---:|---:|---:|\n")
                for r in d["dram_pages"]:
                    f.write(f"| {r['design']} | {r['gather_scatter_GBps']} | "
                            f"{r['gather_GBps']} | {r['scatter_GBps']} |\n")
                f.write("\n")
            if "block_pools" in d:
                f.write("The same request between block pools of the same 32768 slots (pages "
                        "of B rows, the request's pages a seeded random subset, 8 disjoint "
                        "requests rotated); from pages of 64 KiB the library pairs the rows "
                        "32 KiB apart on the two waves of one workgroup.\n\n")
                f.write("| page size (rows) | page (KiB) | rows paired | gather-scatter | "
                        "gather | scatter |\n|---:|---:|---|---:|---:|---:|\n")
                for r in d["block_pools"]:
                    f.write(f"| {r['page_size']} | {r['page_KiB']} | "
                            f"{'yes' if r['paired'] else 'no'} | {r['gather_scatter_GBps']} | "
                            f"{r['gather_GBps']} | {r['scatter_GBps']} |\n")
                f.write("\n")
            if "kv_block_pools" in d:
                f.write("The same request between pools whose blocks hold a layer's K and V "
                        "pages together (one [36][blocks][2][B][R] tensor per pool over the "
                        "same bytes, page stride 2 B R); from pages of 32 KiB a K row and the "
                        "V row of the same token share a DRAM page, and a gather-scatter or "
                        "scatter runs the two planes of a token on the two waves of one "
                        "workgroup (a gather pairs its staging rows instead).\n\n")
                f.write("| page size (rows) | page (KiB) | planes paired | gather-scatter | "
                        "gather | scatter |\n|---:|---:|---|---:|---:|---:|\n")
                for r in d["kv_block_pools"]:
                    f.write(f"| {r['page_size']} | {r['page_KiB']} | "
                            f"{'yes' if r['planes_paired'] else 'no'} | "
                            f"{r['gather_scatter_GBps']} | {r['gather_GBps']} | "
                            f"{r['scatter_GBps']} |\n")
                f.write("\n")
            if "kv144k_64req_page16_orders" in d:
                f.write("The kv144k_64req_page16 batch (64 requests of 128 pages of 16 tokens, "
                        "two 36 GiB pools, "
                        "half of each pool's pages in use) written as one page-1 request over "
                        "the same slots, its tokens in other orders (a gather-scatter's "
                        "result does not depend on the order).\n\n")
                f.write("| token order | gather-scatter |\n|---|---:|\n")
                for r in d["kv144k_64req_page16_orders"]:
                    f.write(f"| {r['order']} | {r['gather_scatter_GBps']} |\n")
                f.write("\n")
            if "mla_row_patterns" in d:
                f.write("The MLA request (27 planes of 1152-byte rows, 2048 tokens, 32768-slot "
                        "page-1 pools, 64 MB each way) moved the same ways without tables:\n\n")
                f.write("| pattern | 1 row / wave | 2 rows / wave | 4 rows / wave |\n"
                        "|---|---:|---:|---:|\n")
                for r in d["mla_row_patterns"]:
                    f.write(f"| {r['pattern']} | {r['rows_per_wave_1_GBps']} | "
                            f"{r['rows_per_wave_2_GBps']} | {r['rows_per_wave_4_GBps']} |\n")
                f.write("\nThe library's MLA ops in the same process (16 disjoint requests "
                        "rotated):\n\n| op | GB/s |\n|---|---:|\n")
                for op, v in d["library_mla_ops_GBps"].items():
                    f.write(f"| {op} | {v} |\n")
                f.write("\n")
            if "note" in d:
                f.write(f"Note: {d['note']}\n\n")
    print(open(out_path).read())


def pmc_pass(torch, kvx, wl, wdev, dev, stream, workload):
    """A short run for rocprofv3 --pmc: three of each kernel of the workload
    (PMC_WORKLOADS), then three plain copies of COPY_CALIB_BYTES (the
    counters' calibration)."""
    if workload == "mla":
        import numpy as np
        cases = [wl.mla_case(1, k) for k in range(4)]
        g = cases[0].geom
        Q, R, S = g.planes, g.row_bytes, cases[0].src.num_slots
        A = torch.empty((Q, S, R), dtype=torch.uint8, device=dev)
        B = torch.empty((Q, S, R), dtype=torch.uint8, device=dev)
        wdev.fill_hash(A, cases[0].value_seed, stream=stream)
        wdev.fill_hash(B, cases[0].sentinel_seed, stream=stream)
        st = torch.zeros(2048 * Q * R, dtype=torch.uint8, device=dev)
        lay = kvx.Layout(g.num_layers, g.num_kv, g.kv_heads, g.head_dim, g.dtype)

        def dv(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        reqs = kvx.Requests(dv(cases[0].tok_off), 2048)
        tabs = [(kvx.Table(dv(c.src.pg_off), dv(c.src.ids)),
                 kvx.Table(dv(c.dst.pg_off), dv(c.dst.ids))) for c in cases]
        PA, PB = kvx.Pool(A, S), kvx.Pool(B, S)
        for i in range(3):
            kvx.gather_scatter(lay, PA, tabs[i][0], reqs, PB, tabs[i][1], stream=stream)
            kvx.gather(lay, PA, tabs[(i + 1) % 4][0], reqs, st, stream=stream)
            kvx.scatter(lay, st, reqs, PB, tabs[(i + 2) % 4][1], stream=stream)
    else:
        wk = Workload(torch, kvx, wl, wdev, dev, stream,
                      slots=8192 if workload == "kv144k_1gib" else 32768)
        A, B = wk.A, wk.B
        for i in range(3):
            wk.step(i, stream)
    a, b = A.reshape(-1), B.reshape(-1)
    for k in range(3):
        wdev.copy_bytes(b[k * COPY_CALIB_BYTES:], a[k * COPY_CALIB_BYTES:], COPY_CALIB_BYTES,
                        stream=stream)
    torch.cuda.synchronize()
    log(f"pmc pass done ({workload})")


# ----------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="time budget per oracle thread count")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="a short run for counter collection (no JSON line)")
    ap.add_argument("--all-configs", action="store_true",
                    help="time every op on all five workloads (JSON line per op)")
    ap.add_argument("--concurrent", action="store_true",
                    help="gather-scatter while a decode-like HBM reader runs on another stream")
    ap.add_argument("--cu-split", action="store_true",
                    help="the transfer and a full-intensity reader on complementary CU masks")
    ap.add_argument("--sizes", action="store_true",
                    help="gather-scatter and gather of one request of 16 .. 8192 tokens")
    ap.add_argument("--row-sizes", action="store_true",
                    help="~256 MiB each way of rows of 256 B .. 16 KiB (every copy variant)")
    ap.add_argument("--batches", action="store_true",
                    help="49152 tokens split into 1 .. 49152 requests (request lookup cost)")
    ap.add_argument("--comparators", action="store_true",
                    help="the same request moved by one runtime copy per block / per run")
    ap.add_argument("--patterns", action="store_true",
                    help="the request's row patterns moved by a table-free kernel, beside "
                         "the library's ops")
    ap.add_argument("--dram-pages", action="store_true",
                    help="the request's ops over slot placements of equal density: rows that "
                         "share DRAM pages or not")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "OUT", "TITLE", "CMD"),
                    help="markdown summary of a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--pmc-out", default=PMC_SUMMARY, help="where --summarize-pmc writes")
    ap.add_argument("--summarize-counters", nargs="+", metavar="OUT TITLE [TAGS]",
                    help="per-kernel memory, translation and wave metrics from the counter "
                         "passes of the workload tags (comma-separated, default kv144k)")
    ap.add_argument("--pmc-workload", default="kv144k", choices=sorted(PMC_WORKLOADS),
                    help="what --pmc-pass runs")
    ap.add_argument("--summarize-json", nargs=4, metavar=("LOG", "OUT", "TITLE", "CMD"),
                    help="markdown tables from the JSON lines of --concurrent / --cu-split / "
                         "--comparators / --patterns / --dram-pages")
    ap.add_argument("--counter-commands", action="store_true",
                    help="print the rocprofv3 command of every counter pass")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.pmc_out)
        return 0
    if args.summarize_json:
        summarize_json(*args.summarize_json)
        return 0
    if args.summarize_counters:
        if len(args.summarize_counters) not in (2, 3):
            ap.error("--summarize-counters OUT TITLE [TAGS]")
        summarize_counters(*args.summarize_counters)
        return 0
    if args.counter_commands:
        for t in PMC_WORKLOADS:
            for n in COUNTER_PASSES:
                print(counter_pass_command(n, t))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the path on one GPU only: both pools live in that GPU's "
              "HBM and nothing here spans GPUs; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import scatter_kvx_gather_amd as kvx
    import workloads as wl
    from workloads import device as wdev

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 2
    kvx.load_library()
    dev = torch.device("cuda:0")
    if args.cu_split:                      # before any other stream takes a hardware queue
        cu_split(torch, kvx, wl, wdev, dev)
        return 0
    stream = torch.cuda.Stream(device=dev)
    if args.all_configs:
        all_configs(torch, kvx, wl, wdev, dev, stream, reps=5, cpu=not args.no_cpu_baseline)
        return 0
    if args.concurrent:
        concurrent_load(torch, kvx, wl, wdev, dev)
        return 0
    if args.sizes:
        request_sizes(torch, kvx, wl, wdev, dev, stream)
        return 0
    if args.batches:
        batch_sizes(torch, kvx, wl, wdev, dev, stream)
        return 0
    if args.row_sizes:
        row_sizes(torch, kvx, wl, wdev, dev, stream)
        return 0
    if args.comparators:
        comparators(torch, kvx, wl, wdev, dev)
        return 0
    if args.patterns:
        row_patterns(torch, kvx, wl, wdev, dev, stream)
        return 0
    if args.dram_pages:
        dram_pages(torch, kvx, wl, wdev, dev, stream)
        return 0
    if args.pmc_pass:
        pmc_pass(torch, kvx, wl, wdev, dev, stream, args.pmc_workload)
        return 0
    log("setup: 2 pools of 4.5 GiB, 16 request tables")
    wk = Workload(torch, kvx, wl, wdev, dev, stream)
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    settle = settle_steps(torch, wk, stream)
    for i in range(W):
        wk.step(settle["steps"] + i, stream)
    W0 = settle["steps"]                           # step indices continue past the settle
    # timed region: events around the two slowest kernels -- the
    # gather-scatter on even steps, the scatter on odd steps -- and around the
    # whole region; events around every op would cost ~4% of the step, so the
    # other ops are timed in a later diagnostic pass
    live_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # torch creates a HIP event at its first record: record every event once
    # here, so that the timed region creates none (measured: in a process
    # started right after another had used the GPU, creating the events
    # inside the timed region slowed the host's enqueue to ~2 ms per step,
    # 20 steps measuring 2.2 ms/step instead of 0.53)
    for evs in live_ev:
        for e in evs:
            e.record(stream)
    t_start.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()                       # barrier: one rank
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        wk.step(W0 + W + i, stream, live_ev[i], marks=(0, 1) if i % 2 == 0 else (4, 5))
    t_end.record(stream)
    issue = time.perf_counter() - wall0             # host time to enqueue the K steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / K
    gs_ms = sorted(live_ev[i][0].elapsed_time(live_ev[i][1]) for i in range(0, K, 2))
    sc_ms = sorted(live_ev[i][4].elapsed_time(live_ev[i][5]) for i in range(1, K, 2))
    live_ms = {"gather_scatter": sum(gs_ms) / len(gs_ms),
               "scatter": sum(sc_ms) / max(1, len(sc_ms))}

    def pct(v, q):
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))] if v else None

    launch_stats = {op: {"mean": round(sum(v) / len(v), 5), "median": round(pct(v, 0.5), 5),
                         "p95": round(pct(v, 0.95), 5), "max": round(v[-1], 5),
                         "launches": len(v)}
                    for op, v in (("gather_scatter", gs_ms), ("scatter", sc_ms)) if v}
    step_bytes = wk.op_bytes * len(OPS)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"timed {K} steps: {ms_step:.4f} ms/step (wall {wall * 1e3 / K:.4f} ms/step), "
        f"gather_scatter {live_ms['gather_scatter'] * 1e3:.1f} us, "
        f"scatter {live_ms['scatter'] * 1e3:.1f} us")

    # per-op diagnostic pass (events around every op; not part of the value)
    nd = 50
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(nd)]
    torch.cuda.synchronize()
    for i in range(nd):
        wk.step(W0 + W + K + i, stream, events[i])
    torch.cuda.synchronize()
    op_ms = {op: sum(e[j].elapsed_time(e[j + 1]) for e in events) / nd
             for j, op in enumerate(OPS)}
    for op in OPS:
        log(f"  {op:15s} {op_ms[op] * 1e3:8.1f} us  {wk.op_bytes / op_ms[op] / 1e6:8.1f} GB/s")

    # contiguous copy ceiling: the same bytes as one op, over rotating chunks
    ncopy = 16
    chunk = wk.A.shape[1] * wk.R * 4              # 4 planes = 256 MiB contiguous
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ce[0].record(stream)
    for k in range(ncopy):
        p = (k * 4) % wk.Q
        wdev.copy_bytes(wk.B[p:p + 4].reshape(-1), wk.A[p:p + 4].reshape(-1), chunk,
                        stream=stream)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_ms = ce[0].elapsed_time(ce[1]) / ncopy
    copy_gbps = 2 * chunk / (copy_ms * 1e-3) / 1e9

    # the same gather kernel over contiguous rows (2048 consecutive slots of
    # each plane, rotating over the 16 disjoint ranges, into staging): the
    # access-pattern ceiling of the row mover itself
    idents = [kvx.Table(torch.tensor([0, wk.T], dtype=torch.int64, device=dev),
                        torch.arange(k * wk.T, (k + 1) * wk.T, dtype=torch.int32, device=dev))
              for k in range(NREQ)]
    torch.cuda.synchronize()
    ce[0].record(stream)
    for k in range(ncopy):
        kvx.gather(wk.lay, wk.PA, idents[k % NREQ], wk.reqs, wk.S1, stream=stream)
    ce[1].record(stream)
    torch.cuda.synchronize()
    ident_ms = ce[0].elapsed_time(ce[1]) / ncopy

    # every op alone: per launch, rotated inputs, nothing reading the output
    iso = time_isolated(torch, wk, stream)
    for op in OPS:
        log(f"  alone {op:15s} {iso[op]['ms_per_launch'] * 1e3:8.1f} us  {iso[op]['GBps']:8.1f} GB/s"
            f"  {100 * iso[op]['frac_hbm_peak']:.1f}% of peak (one launch: "
            f"{100 * iso[op]['single_launch_frac_hbm_peak']:.1f}%)")

    # the dominant kernel: the slower of the two live-timed kernels (the other
    # ops are ~25% faster in the diagnostic pass); its achieved rate uses the
    # live events of the timed region
    dom = max(live_ms, key=lambda o: live_ms[o])
    if op_ms[max(OPS, key=lambda o: op_ms[o])] > 1.05 * live_ms[dom]:
        log("warning: an op without live events is the slowest in the diagnostic pass")
    dom_ms = live_ms[dom]
    # kernel instance the library picks for these 2 KiB rows: one row per
    # wave when a launch moves more than one round of resident waves at
    # 8 KiB chunks (32 waves per CU), otherwise 4 rows per 8 KiB chunk
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    u = 1 if wk.op_bytes // 2 > cus * 32 * 8192 else 4
    # batches of more than 64 requests take the instances with the 64-way
    # request search
    m = "true" if wk.reqs.num_reqs > 64 else "false"
    # (the last template argument: nontemporal stores, the default)
    kernel_of = {"gather_scatter": f"k_paged<PoolRef, PoolRef, 2, {u}, {m}, true>",
                 "gather": f"k_paged<PoolRef, StageRef, 2, {u}, {m}, true>",
                 "scatter": f"k_paged<StageRef, PoolRef, 2, {u}, {m}, true>",
                 "rebuild": f"k_permute_rows<true, 2, {u}, true>",
                 "extract": f"k_permute_rows<false, 2, {u}, true>"}
    achieved = wk.op_bytes / (dom_ms * 1e-3) / 1e9
    traffic, traffic_kernel = read_traffic()
    if traffic is not None and traffic_kernel and "PoolRef, kvx::PoolRef" not in traffic_kernel:
        traffic = None
    if traffic is not None and traffic_kernel and dom == "gather_scatter":
        measured = traffic_kernel.split("(")[0].replace("void ", "").replace("kvx::", "")
        if measured != kernel_of[dom]:
            log(f"warning: counter summary names {measured}, expected {kernel_of[dom]}")
            kernel_of[dom] = measured
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic if dom == "gather_scatter" else None,
                "kernel": kernel_of[dom], "op": dom,
                "launch_ms": round(dom_ms, 5),
                "timing": "HIP events around its launches in the timed region",
                "algorithmic_bytes_per_launch": wk.op_bytes}

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "settle": settle,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": "kv144k_2048tok_page1: 1 request x 2048 tokens x 36 layers x {K,V} x "
                        "8 kv_heads x 128 (144 KiB/token, 288 MiB), bf16 payload copied "
                        "bitwise; token-paged pools of 32768 slots (4.5 GiB each), 16 "
                        "disjoint requests rotated",
            "step": "gather_scatter + gather + rebuild_permute + extract_permute + scatter; "
                    "staging and HF hand-offs double-buffered (each op reads what the "
                    "previous step produced), so no op reads its input from the Infinity "
                    "Cache",
            "bytes_per_step": step_bytes,
            "seeds": wk.seeds,
            "tables_sha256": wk.tables_sha256,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "GiBps": round(value * 1e9 / 2 ** 30, 1),
        "table_bytes_per_step": wk.table_bytes_per_step,
        "ms_per_288MiB_request": round(live_ms["gather_scatter"], 5),
        "launch_ms": launch_stats,
        "ops": {op: {"ms": round(op_ms[op], 5),
                     "GBps": round(wk.op_bytes / (op_ms[op] * 1e-3) / 1e9, 1)} for op in OPS},
        "ops_timing": "diagnostic pass after the timed region, events around every op",
        "copy_ceiling": {"plain_copy_GBps": round(copy_gbps, 1),
                         "plain_copy_bytes": 2 * chunk,
                         "gather_contiguous_rows_GBps":
                             round(wk.op_bytes / (ident_ms * 1e-3) / 1e9, 1)},
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
        "host_issue_ms_per_step": round(issue * 1e3 / K, 5),
        "roofline": roofline,
        "ops_isolated": iso,
        "ops_isolated_timing": "each op alone, rotated requests and inputs, nothing reading "
                               "the output; after 8 warm launches: 24 launches back to back "
                               "between two HIP events on the launch stream (ms_per_launch, "
                               "GBps, frac_hbm_peak: the sustained rate), and 24 with events "
                               "around each launch (single_launch_*: median)",
        "bar": {"target_frac_hbm_peak": 0.70,
                "gather": {"frac": iso["gather"]["frac_hbm_peak"],
                           "met": iso["gather"]["frac_hbm_peak"] >= 0.70},
                "gather_scatter": {"frac": iso["gather_scatter"]["frac_hbm_peak"],
                                   "met": iso["gather_scatter"]["frac_hbm_peak"] >= 0.70}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # four more steps (the isolated timing above wrote into the double
        # buffers, and the last step's scatter carries rows gathered three
        # steps before it), then the last step's results are checked against
        # the oracle
        j = W + K + 1000
        for i in range(j - 3, j + 1):
            wk.step(i, stream)
        torch.cuda.synchronize()
        res, ncores, parity, share = cpu_baseline(wk, args.cpu_seconds, parity_step=j)
        result["parity"] = parity
        steps_n, el_n = res[ncores]
        steps_1, el_1 = res[1]
        model, sockets = host_cpu()
        result["cpu_baseline"] = {
            "value": round(steps_n * step_bytes / el_n / 1e9, 2), "unit": "GB/s",
            "cores": ncores, "kind": "oracle",
            "sample": f"{steps_n} full steps (the same 5 ops, requests and double buffers on "
                      f"host copies of the same 4.5 GiB pools) in {el_n:.1f} s with {ncores} "
                      f"threads (median of 3 runs)",
            "cpu_model": model, "sockets": sockets,
            "nproc": share["nproc"], "affinity_cpus": share["affinity"],
            "cgroup_cpus": share["cgroup_cpus"],
            "threads_rule": "every usable core: the affinity mask, capped by the cgroup CPU "
                            "quota when one is set",
            "one_thread_GBps": round(steps_1 * step_bytes / el_1 / 1e9, 2),
            "ms_per_step": round(el_n / steps_n * 1e3, 2),
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
