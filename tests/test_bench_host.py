"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the kernel
source hash that gates the committed traffic figure, the trace summary and
the CPU-share probe.  Nothing here touches a GPU."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stdout + p.stderr
    assert p.stdout.strip() == "" or not p.stdout.strip().startswith("{")


def test_source_hash_ignores_comments_and_follows_code():
    b = _bench()
    texts = {}
    for rel in b.KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            texts[rel] = f.read()
    base = b.kernel_source_sha256(texts)
    assert base == b.kernel_source_sha256()
    first = b.KERNEL_SOURCES[0]
    commented = dict(texts)
    commented[first] = "// a note\n/* a block\n comment */\n" + texts[first] + "\n   \n"
    assert b.kernel_source_sha256(commented) == base
    edited = dict(texts)
    edited[first] = texts[first].replace("constexpr int kWave = 64;", "constexpr int kWave = 32;")
    assert edited[first] != texts[first]
    assert b.kernel_source_sha256(edited) != base


def test_traffic_is_withheld_when_the_kernels_changed(tmp_path, monkeypatch):
    b = _bench()
    good = tmp_path / "good.md"
    good.write_text("# t\n\n- kernel: `k`\n- traffic_bytes_per_launch: 604229101\n"
                    f"- kernel_source_sha256: `{b.kernel_source_sha256()}`\n")
    monkeypatch.setattr(b, "PMC_SUMMARY", str(good))
    assert b.read_traffic() == (604229101, "k")
    stale = tmp_path / "stale.md"
    stale.write_text("# t\n\n- kernel: `k`\n- traffic_bytes_per_launch: 604229101\n"
                     "- kernel_source_sha256: `" + "0" * 64 + "`\n")
    monkeypatch.setattr(b, "PMC_SUMMARY", str(stale))
    assert b.read_traffic() == (None, "k")
    monkeypatch.setattr(b, "PMC_SUMMARY", str(tmp_path / "missing.md"))
    assert b.read_traffic() == (None, None)


def test_trace_summary_names_the_helper_kernels(tmp_path):
    b = _bench()
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    (d / "bench_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs"\n'
        '"__amd_rocclr_copyBuffer",100,2000000,20000,60.0,2000,24000\n'
        '"void kvx::k_paged<kvx::PoolRef, kvx::PoolRef, 2, 1, false, true>(x)",10,1187000,'
        '118700,35.0,114100,128200\n'
        '"(anonymous namespace)::k_copy16(y)",2,177200,88600,5.0,77400,90900\n')
    out = tmp_path / "out.md"
    b.summarize_trace(str(tmp_path / "trace"), str(out), "title", "the command")
    text = out.read_text()
    lines = text.splitlines()
    rows = [ln for ln in lines if ln.startswith("| `")]
    assert [r.split("`")[1].split("(")[0].split("<")[0] for r in rows] == [
        "__amd_rocclr_copyBuffer", "void kvx::k_paged", ""]
    assert "k_copy16" in rows[2]
    assert "| 118.7 | 114.1 | 128.2 |" in rows[1]
    assert "    the command" in lines
    notes = [ln for ln in lines if ln.startswith("* `")]
    assert [n.split("`")[1] for n in notes] == ["__amd_rocclr_copyBuffer", "k_copy16"]


def test_cpu_share_is_within_the_machine():
    b = _bench()
    s = b.cpu_share()
    assert 1 <= s["usable"] <= s["affinity"] <= s["nproc"]
    model, sockets = b.host_cpu()
    assert isinstance(model, str) and model and sockets >= 1


def test_dram_page_placements_have_the_structure_they_name():
    import numpy as np
    b = _bench()
    NS, T, N = 32768, 2048, 8
    for i, (label, sk, dk) in enumerate(b.DRAM_PAGE_DESIGNS):
        for kind, arg in (sk, dk):
            sets = b.dram_page_sets(kind, arg, np.random.default_rng(i), NS, T, N, 2048)
            assert len(sets) == N, label
            allx = np.concatenate(sets)
            assert len(np.unique(allx)) == N * T, label          # disjoint requests
            assert allx.min() >= 0 and allx.max() < NS, label
            for x in sets:
                assert len(x) == T
                if kind == "sorted":
                    assert np.all(np.diff(x) > 0)
                if kind == "pairs":
                    dist, gap = arg
                    blk = x.reshape(-1, 2, gap)                 # [starts..., partners...]
                    assert np.all(blk[:, 1, :] - blk[:, 0, :] == dist), label
                    assert np.all(blk[:, 0, :] % (2 * dist) < dist), label
                if kind == "pages":
                    B, grouped = arg
                    runs = x.reshape(-1, B)
                    base = runs.min(axis=1)
                    assert np.all(base % B == 0), label
                    assert np.all(np.sort(runs, axis=1) == base[:, None] + np.arange(B)), label
                    off = runs - base[:, None]
                    if grouped:
                        g = b.DRAM_SEG // 2048
                        # consecutive tokens are g rows (32 KiB) apart within a group
                        assert np.all(off[:, :B // g] == g * np.arange(B // g)), label
                    else:
                        assert np.all(off == np.arange(B)), label


def test_settle_phase_stops_when_two_blocks_agree_or_at_its_cap():
    """settle_steps on fake CUDA objects: blocks of 8 steps until two blocks
    in a row agree within 3% (and the host outruns the GPU), else until the
    time cap; the step indices it used are the ones it reports."""
    b = _bench()
    seq = {"gpu": []}

    class Ev:
        def __init__(self, enable_timing=True):
            pass

        def record(self, stream=None):
            pass

        def elapsed_time(self, other):
            return seq["gpu"].pop(0) * 8

    class Cuda:
        Event = Ev

        @staticmethod
        def synchronize():
            pass

    class Torch:
        cuda = Cuda

    class Wk:
        def __init__(self):
            self.steps = []

        def step(self, i, stream):
            self.steps.append(i)

    seq["gpu"] = [1.4, 0.53, 0.52, 0.52]
    wk = Wk()
    out = b.settle_steps(Torch, wk, None)
    assert out["steps"] == 24 and wk.steps == list(range(24))
    assert [g for g, _ in out["blocks_gpu_host_ms_per_step"]] == [1.4, 0.53, 0.52]
    seq["gpu"] = [1.0 + (k % 2) for k in range(1000000)]      # never agrees
    wk = Wk()
    out = b.settle_steps(Torch, wk, None, max_s=0.05)
    assert out["steps"] == len(wk.steps) and out["steps"] % 8 == 0 and out["seconds"] >= 0.05
