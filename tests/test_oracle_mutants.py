"""Plant a mistake in the oracle (on the CPU) and check that the pins catch it.

Each mutant is a textual edit of a copy of oracle/kvx_oracle.c, compiled into a
temporary directory and driven by the pin checks in a child process (so a
mutant that reads or writes out of bounds and crashes counts as caught).  The
real oracle source is never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvx_oracle.c")

# the page-table index range checks of the row and head-sliced lookups
_ROWS_INDEX = ("    if (s->pg_off[r] < -k || s->pg_off[r] >= s->num_ids - k) return -1;\n"
               "    int64_t idx = s->pg_off[r] + k;\n"
               "    int64_t page = (int64_t)s->ids[idx];\n"
               "    if (page < 0 || page >= s->num_pages) return -1;\n"
               "    return page;")
_HEADS_INDEX = ("    if (s->pg_off[r] < -k || s->pg_off[r] >= s->num_ids - k) return -1;\n"
                "    int64_t idx = s->pg_off[r] + k;\n"
                "    int64_t page = (int64_t)s->ids[idx];\n"
                "    if (page < 0 || page >= s->num_pages) return -1;\n"
                "    int64_t row")
_UPPER = " || s->pg_off[r] >= s->num_ids - k"
_LOWER = "s->pg_off[r] < -k || "

MUTANTS = {
    "row_in_page_uses_div": ("(t % s->page_size) * s->stride", "(t / s->page_size) * s->stride"),
    "page_index_uses_mod": ("int64_t k = t / s->page_size;\n" + _ROWS_INDEX,
                            "int64_t k = t % s->page_size;\n" + _ROWS_INDEX),
    "page_stride_ignored": ("return page * s->page_stride + (t % s->page_size) * s->stride;",
                            "return page * s->page_size * s->stride + (t % s->page_size) * s->stride;"),
    "page_stride_default_wrong": ("page_stride != 0 ? page_stride : (int64_t)page_size * stride",
                                  "page_stride != 0 ? page_stride : stride"),
    "staging_drops_Q_factor": ("(j->tok_off[r] * j->Q + q * n + t)", "(j->tok_off[r] + q * n + t)"),
    "staging_token_major": ("(j->tok_off[r] * j->Q + q * n + t)",
                            "(j->tok_off[r] * j->Q + t * j->Q + q)"),
    "bound_off_by_one": ("page >= s->num_pages) return -1;\n    return page;",
                         "page > s->num_pages) return -1;\n    return page;"),
    "last_token_dropped": ("for (int64_t t = 0; t < n; ++t)", "for (int64_t t = 0; t + 1 < n; ++t)"),
    "gather_reads_plane0": ("memcpy(staged, j->src.planes[q]", "memcpy(staged, j->src.planes[0]"),
    "gs_dst_uses_src_side": ("int64_t d = row_offset(&j->dst, r, t);\n                if (s < 0 || d < 0)",
                             "int64_t d = row_offset(&j->src, r, t);\n                if (s < 0 || d < 0)"),
    "gs_ignores_dst_oor": ("if (s < 0 || d < 0)", "if (s < 0)"),
    "hf_index_transposed": ("((int64_t)h * j->s_cap + s)", "((int64_t)s * j->H + h)"),
    "flat_index_transposed": ("(((int64_t)q * j->seq + s) * j->H + h)",
                              "(((int64_t)q * j->H + h) * j->seq + s)"),
    "permute_direction_swapped": ("if (j->rebuild) memcpy(hf_row, flat_row, (size_t)j->Db);",
                                  "if (!j->rebuild) memcpy(hf_row, flat_row, (size_t)j->Db);"),
    "permute_runs_to_s_cap": ("for (int64_t s = 0; s < j->seq; ++s)",
                              "for (int64_t s = 0; s < j->s_cap; ++s)"),
    "skip_not_counted": ("if (s < 0) { ++skipped; continue; }", "if (s < 0) { continue; }"),
    "hnd_index_swapped": ("(h * s->page_size + row) * Db", "(row * s->H + h) * Db"),
    "nhd_head_offset_dropped": ("(page * s->page_size + row) * s->stride + h * Db",
                                "(page * s->page_size + row) * s->stride"),
    "dst_slice_uses_src_h0": ("head_offset(&j->dst, j->Db, r, t, j->dst.h0 + k)",
                              "head_offset(&j->dst, j->Db, r, t, j->src.h0 + k)"),
    "hnd_head_scaled_by_stride": ("(h * s->page_size + row) * Db",
                                  "(h * s->page_size + row) * s->stride"),
    "hnd_page_base_missing_page_size": ("return page * s->page_size * s->stride + (h",
                                        "return page * s->stride + (h"),
    "heads_skip_counted_per_head": ("                ++skipped;\n                continue;\n            }\n            for (int32_t k = 0; k < j->nh; ++k)",
                                    "                skipped += j->nh;\n                continue;\n            }\n            for (int32_t k = 0; k < j->nh; ++k)"),
    "heads_last_head_dropped": ("for (int32_t k = 0; k < j->nh; ++k)",
                                "for (int32_t k = 0; k + 1 < j->nh; ++k)"),
    "index_upper_unchecked": (_ROWS_INDEX, _ROWS_INDEX.replace(_UPPER, "")),
    "index_upper_off_by_one": (_ROWS_INDEX, _ROWS_INDEX.replace(">= s->num_ids - k",
                                                                "> s->num_ids - k")),
    "index_lower_unchecked": (_ROWS_INDEX, _ROWS_INDEX.replace(_LOWER, "")),
    "list_bounded_by_next_start": (_ROWS_INDEX, _ROWS_INDEX.replace(
        "int64_t idx = s->pg_off[r] + k;\n",
        "int64_t idx = s->pg_off[r] + k;\n    if (idx >= s->pg_off[r + 1]) return -1;\n")),
    "heads_index_upper_unchecked": (_HEADS_INDEX, _HEADS_INDEX.replace(_UPPER, "")),
    "heads_index_lower_unchecked": (_HEADS_INDEX, _HEADS_INDEX.replace(_LOWER, "")),
}

DRIVER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._lib = oracle.bind({lib!r})
from tests import oracle_pins
for check in oracle_pins.ALL_CHECKS:
    try:
        check()
    except AssertionError:
        print("CAUGHT", check.__name__, flush=True)
        sys.exit(0)
print("MISSED", flush=True)
sys.exit(3)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "mutant.c")
        lib = os.path.join(tmp, "libmutant.so")
        open(src, "w").write(text.replace(old, new))
        subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-pthread", src, "-o", lib], check=True)
        p = subprocess.run([sys.executable, "-c", DRIVER.format(root=ROOT, lib=lib)], cwd=ROOT,
                           capture_output=True, text=True, timeout=300)
    out = p.stdout + p.stderr
    # caught by a pin (exit 0 after CAUGHT) or crashed on its own bad access
    assert "MISSED" not in out, f"mutant {name} passed every pin:\n{out[-2000:]}"
    assert p.returncode == 0 or p.returncode < 0 or "CAUGHT" in out or "Error" in out, out[-2000:]
