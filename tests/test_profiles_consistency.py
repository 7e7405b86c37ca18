"""The measured HBM traffic bench.py reports and the committed counter summary
agree: same kernel-source hash and the same FETCH_SIZE / WRITE_SIZE readings
for the split kernel; every kernel-trace summary names the same sources.
CPU only (reads text files)."""

import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _read(name):
    with open(os.path.join(PROFILES, name), encoding="utf-8") as f:
        return f.read()


def _hash(text):
    m = re.search(r"=\s*([0-9a-f]{64})\.", text)
    assert m, "no sources hash in the summary"
    return m.group(1)


def _first_number(row):
    return float(row.split("|")[2].strip().replace(",", ""))


def test_counter_summary_matches_bench_constants():
    text = _read("split_kernel_ragged_b16_counters.md")
    t = bench.MEASURED_TRAFFIC
    assert _hash(text) == t["sources_sha256"]
    fetch = next(ln for ln in text.splitlines() if ln.startswith("| FETCH_SIZE (KiB)"))
    write = next(ln for ln in text.splitlines() if ln.startswith("| WRITE_SIZE (KiB)"))
    assert abs(_first_number(fetch) - t["fetch_kib"]) < 0.06
    assert abs(_first_number(write) - t["write_kib"]) < 0.06


def test_trace_summaries_name_the_measured_sources():
    h = bench.MEASURED_TRAFFIC["sources_sha256"]
    for name in ("split_kernel_ragged_b16_kernel_trace.md", "all_workloads_kernel_trace.md",
                 "next_rows_ragged_b16_kernel_trace.md",
                 "split_and_combine_uniform_b8_boundary_b16_counters.md"):
        assert _hash(_read(name)) == h, name


def test_summaries_give_their_commands():
    for name in os.listdir(PROFILES):
        text = _read(name)
        assert "rocprofv3" in text and "bench.py" in text, name
