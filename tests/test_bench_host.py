"""Host-side logic of bench.py, on the CPU: the command line refuses more
than one GPU and a machine without one (no CPU fallback, no JSON line), the
A/B/B/A helper runs its arms in A B B A order and reports the medians and the
paired difference it claims, and the counter traffic is reported only for the
measured workload and kernel sources."""

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def test_no_gpu_fails_loudly_without_a_result_line():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the refusal without one")
    r = _run("--steps", "4", "--warmup", "1", "--no-cpu-baseline", "--quick", "--no-extras")
    assert r.returncode != 0
    assert "needs a GPU" in r.stderr
    assert '"metric"' not in r.stdout


class _FakeClock:
    def __init__(self):
        self.t = 0.0

    def __call__(self):
        return self.t


def test_abba_order_medians_and_paired_difference(monkeypatch):
    import torch
    clock = _FakeClock()
    monkeypatch.setattr(bench.time, "perf_counter", clock)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []
    # Arm A costs 10 us per step; arm B 12 us in its first block of a round
    # and 13 us in its second, so the paired difference per round is 2.5 us.
    state = {"b_in_round": 0}

    def arm_a(steps):
        calls.append("A")
        clock.t += steps * 10e-6

    def arm_b(steps):
        calls.append("B")
        clock.t += steps * (12e-6 if state["b_in_round"] % 2 == 0 else 13e-6)
        state["b_in_round"] += 1

    res = bench.abba({"A": arm_a, "B": arm_b}, ("A", "B"), rounds=5, block=100)
    assert calls == ["A", "B", "B", "A"] * 5
    assert res["A"]["n"] == 10 and res["B"]["n"] == 10
    assert res["A"]["median"] == pytest.approx(10.0)
    assert res["B"]["median"] == pytest.approx(12.5)
    assert res["B"]["iqr"] == pytest.approx([12.0, 13.0])
    assert res["paired_B_minus_A"]["n"] == 5
    assert res["paired_B_minus_A"]["median"] == pytest.approx(2.5)
    assert res["rounds"] == 5 and res["block_steps"] == 100


def test_traffic_only_for_the_measured_workload_and_sources(monkeypatch):
    t = bench.MEASURED_TRAFFIC
    expected = (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0
    assert bench.measured_traffic_bytes(4) == pytest.approx(expected)
    for config in (1, 2, 3, 5):
        assert bench.measured_traffic_bytes(config) is None
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic_bytes(4) is None


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    # The hash that guards the counter figures changes with the code of the
    # kernel sources, not with their comments or blank lines.
    import shutil
    src = os.path.join(ROOT, "decode_attention_paged_e5m2_amd", "csrc")
    dst = tmp_path / "decode_attention_paged_e5m2_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("xqa_kernels.hip", "xqa_internal.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_sources_sha256()
    kern = dst / "xqa_kernels.hip"
    text = kern.read_text(encoding="utf-8")
    kern.write_text("// a new comment\n\n/* and a\n block one */\n" + text, encoding="utf-8")
    assert bench.kernel_sources_sha256() == h0
    kern.write_text(text + "\nstatic int extra_symbol;\n", encoding="utf-8")
    assert bench.kernel_sources_sha256() != h0
