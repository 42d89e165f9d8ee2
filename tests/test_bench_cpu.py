"""bench.py host logic that runs without a GPU: the single-GPU guard, the
traffic figure's source check and the oracle baseline."""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_recorded_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    prof = tmp_path / "p.txt"

    def write(h):
        prof.write_text("# summary\n  indented = ignored\ntraffic_bytes_per_launch=1234\n"
                        f"kernel_sources_sha256={h}\nkernel_sources=k.hip\n")

    write(hashlib.sha256(b"kernel v1\n").hexdigest())
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(tmp_path / "bench.py"))
    assert bench.recorded_traffic("p.txt") == 1234
    src.write_text("kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.recorded_traffic("p.txt") is None
    assert bench.recorded_traffic("missing.txt") is None


def test_cpu_baseline_times_whole_steps():
    """Every pair of the batch, whole steps on worker processes (all at once
    and one at a time), medians, the CPU model recorded."""
    from long_context_sparse_page_amd import synth

    w = synth.workload(0, batch=2)
    w.context = [4064, 2 * 4064]
    r = bench.cpu_baseline(w, list(w.context), steps=3, workers=2)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["unit"] == "steps/s"
    assert r["value"] > 0 and r["one_core"]["cores"] == 1 and r["one_core"]["value"] > 0
    assert "all 2 (sequence, KV head) pairs" in r["sample"] and "median of 3 whole steps" in r["sample"]
    assert r["cpu_model"]


def test_cpu_baseline_sample_is_scaled_by_pages():
    """More pairs than the sample holds: a seeded sample, scaled by scored +
    attended pages, and said so."""
    from long_context_sparse_page_amd import synth

    w = synth.workload(0, batch=2)
    w.context = [4064, 4064]
    r = bench.cpu_baseline(w, list(w.context), steps=3, workers=1, max_pairs=1)
    assert "a seeded sample of 1 of 2 pairs, scaled x2.00" in r["sample"]
    assert r["cores"] == 1


def test_cpu_baseline_child_prints_one_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cpu-baseline-child", "--workload", "0",
                        "--rank", "8", "--budget", "512", "--steps-done", "0", "--summary", "kv",
                        "--lens", "[4064]", "--cpu-steps", "3"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    import json
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["kind"] == "oracle" and d["value"] > 0
