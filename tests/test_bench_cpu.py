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


def test_cpu_baseline_on_a_small_sample():
    from long_context_sparse_page_amd import synth

    w = synth.workload(0)
    r = bench.cpu_baseline(w, list(w.context), 0.3)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "steps/s"
    assert r["value"] > 0
    assert "1 of 1" in r["sample"]


@pytest.mark.parametrize("lens,expect", [([4064, 4064], 2.0), ([4064, 2 * 4064], None)])
def test_cpu_baseline_scales_by_pages(lens, expect):
    """Equal lengths scale by the pair count; other lengths by scored + attended pages."""
    from long_context_sparse_page_amd import synth

    w = synth.workload(0)
    w.batch = 2
    w.context = [4064, 4064]
    r = bench.cpu_baseline(w, lens, 0.2)
    if expect is not None:
        assert "scaled x2 to one step" in r["sample"]
    else:
        assert "by scored + attended pages" in r["sample"]
