"""CPU tests of the benchmark's host logic: the one-GPU guard, the
counter-derived traffic that is only reported for the kernel source it was
measured on, and the scheduler timing legs (product through the C ABI and
the reference scheduler) agreeing on what they scheduled."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel source A\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"rowwise": "k.hip"})
    assert bench.load_traffic("rowwise") is None               # no summary yet
    js = {"source_hash": bench.source_hash("k.hip"), "traffic_bytes_per_launch": 12345}
    (prof / "rowwise_c3_counters.json").write_text(json.dumps(js))
    assert bench.load_traffic("rowwise") == 12345
    src.write_text("kernel source B\n")                         # the kernel changed since
    assert bench.load_traffic("rowwise") is None
    # a kernel built from two sources: a change in either one drops the figure
    (tmp_path / "k2.hip").write_text("second source\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"rowwise": ["k.hip", "k2.hip"]})
    js["source_hash"] = bench.source_hash(["k.hip", "k2.hip"])
    (prof / "rowwise_c3_counters.json").write_text(json.dumps(js))
    assert bench.load_traffic("rowwise") == 12345
    (tmp_path / "k2.hip").write_text("second source, changed\n")
    assert bench.load_traffic("rowwise") is None


@pytest.mark.parametrize("shared", [False, True])
def test_scheduler_timing_legs_agree(shared):
    pytest.importorskip("numpy")
    from paged_kv_attention_reshape_amd import _sched
    if not os.path.exists(_sched.SCHED_LIB_PATH):
        pytest.skip("libpa_sched.so is not built")
    a = bench.scheduler_timing(product=True, steps=40, shared=shared)
    b = bench.scheduler_timing(product=False, steps=40, shared=shared)
    for k in ("scheduled_tokens", "preemptions", "prefix_hit_tokens", "evictions", "cow_copies"):
        assert a.get(k) == b.get(k), k
    assert a["scheduled_tokens"] > 0
    if shared:
        assert a["prefix_hit_tokens"] > 0
