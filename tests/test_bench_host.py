"""Host-side contracts of bench.py (no GPU): the single-GPU guard and the rule
that HBM traffic is reported only from counters taken on the current kernel
source for the same workload."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout.strip() == ""          # no result line is printed


def _write(path, **kw):
    base = {"kernel_source_hash": bench.kernel_source_hash(), "workload": "wan: B=1 H=40 ...",
            "hbm_bytes_per_launch": 123456789}
    base.update(kw)
    path.write_text(json.dumps(base))


def test_traffic_only_from_matching_counters(tmp_path, monkeypatch):
    f = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS", str(f))
    assert bench.traffic_from_profile("wan") is None                 # no file
    f.write_text("{not json")
    assert bench.traffic_from_profile("wan") is None                 # unreadable
    _write(f)
    assert bench.traffic_from_profile("wan") == 123456789
    assert bench.traffic_from_profile("mochi") is None               # another workload
    assert bench.traffic_from_profile("wan720") is None              # a prefix is not a match
    _write(f, kernel_source_hash="0" * 16)
    assert bench.traffic_from_profile("wan") is None                 # kernel changed since


def test_kernel_source_hash_covers_the_forward_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16
    src = tmp_path / "k.hip"
    src.write_text("a")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    monkeypatch.setattr(bench, "ROOT", "/")
    a = bench.kernel_source_hash()
    src.write_text("b")
    assert bench.kernel_source_hash() != a
