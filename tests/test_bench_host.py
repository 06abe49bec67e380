"""Host-side contracts of bench.py (no GPU): the single-GPU guard, the rule
that memory traffic is reported only from counters taken on the current
kernel source for the same workload, and the CPU baseline's process pool."""

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
            "traffic_bytes_per_launch": 123456789,
            "memory_side_read_bytes_per_launch": 1000, "memory_side_write_bytes_per_launch": 10}
    base.update(kw)
    path.write_text(json.dumps(base))


def test_traffic_only_from_matching_counters(tmp_path, monkeypatch):
    f = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS", str(f))
    assert bench.traffic_from_profile("wan") == (None, None)         # no file
    f.write_text("{not json")
    assert bench.traffic_from_profile("wan") == (None, None)         # unreadable
    _write(f)
    t, extra = bench.traffic_from_profile("wan")
    assert t == 123456789
    assert extra == {"memory_side_read_bytes_per_launch": 1000, "memory_side_write_bytes_per_launch": 10}
    assert bench.traffic_from_profile("mochi") == (None, None)       # another workload
    assert bench.traffic_from_profile("wan720") == (None, None)      # a prefix is not a match
    _write(f, kernel_source_hash="0" * 16)
    assert bench.traffic_from_profile("wan") == (None, None)         # kernel changed since


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


def test_cpu_baseline_pool_over_heads():
    """The oracle leg runs one process per head group with one BLAS thread
    each, and records the host it ran on."""
    import numpy as np
    import synth
    from tests.gpu_util import small_cfg
    cfg = small_cfg(B=1, H=4, L=1024, S=1000, d=64, block=128, dtype="bf16", seed=3)
    q, k, v = synth.gen_qkv(cfg)
    rp, ci = synth.random_csr(np.random.default_rng(1), cfg.H, cfg.nqb, cfg.nkb_valid, 0.3)
    r = bench.cpu_baseline(q, k, v, rp, ci, cfg, 1.0, workers=2)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["value"] > 0
    assert r["host"]["nproc"] >= 1 and "cpu_model" in r["host"] and "ram_gib" in r["host"]
    assert "2 processes" in r["sample"]
