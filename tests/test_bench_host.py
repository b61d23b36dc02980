"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the committed
counter traffic and its source-hash guard, and the configuration lists."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_several_gpus_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_target_configurations_and_entry_keys():
    assert [label for label, _ in bench.TARGET_CONFIGS] == ["ep32", "ep32_fp8", "ep256", "zipf", "hier8x8"]
    for key in ("value", "ms_per_step", "hbm_frac_step", "roofline", "cpu_baseline", "config"):
        assert key in bench.PER_CONFIG_KEYS


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_FILES))
def test_kernel_source_hash_is_stable_and_distinct_per_source_set(kernel):
    h = bench.kernel_source_hash(kernel)
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash(kernel)


def test_committed_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    """The counter figure is reported only while the kernel's sources hash to
    the value recorded with the counters; otherwise None (not a stale number)."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"workload": "w", "fetch_factor": 2.0, "write_factor": 1.0,
           "kernels": {"dispatch_kernel": {"source_sha": "0123456789abcdef",
                                           "hbm_bytes_per_launch": 4.5e8}}}
    (prof / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "0123456789abcdef")
    assert bench.committed_traffic("w", "dispatch_kernel") == 4.5e8
    assert bench.committed_traffic("w", "combine_kernel") is None      # kernel not recorded
    assert bench.committed_traffic("other", "dispatch_kernel") is None  # no summary
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "fedcba9876543210")
    assert bench.committed_traffic("w", "dispatch_kernel") is None      # sources changed
    (prof / "traffic_w.json").write_text("{not json")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "0123456789abcdef")
    assert bench.committed_traffic("w", "dispatch_kernel") is None      # unreadable summary


def test_committed_summaries_are_well_formed():
    """Every committed traffic summary names its workload, the two counter
    scale factors and, per kernel, a 16-digit source hash (none for the
    runtime's and PyTorch's own kernels)."""
    d = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(d) if f.startswith("traffic_") and f.endswith(".json")]
    assert files
    for f in files:
        rec = json.load(open(os.path.join(d, f)))
        assert rec["workload"] == f[len("traffic_"):-len(".json")]
        assert 1.5 < rec["fetch_factor"] < 2.5 and 0.5 < rec["write_factor"] < 1.5
        for name, k in rec["kernels"].items():
            assert k["source_sha"] is None or len(k["source_sha"]) == 16, (f, name)
            assert k["hbm_bytes_per_launch"] >= 0
