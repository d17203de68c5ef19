"""bench.py's host-side contract, on the CPU: the multi-GPU refusal, the
sweep's config filter and the counter-summary lookup."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_sweep_rejects_unknown_configs():
    import bench
    assert "headline" in bench.SWEEP_CONFIGS
    assert set(bench.FUSED_SWEEP_CONFIGS) <= set(bench.SWEEP_CONFIGS)

    class Args:
        only = "headline,no_such_config"
    with pytest.raises(SystemExit, match="no_such_config"):
        bench.sweep(Args(), None, None, None, None)


def test_traffic_lookup_follows_the_kernel_hash(tmp_path, monkeypatch):
    # counters are reported only for the workload they were taken on and
    # while the kernel's own sources are unchanged
    import bench
    from chunked_kda_prefill_amd import build as kbuild
    rec = {"workload": "w", "fetch_factor": 2.0, "write_factor": 1.0,
           "kda_intra": {"fetch_kib": 10.0, "write_kib": 5.0,
                         "kernel_hash": kbuild.kernel_hash("kda_intra.hip")},
           "kda_recurrence": {"fetch_kib": 1.0, "write_kib": 1.0, "kernel_hash": "stale"}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "headline_hbm_traffic.md").write_text(
        f"x\n<!-- traffic-json: {json.dumps(rec)} -->\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", "kda_intra") == 25 * 1024
    assert bench.measured_traffic("w", "kda_recurrence") is None
    assert bench.measured_traffic("other", "kda_intra") is None
    assert bench.measured_traffic("w", "no_such_kernel") is None
