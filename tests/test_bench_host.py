"""Host logic of bench.py (CPU): committed counter figures are used only for the kernel source
they were measured on, and the one-GPU contract is enforced before anything touches a device."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _recorded_hash(fname, key):
    return json.load(open(os.path.join(ROOT, "profiles", fname)))[key]["source_sha256_16"]


def test_counter_figures_follow_the_source_hash(monkeypatch):
    for fname, lookup in (("traffic.json", bench.measured_traffic), ("mfma.json", bench.measured_mfma)):
        recorded = _recorded_hash(fname, "prefill_attn_lse")
        monkeypatch.setattr(bench, "kernel_source_hash", lambda name: recorded)
        got = lookup("prefill_attn_lse", "prefill_attn.hip")
        assert got is not None
        if lookup is bench.measured_mfma:
            assert 0.0 < got["mfma_util"] < 1.0
            assert got["executed_flops_per_launch"] >= 2 * 128 * 32 * 4000 * 4001   # at least the causal triangle
        else:
            assert got > 0
        monkeypatch.setattr(bench, "kernel_source_hash", lambda name: "0000000000000000")
        assert lookup("prefill_attn_lse", "prefill_attn.hip") is None
        assert lookup("no_such_kernel", "prefill_attn.hip") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
