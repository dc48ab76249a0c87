"""Host-side checks of bench.py: the one-GPU guard and the profile-backed
traffic figure (no GPU needed)."""

from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_matching_sources_and_workload(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()
    prof = tmp_path / "p.txt"
    prof.write_text(f"first 16 hex): {digest}\n  total HBM traffic per launch   = 1,234 B\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.profiled_traffic("v3_b64_ctx8k_paged_bf16") == 1234
    assert bench.profiled_traffic("tiny_f32") is None
    prof.write_text("first 16 hex): 0000000000000000\n  total HBM traffic per launch = 1,234 B\n")
    assert bench.profiled_traffic("v3_b64_ctx8k_paged_bf16") is None


def test_prefill_traffic_only_for_matching_sources_and_workload(tmp_path, monkeypatch):
    # the committed summary matches the committed prefill sources
    assert bench.prefill_traffic("v3_prefill_b2_8k_bf16") is not None
    assert bench.prefill_traffic("v3_prefill_b2_8k_fp8") is None
    prof = tmp_path / "p.txt"
    prof.write_text("first 16 hex): 0000000000000000\n  total HBM traffic per launch = 1,234 B\n")
    monkeypatch.setattr(bench, "PREFILL_TRAFFIC_PROFILE", str(prof))
    assert bench.prefill_traffic("v3_prefill_b2_8k_bf16") is None
