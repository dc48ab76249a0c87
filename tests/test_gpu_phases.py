"""The instrumented build (libmla_phases.so, include/mla_debug.h): its
split-KV phase timers account for every cycle of every working wave, and the
report runs on a uniform batch.  Runs the report as its own process, since
the binding loads one library per process."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_phase_report_accounts_for_every_cycle():
    print("[gpu-case] phase_report batch 8 x 8192", flush=True)
    r = subprocess.run([sys.executable, "-m", "mla_latent_kv_06_amd.phase_report", "--batch", "8",
                        "--ctx", "8192", "--runs", "3", "--json"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    out = json.loads(r.stdout.strip().splitlines()[-1])
    # 8 x 128 tiles on 256 workgroups: 4 tiles (8 half-tiles) each, walked as
    # the first half's scores, 6 steady-state iterations and the last one;
    # the laps (checked in the tool) sum to each wave's cycles
    assert out["steady_half_tiles_per_wave"] == 6
    shares = sum(v["share"] for v in out["laps"].values())
    assert abs(shares - 1.0) < 1e-6
    assert 0.5 < out["clock_ghz"] < 3.0
