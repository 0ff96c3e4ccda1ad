"""Host-side checks of bench.py: the one-GPU contract and the CPU baseline record."""
import os
import subprocess
import sys

import numpy as np

import bench
from rnnt_inputs import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_record():
    """One sample of a small batch through the oracle: the record carries the fields the bench line
    reports, and the rate is the sample's time extrapolated to the batch's padded cells."""
    inp = make_inputs(3, 12, 4, 40, 8, 8, 8, dtype="bf16", seed=5, t_range=(6, 12), u_range=(1, 4))
    rec = bench.cpu_baseline(inp, 0.0)  # budget 0: exactly one sample, the smallest
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "cells/s"
    assert rec["cores"] >= 1 and np.isfinite(rec["value"]) and rec["value"] > 0
    smallest = int(np.argmin(inp.T_len * (inp.U_len + 1)))
    assert f"[{smallest}]" in rec["sample"]
