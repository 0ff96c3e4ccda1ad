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
    """A small batch through the oracle pool (two worker processes, budget 0: each worker's first
    sample only): the record carries the fields the bench line reports, and the rate is the
    completed samples' valid cells over the wall time, with the padded numerator."""
    inp = make_inputs(5, 12, 4, 40, 8, 8, 8, dtype="bf16", seed=5, t_range=(6, 12), u_range=(1, 4))
    rec = bench.cpu_baseline(inp, 0.0, workers=2)
    assert {"value", "unit", "cores", "kind", "sample"} <= set(rec)
    assert rec["kind"] == "oracle" and rec["unit"] == "cells/s"
    assert rec["cores"] == 2 and np.isfinite(rec["value"]) and rec["value"] > 0
    assert "2 processes" in rec["sample"] and "2 of the batch's 5 samples" in rec["sample"]
    assert abs(rec["value"] / rec["valid_cells_per_s"] - inp.padded_cells / inp.valid_cells) < 1e-9
