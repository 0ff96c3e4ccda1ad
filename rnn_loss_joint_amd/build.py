"""Build the gfx950 shared library librnnt_mi355.so in this package directory.

    python -m rnn_loss_joint_amd.build [--jobs N]

Each translation unit is compiled by hipcc for gfx950 into _build/ (in
parallel), then linked with hipcc -shared. Packed FP32 VALU instructions are
disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librnnt_mi355.so")
ARCH = "gfx950"
SOURCES = ["api.hip", "joint.hip", "lattice.hip", "gemm.hip", "mma.hip", "dz_dwo.hip", "scores3.hip", "labels.hip", "plan.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
          f"-I{os.path.join(PKG, '..', 'include')}"]


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c", path, "-o", out]
    else:
        cmd = ["g++", *COMMON, "-c", path, "-o", out]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=1200)
    msgs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    print(f"  {src}: {time.time() - t0:.1f}s", flush=True)
    return out


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    t0 = time.time()
    print("built", build(a.jobs), f"in {time.time() - t0:.1f}s")


if __name__ == "__main__":
    main()
