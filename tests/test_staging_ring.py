"""The forward's plan upload does not wait on the host in steady state.

tests/host/staging_ring_test.cpp drives the library's staging ring (csrc/staging.hpp,
compiled here with g++) through a simulated runtime whose events complete only when the
test says so: two forward uploads back to back on a busy stream enqueue without a host
wait, completed slots are reused, and a host wait happens (and is counted) only when the
ring's slot limit is reached.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rnn_loss_joint_amd", "csrc")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def test_staging_ring_never_waits_in_steady_state(tmp_path):
    exe = str(tmp_path / "staging_ring_test")
    r = subprocess.run(["g++", "-O1", "-std=c++17", *SANITIZE, f"-I{CSRC}", os.path.join(ROOT, "tests", "host",
                                                                              "staging_ring_test.cpp"),
                        "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
