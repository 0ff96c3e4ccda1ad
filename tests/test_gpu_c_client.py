"""The loss through the C ABI from a C program: no Python, no torch in the computing process.

tests/host/abi_gpu_client.c allocates device buffers with hipMalloc, copies the inputs, calls
rnnt_loss_query / rnnt_loss_fwd / rnnt_loss_bwd on the default stream and writes the costs and
gradients back to files; this test writes the inputs, runs the client as a child process and
compares its outputs with the fp64 oracle at the dtype's tolerances (fp32 and bf16, tiled and
untiled).
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import rnn_loss_joint_amd as rl
from rnnt_inputs import make_inputs
from test_gpu_parity import check_costs, check_grads, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GRADS = {"dhA": "hA", "dhL": "hL", "dWA": "WA", "dWL": "WL", "dbZ": "bZ", "dWO": "WO", "dbO": "bO"}


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("cclient") / "abi_gpu_client")
    lib_dir = os.path.dirname(rl.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
           "-I/opt/rocm/include", os.path.join(ROOT, "tests", "host", "abi_gpu_client.c"), f"-L{lib_dir}",
           "-lrnnt_mi355", "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


def raw(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":  # the values are exact in bf16: the upper half of each fp32
        return (a.view(np.uint32) >> 16).astype(np.uint16).tobytes()
    return a.tobytes()


@pytest.mark.parametrize("dtype,mode", [("f32", "tiled"), ("bf16", "tiled"), ("bf16", "untiled")])
def test_c_client_matches_oracle(client, tmp_path, dtype, mode):
    inp = make_inputs(3, 70, 18, 500, 64, 48, 640 if dtype == "bf16" else 64, dtype=dtype, seed=91,
                      t_range=(20, 70), u_range=(0, 18), bias_std=0.2)
    B, T, HA = inp.hA.shape
    U1, HL = inp.hL.shape[1], inp.hL.shape[2]
    V, H = inp.WO.shape
    d = tmp_path
    (d / "dims.txt").write_text(f"{B} {T} {U1 - 1} {V} {HA} {HL} {H} {int(inp.blank)} {1 if dtype == 'bf16' else 0} "
                                f"{1 if mode == 'untiled' else 0} 32 8\n")
    (d / "T_len").write_bytes(np.ascontiguousarray(inp.T_len, np.int32).tobytes())
    (d / "U_len").write_bytes(np.ascontiguousarray(inp.U_len, np.int32).tobytes())
    (d / "labels").write_bytes(np.ascontiguousarray(inp.labels, np.int32).tobytes())
    for name in ("hA", "hL", "WA", "WL", "bZ", "WO", "bO"):
        (d / name).write_bytes(raw(getattr(inp, name), dtype))
    say(f"C client {dtype} {mode}")
    r = subprocess.run([client, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    costs = np.fromfile(d / "costs", np.float32).astype(np.float64)
    grads = {k: np.fromfile(d / k, np.float32).astype(np.float64).reshape(getattr(inp, v).shape)
             for k, v in GRADS.items()}
    ref = oracle.loss_and_grads(inp)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
