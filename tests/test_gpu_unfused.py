"""The unfused batched comparator of bench.py against the fp64 oracle.

bench.py --unfused-baseline times an unfused batched loss over the materialised
[B, T, U+1, V] scores (torch GEMMs, log_softmax and elementwise passes, this library's
lattice kernel for alpha / beta), the structure the pages compare the fused, tiled loss
against ("Flash RNN-T ...", section "What changed in practice"; "Neural transducer
training ...", section "Transducer training", f^W_1..4 as separate passes). Its
time and memory ratios are only meaningful if it computes the same loss: here its costs
and every gradient meet the bf16 tolerances against the oracle at the small workload.
"""
import numpy as np
import pytest

import bench
import oracle
from rnnt_inputs import workload_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(400)
def test_unfused_comparator_matches_oracle(gpu_lib):
    import torch

    inp = workload_inputs("small-bf16")
    print("unfused comparator, small workload", flush=True)
    ms, peak, costs, grads = bench.unfused_baseline(torch, gpu_lib, inp, 1, 1)
    torch.cuda.synchronize()
    assert ms > 0 and peak > 0
    ref = oracle.loss_and_grads(inp)
    c = costs.cpu().numpy().astype(np.float64)
    rel = np.max(np.abs(c - ref.costs) / np.abs(ref.costs))
    assert rel <= 2e-3, rel
    for k, r in ref.grads.items():
        g = grads[k].float().cpu().numpy().astype(np.float64)
        err = np.max(np.abs(g - r))
        assert err <= 2e-2 * np.max(np.abs(r)), (k, err, np.max(np.abs(r)))
