"""Pruned lattice on the GPU against the fp64 oracle's pruned loss.

The bands (lo[b, t] <= u < lo[b, t] + S per frame) come from rnnt_inputs.diagonal_band.
The same tolerances as the full loss (per dtype). At the 40 s x 256 shape: the W^O = 0
closed form for every sample (every in-band alignment has probability V^-(T_b + U_b), so
cost_b = (T_b + U_b) ln V - ln(number of in-band alignments), the count by a plain integer
recursion here) and the oracle on one sample.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from rnnt_inputs import diagonal_band, make_inputs, workload_inputs
from test_gpu_parity import GRADS, TOL, check_costs, check_grads, say

pytestmark = pytest.mark.gpu


def run_pruned(rl, inp, lo, S, mode="tiled", tile=(64, 32), tpw=0, dcosts=None):
    import torch

    prob = rl.Problem(inp, mode=mode, tile=tile, tiles_per_wave=tpw, band=(lo, S))
    costs = prob.forward().clone()
    dc = None if dcosts is None else torch.tensor(np.asarray(dcosts, np.float32), device=prob.device)
    grads = prob.backward(dc)
    torch.cuda.synchronize()
    out = costs.cpu().numpy().astype(np.float64), {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    del prob
    return out


def pruned_check(rl, inp, S, **kw):
    T = inp.hA.shape[1]
    lo = diagonal_band(inp.T_len, inp.U_len, T, S)
    ref = oracle.loss_and_grads(inp, band=(lo, S))
    costs, grads = run_pruned(rl, inp, lo, S, **kw)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
    return costs, grads


@pytest.mark.parametrize("mode,tile,tpw", [("tiled", (32, 16), 5), ("untiled", (32, 16), 0), ("tiled", (20, 7), 2)])
def test_pruned_fp32(gpu_lib, mode, tile, tpw):
    inp = make_inputs(3, 75, 41, 300, 48, 40, 64, dtype="f32", seed=141, t_range=(20, 75), u_range=(0, 41),
                      bias_std=0.3)
    say(f"pruned fp32 B=3 T=75 U=41 S=6 {mode} tile={tile}")
    pruned_check(gpu_lib, inp, 6, mode=mode, tile=tile, tpw=tpw)


@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_pruned_bf16_reduced(gpu_lib, mode):
    inp = make_inputs(4, 100, 30, 1000, 128, 96, 128, dtype="bf16", seed=151, t_range=(40, 100), u_range=(0, 30),
                      bias_std=0.1)
    say(f"pruned bf16 reduced S=8 {mode}")
    pruned_check(gpu_lib, inp, 8, mode=mode, tile=(32, 16), tpw=5)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("mode,S", [("tiled", 16), ("untiled", 16), ("tiled", 4)])
def test_pruned_small_workload(gpu_lib, mode, S):
    say(f"pruned small workload S={S} {mode}")
    pruned_check(gpu_lib, workload_inputs("small-bf16"), S, mode=mode)


def band_paths_log(lo, S, Tb, Ub):
    """ln of the number of alignments whose every cell lies in the band (exact integers)."""
    prev = {}
    for t in range(Tb):
        row = {}
        for u in range(lo[t], min(lo[t] + S, Ub + 1)):
            c = 1 if (t == 0 and u == 0) else prev.get(u, 0) + row.get(u - 1, 0)
            row[u] = c
        prev = row
    return math.log(prev[Ub])


@pytest.mark.timeout(600)
def test_pruned_40s_b256(gpu_lib):
    inp = workload_inputs("40s-b256-bf16")
    S = 32
    lo = diagonal_band(inp.T_len, inp.U_len, inp.hA.shape[1], S)
    say(f"pruned 40s-b256 S={S}, W^O = 0: closed-form cost for every sample")
    inp0 = dataclasses.replace(inp, WO=np.zeros_like(inp.WO), bO=np.zeros_like(inp.bO))
    c0, _ = run_pruned(gpu_lib, inp0, lo, S)
    for b in range(len(inp.T_len)):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        want = (Tb + Ub) * math.log(1024) - band_paths_log(lo[b], S, Tb, Ub)
        assert abs(c0[b] - want) <= 1e-5 * want, (b, c0[b], want)
    say("pruned 40s-b256, oracle on sample 5")
    e = np.zeros(len(inp.T_len))
    e[5] = 1.0
    costs, grads = run_pruned(gpu_lib, inp, lo, S, dcosts=e)
    ref = oracle.loss_and_grads(inp, dcosts=e, samples=[5], band=(lo, S))
    check_costs(inp, costs, ref.costs, samples=[5])
    check_grads(inp, grads, ref.grads)
