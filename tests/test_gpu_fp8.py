"""The fp8 output layer (RNNT_BF16_FP8) on the GPU against the fp64 oracle's fp8 reading.

The oracle with fp8_scores=True rounds the output layer's two operands to OCP E4M3 (z by
2^8, W^O by its power-of-two scale) and keeps every other step exact; the library must match
it at the bf16 tolerances (cost 2e-3 relative, gradients 2e-2 of max-abs), the same budget
the bf16 path meets against the exact oracle. Each check also prints the distance of the fp8
result from the exact (unrounded) oracle: that is the approximation the fp8 product makes,
recorded, not asserted beyond a loose bound. At the 40 s x 256 shape the W^O = 0 closed form
holds for every sample (zero rounds to zero) and the oracle checks one sample.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from rnnt_inputs import make_inputs, workload_inputs
from test_gpu_parity import GRADS, check_costs, check_grads, lnC, say

pytestmark = pytest.mark.gpu


def run_fp8(rl, inp, tile=(64, 32), tpw=0, dcosts=None):
    import torch

    prob = rl.Problem(inp, mode="tiled", tile=tile, tiles_per_wave=tpw, fp8=True)
    costs = prob.forward().clone()
    dc = None if dcosts is None else torch.tensor(np.asarray(dcosts, np.float32), device=prob.device)
    grads = prob.backward(dc)
    torch.cuda.synchronize()
    out = costs.cpu().numpy().astype(np.float64), {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    del prob
    return out


def distance_from_exact(inp, costs, grads, samples=None, dcosts=None):
    """Print how far the fp8 result lies from the exact oracle (the approximation itself)."""
    ref = oracle.loss_and_grads(inp, dcosts=dcosts, samples=samples)
    idx = range(len(inp.T_len)) if samples is None else samples
    c = max(abs(costs[b] - ref.costs[b]) / abs(ref.costs[b]) for b in idx)
    g = {k: np.max(np.abs(grads[k] - ref.grads[k])) / max(np.max(np.abs(ref.grads[k])), 1e-30) for k in GRADS}
    say("  fp8 vs exact oracle: cost max rel " + f"{c:.2e}, grad err / max-abs "
        + " ".join(f"{k} {v:.1e}" for k, v in g.items()))
    return c, g


def fp8_check(rl, inp, **kw):
    ref = oracle.loss_and_grads(inp, fp8_scores=True)
    costs, grads = run_fp8(rl, inp, **kw)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
    c, _ = distance_from_exact(inp, costs, grads)
    assert c <= 2e-2
    return costs, grads


@pytest.mark.parametrize("tile,tpw", [((32, 16), 5), ((20, 7), 2)])
def test_fp8_small_hidden(gpu_lib, tile, tpw):
    # H = 128: the E4M3 rows are padded to 640 bytes (five stages of 128)
    inp = make_inputs(4, 100, 30, 1000, 128, 96, 128, dtype="bf16", seed=161, t_range=(40, 100), u_range=(0, 30),
                      bias_std=0.1)
    say(f"fp8 B=4 T=100 U=30 V=1000 H=128 tile={tile}")
    fp8_check(gpu_lib, inp, tile=tile, tpw=tpw)


def test_fp8_differs_from_bf16(gpu_lib):
    """The E4M3 product is really taken: the fp8 costs differ from the bf16 path's."""
    inp = make_inputs(3, 60, 20, 1024, 64, 64, 640, dtype="bf16", seed=163, t_range=(30, 60), u_range=(5, 20),
                      bias_std=0.1)
    c8, _ = run_fp8(gpu_lib, inp)
    prob = gpu_lib.Problem(inp, mode="tiled")
    c16 = prob.forward().clone().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(c8 - c16)) > 1e-4 * np.max(np.abs(c16))


@pytest.mark.timeout(400)
def test_fp8_small_workload(gpu_lib):
    say("fp8 small workload, full oracle comparison")
    fp8_check(gpu_lib, workload_inputs("small-bf16"))


@pytest.mark.timeout(400)
def test_fp8_vocab4096_sampled(gpu_lib):
    inp = workload_inputs("vocab4096-bf16")
    e = np.zeros(len(inp.T_len))
    e[2] = 1.0
    say("fp8 vocab4096, oracle on sample 2")
    costs, grads = run_fp8(gpu_lib, inp, tile=(32, 16), dcosts=e)
    ref = oracle.loss_and_grads(inp, dcosts=e, samples=[2], fp8_scores=True)
    check_costs(inp, costs, ref.costs, samples=[2])
    check_grads(inp, grads, ref.grads)
    distance_from_exact(inp, costs, grads, samples=[2], dcosts=e)


@pytest.mark.timeout(600)
def test_fp8_40s_b256(gpu_lib):
    inp = workload_inputs("40s-b256-bf16")
    say("fp8 40s-b256, W^O = 0: closed-form cost for every sample")
    inp0 = dataclasses.replace(inp, WO=np.zeros_like(inp.WO), bO=np.zeros_like(inp.bO))
    c0, _ = run_fp8(gpu_lib, inp0)
    V = inp.WO.shape[0]
    for b in range(len(inp.T_len)):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        want = (Tb + Ub) * math.log(V) - lnC(Tb + Ub - 1, Ub)
        assert abs(c0[b] - want) <= 1e-5 * want, (b, c0[b], want)
    say("fp8 40s-b256, oracle on sample 9")
    e = np.zeros(len(inp.T_len))
    e[9] = 1.0
    costs, grads = run_fp8(gpu_lib, inp, dcosts=e)
    ref = oracle.loss_and_grads(inp, dcosts=e, samples=[9], fp8_scores=True)
    check_costs(inp, costs, ref.costs, samples=[9])
    check_grads(inp, grads, ref.grads)
    distance_from_exact(inp, costs, grads, samples=[9], dcosts=e)


def test_fp8_with_pruned_lattice(gpu_lib):
    """The fp8 output layer on a pruned lattice (both options together) against the oracle with both."""
    import torch

    from rnnt_inputs import diagonal_band

    inp = make_inputs(3, 90, 37, 1024, 96, 64, 640, dtype="bf16", seed=181, t_range=(40, 90), u_range=(10, 37),
                      bias_std=0.1)
    S = 8
    lo = diagonal_band(inp.T_len, inp.U_len, 90, S)
    say("fp8 output layer on a pruned lattice, S = 8")
    prob = gpu_lib.Problem(inp, tile=(32, 16), tiles_per_wave=5, band=(lo, S), fp8=True)
    costs = prob.forward().clone().cpu().numpy().astype(np.float64)
    grads = {k: v.cpu().numpy().astype(np.float64) for k, v in prob.backward().items()}
    torch.cuda.synchronize()
    ref = oracle.loss_and_grads(inp, band=(lo, S), fp8_scores=True)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
