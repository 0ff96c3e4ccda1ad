"""Randomised parity sweep: many small problems with drawn shapes and options against the oracle.

Each case draws (from a fixed seed, so the sweep is the same every run) the batch size, lengths
(ragged, including T_b = 1 and U_b = 0), vocabulary size (not a multiple of 256), hidden sizes,
blank id, the mode (tiled / untiled), the dtype (fp32, bf16, bf16 with the fp8 output layer),
the tile shape and tiles per wave, optionally a pruned lattice, and non-unit upstream gradients,
then compares every cost and gradient with the fp64 oracle at the dtype's tolerances (the fp8
cases against the oracle's fp8 reading). Sizes keep the oracle at about a second per case. A
second sweep draws bf16 untiled problems with H >= 512 only: the persistent forward score kernel
with its score store and the backward's dh formed in place of the kept scores.
"""
import numpy as np
import pytest

import oracle
from rnnt_inputs import diagonal_band, make_inputs
from test_gpu_parity import check_costs, check_grads, say

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    B = int(rng.integers(1, 7))
    T = int(rng.integers(1, 120))
    U = int(rng.integers(0, 64))
    V = int(rng.choice([7, 50, 300, 513, 1000, 1030, 2100]))
    H = int(rng.choice([8, 64, 136, 256, 520, 640, 768]))
    HA, HL = int(rng.choice([8, 64, 96])), int(rng.choice([8, 40, 64]))
    kind = ["f32", "bf16", "fp8"][i % 3]
    mode = "untiled" if (kind != "fp8" and rng.random() < 0.3) else "tiled"
    tile = (int(rng.integers(1, 80)), int(rng.integers(1, 40)))
    tpw = int(rng.choice([0, 1, 2, 5]))
    blank = int(rng.choice([0, 0, V - 1, V // 2]))
    pruned = rng.random() < 0.3 and mode == "tiled"
    inp = make_inputs(B, T, U, V, HA, HL, H, dtype="f32" if kind == "f32" else "bf16", seed=2000 + i,
                      t_range=(1, T), u_range=(0, U), bias_std=0.2, blank=blank)
    dcosts = rng.uniform(-1.5, 2.0, B)
    return inp, kind, mode, tile, tpw, pruned, dcosts


def draw_untiled_case(i):
    rng = np.random.default_rng(4000 + i)
    B = int(rng.integers(1, 7))
    T = int(rng.integers(1, 120))
    U = int(rng.integers(0, 64))
    V = int(rng.choice([7, 300, 513, 1000, 1024, 1030, 2100]))
    H = int(rng.choice([512, 520, 640, 768]))
    HA, HL = int(rng.choice([8, 64, 96])), int(rng.choice([8, 40, 64]))
    blank = int(rng.choice([0, V - 1, V // 2]))
    pruned = rng.random() < 0.3
    inp = make_inputs(B, T, U, V, HA, HL, H, dtype="bf16", seed=5000 + i, t_range=(1, T), u_range=(0, U),
                      bias_std=0.2, blank=blank)
    dcosts = rng.uniform(-1.5, 2.0, B)
    return inp, "bf16", "untiled", (64, 32), 0, pruned, dcosts


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(gpu_lib, i):
    run_case(gpu_lib, i, *draw_case(i))


@pytest.mark.parametrize("i", range(16))
def test_random_untiled_case(gpu_lib, i):
    run_case(gpu_lib, 1000 + i, *draw_untiled_case(i))


def run_case(gpu_lib, i, inp, kind, mode, tile, tpw, pruned, dcosts):
    import torch

    B, T, _ = inp.hA.shape
    U = inp.hL.shape[1] - 1
    V, H = inp.WO.shape
    band = None
    if pruned:
        S = int(np.random.default_rng(3000 + i).integers(2, 8))
        try:
            band = (diagonal_band(inp.T_len, inp.U_len, T, S), S)
        except ValueError:
            band = None  # this width cannot hold an alignment of some sample
    say(f"case {i}: B={B} T={T} U={U} V={V} H={H} {kind} {mode} tile={tile} tpw={tpw} blank={inp.blank}"
        f" band={None if band is None else band[1]} T_len={list(inp.T_len)} U_len={list(inp.U_len)}")
    prob = gpu_lib.Problem(inp, mode=mode, tile=tile, tiles_per_wave=tpw, band=band, fp8=kind == "fp8")
    costs = prob.forward().clone()
    dc = torch.tensor(dcosts.astype(np.float32), device=prob.device)
    grads = prob.backward(dc)
    torch.cuda.synchronize()
    costs = costs.cpu().numpy().astype(np.float64)
    grads = {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    ref = oracle.loss_and_grads(inp, dcosts=dcosts, band=band, fp8_scores=kind == "fp8")
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
