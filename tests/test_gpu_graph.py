"""The forward and backward captured into a HIP graph and replayed.

One problem's fwd+bwd is captured (torch.cuda.graph: the library's launches and its plan copy
go to the capture stream) and the graph is replayed three times. Before each replay the program
runs, eagerly, the forward and backward of another problem with another plan (so the plan
staging slots and, for the allocation-free forward, the static scratch array are reused in
between) and synchronises; every replay must give the eager results bit for bit. Covered: bf16
tiled, bf16 untiled, the allocation-free forward and the fp8 output layer.
"""
import numpy as np
import pytest

from rnnt_inputs import make_inputs
from test_gpu_parity import say

pytestmark = pytest.mark.gpu

GRADS = ("dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO")


def fwd_bwd(rl, prob, noalloc):
    if noalloc:
        rl.rnnt_loss_fwd_noalloc(prob.desc, prob.hA, prob.hL, prob.labels, prob.T_len, prob.U_len, prob.WA, prob.WL,
                                 prob.bZ, prob.WO, prob.bO, prob.costs, prob.saved)
    else:
        prob.forward()
    prob.backward()


def graph_replays(rl, mode="tiled", fp8=False, noalloc=False):
    import torch

    inp = make_inputs(4, 120, 30, 1000, 256, 192, 640, dtype="bf16", seed=401, t_range=(60, 120),
                      u_range=(0, 30), bias_std=0.1)
    other_inp = make_inputs(3, 90, 20, 1000, 256, 192, 640, dtype="bf16", seed=402, t_range=(30, 90),
                            u_range=(5, 20), bias_std=0.1)
    prob = rl.Problem(inp, mode=mode, tile=(32, 16), fp8=fp8)
    other = rl.Problem(other_inp, mode=mode, tile=(64, 32), fp8=fp8)
    fwd_bwd(rl, prob, noalloc)
    torch.cuda.synchronize()
    ref_costs = prob.costs.clone()
    ref_grads = {k: prob.grads[k].clone() for k in GRADS}
    # warm-up on a side stream, then the capture (torch's recipe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd_bwd(rl, prob, noalloc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd_bwd(rl, prob, noalloc)
    torch.cuda.synchronize()
    for rep in range(3):
        prob.costs.fill_(float("nan"))
        for k in GRADS:
            prob.grads[k].fill_(float("nan"))
        fwd_bwd(rl, other, noalloc)  # eager work with another plan between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(prob.costs.view(torch.int32), ref_costs.view(torch.int32)), f"replay {rep}: costs"
        for k in GRADS:
            assert torch.equal(prob.grads[k].view(torch.int32), ref_grads[k].view(torch.int32)), f"replay {rep}: {k}"
    del graph


@pytest.mark.parametrize("mode,fp8,noalloc", [("tiled", False, False), ("untiled", False, False),
                                              ("tiled", False, True), ("tiled", True, False)],
                         ids=["bf16-tiled", "bf16-untiled", "noalloc-forward", "fp8-tiled"])
def test_graph_replay_matches_eager(gpu_lib, mode, fp8, noalloc):
    say(f"graph capture and replay: {mode}{' fp8' if fp8 else ''}{' no-alloc forward' if noalloc else ''}")
    graph_replays(gpu_lib, mode=mode, fp8=fp8, noalloc=noalloc)
