"""rnnt_loss_fwd_noalloc: the forward with the library's static scratch array as its workspace.

Through the C ABI, on two calls in a row (the second on a smaller batch), the allocation-free
forward gives the same costs as rnnt_loss_fwd bit for bit, and its `saved` drives rnnt_loss_bwd to
the same gradients bit for bit; device memory is not allocated by the call; a request whose
forward needs more than the array is refused before any launch; fp32 mode needs no scratch; the
fp8 output layer's forward and the untiled mode's forward run from the array as well.
"""
import numpy as np
import pytest

from rnnt_inputs import make_inputs

pytestmark = pytest.mark.gpu

GRADS = ("dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO")


def both_ways(rl, inp, tile=(64, 32), tpw=0, fp8=False, mode="tiled"):
    import torch

    prob = rl.Problem(inp, mode=mode, tile=tile, tiles_per_wave=tpw, fp8=fp8)
    ref_costs = prob.forward().clone()
    ref_grads = {k: v.clone() for k, v in prob.backward().items()}
    torch.cuda.synchronize()
    saved = torch.empty_like(prob.saved)
    costs = torch.full_like(prob.costs, float("nan"))
    free0 = torch.cuda.mem_get_info()[0]
    rl.rnnt_loss_fwd_noalloc(prob.desc, prob.hA, prob.hL, prob.labels, prob.T_len, prob.U_len, prob.WA, prob.WL,
                             prob.bZ, prob.WO, prob.bO, costs, saved)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    g = prob.grads
    rl.rnnt_loss_bwd(prob.desc, prob.hA, prob.hL, prob.labels, prob.T_len, prob.U_len, prob.WA, prob.WL, prob.bZ,
                     prob.WO, prob.bO, None, saved, prob.workspace, g["dhA"], g["dhL"], g["dWA"], g["dWL"],
                     g["dbZ"], g["dWO"], g["dbO"])
    torch.cuda.synchronize()
    assert torch.equal(costs.view(torch.int32), ref_costs.view(torch.int32))
    for k in GRADS:
        assert torch.equal(g[k].view(torch.int32), ref_grads[k].view(torch.int32)), k
    return free0, free1


def test_noalloc_forward_matches_forward(gpu_lib):
    rl = gpu_lib
    big = make_inputs(6, 200, 50, 1024, 512, 512, 640, dtype="bf16", seed=301, t_range=(120, 200),
                      u_range=(20, 50), bias_std=0.1)
    small = make_inputs(3, 90, 20, 700, 256, 192, 512, dtype="bf16", seed=302, t_range=(30, 90),
                        u_range=(0, 20), bias_std=0.1)
    print("noalloc forward: B=6 T=200 U=50 V=1024, then B=3 T=90 U=20 V=700", flush=True)
    both_ways(rl, big)
    free0, free1 = both_ways(rl, small, tile=(32, 16), tpw=5)
    assert free0 == free1, (free0, free1)  # the call itself allocates no device memory


def test_noalloc_forward_fp8(gpu_lib):
    """The fp8 output layer's forward (E4M3 W^O table and z rows in the scratch array)."""
    inp = make_inputs(4, 120, 30, 1024, 256, 192, 640, dtype="bf16", seed=304, t_range=(60, 120),
                      u_range=(5, 30), bias_std=0.1)
    print("noalloc forward: fp8 output layer", flush=True)
    both_ways(gpu_lib, inp, fp8=True)


def test_noalloc_forward_untiled(gpu_lib):
    """Untiled mode: the forward keeps the scores and z in `saved` (the score kernel's store
    path), its statistics and score tables in the scratch array; the backward forms dh from the
    kept scores in place."""
    inp = make_inputs(4, 120, 30, 1000, 256, 192, 640, dtype="bf16", seed=305, t_range=(60, 120),
                      u_range=(0, 30), bias_std=0.1)
    print("noalloc forward: untiled", flush=True)
    both_ways(gpu_lib, inp, mode="untiled")


def test_noalloc_forward_fp32_and_limit(gpu_lib):
    import torch

    rl = gpu_lib
    inp = make_inputs(3, 40, 12, 300, 64, 48, 64, dtype="f32", seed=303, t_range=(10, 40), u_range=(0, 12),
                      bias_std=0.2)
    print("noalloc forward: fp32", flush=True)
    both_ways(rl, inp, tile=(32, 8))
    # the 40 s x 256 shape at the default wave size needs ~0.7 GB of forward scratch: refused
    # (every buffer has its full size, so nothing could be addressed out of bounds either way)
    B, T, U, V, H = 256, 1000, 200, 1024, 640
    d = rl.make_desc(B, T, U, V, 512, 512, H)
    T_len, U_len = np.full(B, T, np.int32), np.full(B, U, np.int32)
    s, _ = rl.rnnt_loss_query(d, T_len, U_len)
    z = lambda *shape: torch.zeros(*shape, dtype=torch.bfloat16, device="cuda")
    hA, hL, WA, WL, bZ, WO, bO = z(B, T, 512), z(B, U + 1, 512), z(H, 512), z(H, 512), z(H), z(V, H), z(V)
    labels = torch.zeros(B, U + 1, dtype=torch.int32, device="cuda")
    costs = torch.empty(B, device="cuda")
    saved = torch.empty(s, dtype=torch.uint8, device="cuda")
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_loss_fwd_noalloc(d, hA, hL, labels, T_len, U_len, WA, WL, bZ, WO, bO, costs, saved)
    assert e.value.status == rl.RNNT_E_WORKSPACE and "scratch" in str(e.value)
