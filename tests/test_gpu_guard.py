"""Guard bytes around every buffer the library writes: the kernels stay inside the bytes the
query declares.

`saved`, `workspace`, the costs and the seven gradient outputs are each placed inside a larger
device allocation with 64 KiB of a byte pattern before and after; after a forward and a
backward the pattern must be intact (and the results must still match the oracle, so the
buffers were really used). Covered: bf16 tiled (two tile shapes, ragged lengths), bf16
untiled (both score kernels), fp32 tiled, the fp8 output layer and a pruned lattice.
"""
import numpy as np
import pytest

import oracle
from rnnt_inputs import diagonal_band, make_inputs
from test_gpu_parity import check_costs, check_grads, say

pytestmark = pytest.mark.gpu

GUARD = 64 << 10
PATTERN = 0xA5


class Guarded:
    """A device byte buffer of n bytes with GUARD pattern bytes on both sides."""

    def __init__(self, torch, n, dev):
        self.n = max(int(n), 1)
        self.raw = torch.full((self.n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device=dev)
        self.body = self.raw[GUARD:GUARD + self.n]

    def view(self, torch, dtype, shape):
        return self.body.view(dtype)[:int(np.prod(shape))].view(*shape)

    def intact(self):
        lo, hi = self.raw[:GUARD], self.raw[GUARD + self.n:]
        return bool((lo == PATTERN).all()) and bool((hi == PATTERN).all())


def run_guarded(rl, inp, mode="tiled", tile=(64, 32), tpw=0, fp8=False, band=None):
    import torch

    dev = torch.device("cuda:0")
    B, T, HA = inp.hA.shape
    U1, HL = inp.hL.shape[1], inp.hL.shape[2]
    V, H = inp.WO.shape
    dtype = "bf16-fp8" if fp8 else inp.dtype
    d = rl.make_desc(B, T, U1 - 1, V, HA, HL, H, blank=int(inp.blank), dtype=dtype, mode=mode, tile=tile,
                     tiles_per_wave=tpw)
    if band is None:
        s_bytes, w_bytes = rl.rnnt_loss_query(d, inp.T_len, inp.U_len)
    else:
        s_bytes, w_bytes = rl.rnnt_loss_query_pruned(d, inp.T_len, inp.U_len, *band)
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(tdt)
    hA, hL, WA, WL, bZ, WO, bO = map(up, (inp.hA, inp.hL, inp.WA, inp.WL, inp.bZ, inp.WO, inp.bO))
    labels = torch.from_numpy(np.ascontiguousarray(inp.labels, dtype=np.int32)).to(dev)
    saved, ws = Guarded(torch, s_bytes, dev), Guarded(torch, w_bytes, dev)
    shapes = dict(costs=(B,), dhA=(B, T, HA), dhL=(B, U1, HL), dWA=(H, HA), dWL=(H, HL), dbZ=(H,), dWO=(V, H),
                  dbO=(V,))
    outs = {k: Guarded(torch, 4 * int(np.prod(s)), dev) for k, s in shapes.items()}
    t = {k: g.view(torch, torch.float32, shapes[k]) for k, g in outs.items()}
    sv, wv = saved.body, ws.body
    if band is None:
        rl.rnnt_loss_fwd(d, hA, hL, labels, inp.T_len, inp.U_len, WA, WL, bZ, WO, bO, t["costs"], sv, wv)
        rl.rnnt_loss_bwd(d, hA, hL, labels, inp.T_len, inp.U_len, WA, WL, bZ, WO, bO, None, sv, wv, t["dhA"],
                         t["dhL"], t["dWA"], t["dWL"], t["dbZ"], t["dWO"], t["dbO"])
    else:
        rl.rnnt_loss_fwd_pruned(d, hA, hL, labels, inp.T_len, inp.U_len, *band, WA, WL, bZ, WO, bO, t["costs"], sv,
                                wv)
        rl.rnnt_loss_bwd_pruned(d, hA, hL, labels, inp.T_len, inp.U_len, *band, WA, WL, bZ, WO, bO, None, sv, wv,
                                t["dhA"], t["dhL"], t["dWA"], t["dWL"], t["dbZ"], t["dWO"], t["dbO"])
    torch.cuda.synchronize()
    for name, g in [("saved", saved), ("workspace", ws)] + list(outs.items()):
        assert g.intact(), f"a kernel wrote outside {name}"
    costs = t["costs"].cpu().numpy().astype(np.float64)
    grads = {k: t[k].cpu().numpy().astype(np.float64) for k in shapes if k != "costs"}
    return costs, grads


CASES = [
    ("bf16 tiled 64x32", dict(dtype="bf16"), dict(), 128),
    ("bf16 tiled 20x7, 3 tiles per wave", dict(dtype="bf16"), dict(tile=(20, 7), tpw=3), 128),
    ("bf16 untiled", dict(dtype="bf16"), dict(mode="untiled"), 128),
    # H = 640: the persistent forward score kernel stores the scores; its last cell tile
    # reads the padding rows after the z rows kept in `saved`
    ("bf16 untiled, persistent score kernel", dict(dtype="bf16"), dict(mode="untiled"), 640),
    ("fp32 tiled 32x16", dict(dtype="f32"), dict(tile=(32, 16), tpw=5), 128),
    ("fp8 output layer", dict(dtype="bf16"), dict(fp8=True), 640),
]


@pytest.mark.parametrize("name,inkw,kw,H", CASES, ids=[c[0] for c in CASES])
def test_writes_stay_inside_declared_buffers(gpu_lib, name, inkw, kw, H):
    inp = make_inputs(3, 90, 37, 700, 96, 64, H, seed=171, t_range=(30, 90), u_range=(0, 37), bias_std=0.1, **inkw)
    say(f"guard bytes: {name}")
    costs, grads = run_guarded(gpu_lib, inp, **kw)
    ref = oracle.loss_and_grads(inp, fp8_scores=bool(kw.get("fp8")))
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


def test_pruned_writes_stay_inside_declared_buffers(gpu_lib):
    inp = make_inputs(3, 90, 37, 700, 96, 64, 128, dtype="bf16", seed=173, t_range=(30, 90), u_range=(5, 37),
                      bias_std=0.1)
    lo = diagonal_band(inp.T_len, inp.U_len, 90, 6)
    say("guard bytes: pruned lattice, S = 6")
    costs, grads = run_guarded(gpu_lib, inp, tile=(32, 16), band=(lo, 6))
    ref = oracle.loss_and_grads(inp, band=(lo, 6))
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
