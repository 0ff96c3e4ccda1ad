"""Parity of the HIP library with the fp64 oracle, through the C ABI.

Tolerances (per sample cost; per gradient tensor relative to its max-abs):
  fp32 mode: cost 1e-5 relative, gradients 1e-4 of max-abs
  bf16 mode: cost 2e-3 relative, gradients 2e-2 of max-abs
Padded gradient rows must be exactly 0. At the full sizes of the large
workloads the oracle computes a few samples, selected on the GPU side by a
one-hot upstream gradient (the gradients are linear in dcosts), and closed
forms (W^O = 0) check every sample's cost.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from rnnt_inputs import make_inputs, poison_padding, workload_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 2e-2)}
GRADS = ("dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(rl, inp, mode="tiled", tile=(64, 32), tpw=0, dcosts=None):
    import torch

    prob = rl.Problem(inp, mode=mode, tile=tile, tiles_per_wave=tpw)
    costs = prob.forward().clone()
    dc = None if dcosts is None else torch.tensor(np.asarray(dcosts, np.float32), device=prob.device)
    grads = prob.backward(dc)
    torch.cuda.synchronize()
    out = costs.cpu().numpy().astype(np.float64), {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}
    del prob
    return out


def check_costs(inp, got, ref, samples=None):
    rc, _ = TOL[inp.dtype]
    idx = range(len(ref)) if samples is None else samples
    worst = 0.0
    for b in idx:
        err = abs(got[b] - ref[b]) / abs(ref[b])
        worst = max(worst, err)
        assert err <= rc, f"sample {b}: cost {got[b]} vs {ref[b]} (rel {err:.2e})"
    say(f"  parity: cost max rel err {worst:.2e} (tolerance {rc:g})")


def check_grads(inp, got, ref):
    _, rg = TOL[inp.dtype]
    errs = {}
    for k in GRADS:
        scale = np.max(np.abs(ref[k]))
        err = np.max(np.abs(got[k] - ref[k]))
        errs[k] = err / max(scale, 1e-30)
        assert err <= rg * max(scale, 1e-30), f"{k}: max err {err:.3e} vs max-abs {scale:.3e}"
    say("  parity: grad err / max-abs " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()) + f" (tolerance {rg:g})")
    for b in range(len(inp.T_len)):
        assert np.all(got["dhA"][b, inp.T_len[b]:] == 0), "padded dhA rows"
        assert np.all(got["dhL"][b, inp.U_len[b] + 1:] == 0), "padded dhL rows"


def full_check(rl, inp, **kw):
    ref = oracle.loss_and_grads(inp)
    costs, grads = run_gpu(rl, inp, **kw)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)
    return costs, grads


def sampled_check(rl, inp, samples, **kw):
    """GPU at full size with a one-hot upstream gradient per sample."""
    B = len(inp.T_len)
    for b in samples:
        e = np.zeros(B)
        e[b] = 1.0
        say(f"  sample {b}: T_b={inp.T_len[b]} U_b={inp.U_len[b]}")
        costs, grads = run_gpu(rl, inp, dcosts=e, **kw)
        ref = oracle.loss_and_grads(inp, dcosts=e, samples=[b])
        check_costs(inp, costs, ref.costs, samples=[b])
        check_grads(inp, grads, ref.grads)
    return costs


def lnC(n, k):
    return math.lgamma(n + 1) - math.lgamma(k + 1) - math.lgamma(n - k + 1)


# ----------------------------------------------------------------------------- lattice kernel alone

# (T, U, T range, U range): the kernel variant lattice_kernel<NW, SW> is chosen by U + 1 in waves
# of 64 rows: 1, 2, 3, 4, 6, 8, 12 and 16 waves, the last at the library's limit U + 1 = 1024; the
# U ranges make rows beyond the first lane group live so neighbours cross lane groups.
LATTICE_CASES = [(70, 40, (1, 70), (0, 40)), (90, 100, (1, 90), (64, 100)),
                 (60, 170, (1, 60), (128, 170)), (50, 255, (1, 50), (192, 255)),
                 (40, 300, (1, 40), (250, 300)), (20, 450, (1, 20), (400, 450)),
                 (24, 700, (1, 24), (500, 700)), (16, 900, (1, 16), (800, 900)),
                 (8, 1023, (1, 8), (1000, 1023))]


def lattice_tol(ref):
    """Per-element bound for an fp32 sweep: relative 1e-5 of the value (rounding accumulated along
    the T_b + U_b steps) plus 1e-4 absolute (the log-add-exp increments)."""
    return 1e-5 * np.abs(ref) + 1e-4


def lattice_layout(B, T, U1):
    """Entries of the documented lattice layout and its index function: cell (t, u) of sample b,
    on diagonal d = t + u, is entry ((b * NQ + d // 4) * US + u) * 4 + d % 4 with
    NQ = ceil((T + U1 - 1) / 4) groups of four diagonals and US = U1 rounded up to 32."""
    NQ, US = (T + U1 - 1 + 3) // 4, (U1 + 31) // 32 * 32

    def ix(b, t, u):
        d = t + u
        return ((b * NQ + d // 4) * US + u) * 4 + d % 4

    return B * NQ * US * 4, ix


@pytest.mark.parametrize("T,U,tr,ur", LATTICE_CASES)
def test_lattice_kernel_matches_oracle(gpu_lib, T, U, tr, ur):
    lattice_vs_oracle(gpu_lib, 5, T, U, tr, ur)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paired_sweeps_of_different_samples(gpu_lib, dtype):
    """Through the loss with B = 160 (more sweeps than CUs): workgroup j sweeps alpha of the j-th
    longest sample and beta of the j-th shortest, three waves each (U + 1 <= 192), with ragged
    lengths so that the halves end at different steps; costs and gradients against the oracle."""
    inp = make_inputs(160, 40, 150, 33, 16, 16, 16, dtype=dtype, seed=707, t_range=(1, 40), u_range=(0, 150))
    say(f"paired sweeps of different samples {dtype}: B=160 T<=40 U<=150")
    full_check(gpu_lib, inp)


@pytest.mark.parametrize("T,U,tr,ur", LATTICE_CASES[:4])
def test_lattice_paired_sweeps_match_oracle(gpu_lib, T, U, tr, ur):
    """More sweeps than CUs (B = 160 on 256 CUs): the paired kernel, one workgroup running an alpha
    and a beta sweep of 1 to 4 waves each. Through rnnt_lattice (no host lengths, so no pairing
    table) both halves sweep the same sample; the loss's pairing of long with short samples, whose
    halves end at different steps, is checked by the B = 1024 and 40 s x 256 tests."""
    lattice_vs_oracle(gpu_lib, 160, T, U, (1, T), (0, U))


def lattice_vs_oracle(rl, B, T, U, tr, ur):
    import torch

    U1 = U + 1
    n, ix_of = lattice_layout(B, T, U1)
    inp = make_inputs(B, T, U, 33, 8, 8, 8, dtype="f32", seed=31 + U, t_range=tr, u_range=ur)
    say(f"lattice kernel: B={B} T={T} U={U} ragged")
    r = oracle.loss_and_grads(inp, want_grads=False)
    # entries outside every lattice hold poison the kernel must not let through
    rng = np.random.default_rng(U)
    poison = np.array([np.nan, np.inf, -np.inf, 1e30, -1e30, 7.0], np.float32)
    phi = rng.choice(poison, size=n).astype(np.float32)
    psi = rng.choice(poison, size=n).astype(np.float32)
    cells = []
    for b, s in enumerate(r.samples):
        Tb, Ub = inp.T_len[b], inp.U_len[b]
        t, u = np.meshgrid(np.arange(Tb), np.arange(Ub + 1), indexing="ij")
        ix = ix_of(b, t, u)
        cells.append(ix)
        phi[ix] = s.phi
        psi[ix[:, :Ub]] = s.psi[:, :Ub]
    dev = torch.device("cuda:0")
    tp = lambda a: torch.from_numpy(a).to(dev)
    al = torch.full((n,), 7.0, device=dev)
    be = torch.full((n,), 7.0, device=dev)
    costs = torch.zeros(B, device=dev)
    d = rl.make_desc(B, T, U, 33, 8, 8, 8)
    rl.rnnt_lattice(d, tp(inp.T_len), tp(inp.U_len), tp(phi), tp(psi), al, be, costs)
    torch.cuda.synchronize()
    al, be, costs = al.cpu().numpy(), be.cpu().numpy(), costs.cpu().numpy()
    touched = np.zeros(n, bool)
    for b, s in enumerate(r.samples):
        Tb, Ub = inp.T_len[b], inp.U_len[b]
        ix = cells[b]
        touched[ix] = True
        assert abs(costs[b] - s.cost) <= 1e-5 * abs(s.cost), f"sample {b}"
        for name, got, ref in (("alpha", al[ix], s.alpha), ("beta", be[ix], s.beta)):
            excess = np.abs(got - ref) - lattice_tol(ref)
            k = np.unravel_index(np.argmax(excess), ref.shape)
            assert excess[k] <= 0, f"{name}, sample {b}, (t, u) = {k}: {got[k]} vs {ref[k]}"
    # entries outside the lattices are untouched
    assert np.all(al[~touched] == 7.0) and np.all(be[~touched] == 7.0)


def test_lattice_large_bitwise_reproducible(gpu_lib):
    """At the 40 s workload's lattice shape (B=256, T=1000, U=200, ragged), two sweeps over the
    same phi / psi give bit-identical alpha, beta and costs, and every lattice cell is written
    (finite). Guards the sweep's cross-wave hand-over and load waits, which a wrong schedule
    breaks only under full-GPU concurrency."""
    import torch

    rl = gpu_lib
    B, T, U = 256, 1000, 200
    U1 = U + 1
    n, ix_of = lattice_layout(B, T, U1)
    rng = np.random.default_rng(2026)
    T_len = rng.integers(500, T + 1, B).astype(np.int32)
    U_len = rng.integers(100, U + 1, B).astype(np.int32)
    say(f"lattice B={B} T={T} U={U}: two sweeps, bitwise")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    phi = torch.empty(n, device=dev).uniform_(-4.5, -2.5, generator=g)
    psi = torch.empty(n, device=dev).uniform_(-4.5, -2.5, generator=g)
    Tl, Ul = torch.from_numpy(T_len).to(dev), torch.from_numpy(U_len).to(dev)
    d = rl.make_desc(B, T, U, 33, 8, 8, 8)
    runs = []
    for _ in range(2):
        al = torch.full((n,), float("nan"), device=dev)
        be = torch.full((n,), float("nan"), device=dev)
        costs = torch.zeros(B, device=dev)
        rl.rnnt_lattice(d, Tl, Ul, phi, psi, al, be, costs)
        torch.cuda.synchronize()
        runs.append((al.view(torch.int32), be.view(torch.int32), costs.view(torch.int32)))
    # lattice cells: (b, t, u) with t < T_b, u <= U_b
    bi = torch.arange(B, device=dev)[:, None, None]
    ti = torch.arange(T, device=dev)[None, :, None]
    ui = torch.arange(U1, device=dev)[None, None, :]
    cell = (ti < Tl.long()[:, None, None]) & (ui <= Ul.long()[:, None, None])
    ix = ix_of(bi, ti, ui).expand(B, T, U1)[cell]
    assert int(ix.numel()) == int((T_len.astype(np.int64) * (U_len + 1)).sum())
    is_cell = torch.zeros(n, dtype=torch.bool, device=dev)
    is_cell[ix] = True

    def where(k):
        # the (b, t, u) of entry k of the layout, or why it is not a lattice cell
        NQ, US = (T + U1 - 1 + 3) // 4, (U1 + 31) // 32 * 32
        b, r = divmod(k, NQ * US * 4)
        q, r = divmod(r, US * 4)
        u, e = divmod(r, 4)
        t = 4 * q + e - u
        kind = "cell" if bool(is_cell[k]) else "not a cell"
        return f"entry {k}: sample {b}, t {t}, u {u} ({kind})"

    for name, x, y in zip(("alpha", "beta"), runs[0][:2], runs[1][:2]):
        diff = (x != y).nonzero()
        assert diff.numel() == 0, f"{name} differs between the sweeps first at {where(int(diff[0]))}"
        # only the lattice cells are written: every other entry keeps the NaN fill
        untouched = x[~is_cell].view(torch.float32)
        assert bool(torch.isnan(untouched).all()), f"{name}: an entry outside the lattices was written"
    assert torch.equal(runs[0][2], runs[1][2]), "costs differ between the sweeps"
    al, be = runs[0][0].view(torch.float32), runs[0][1].view(torch.float32)
    assert bool(torch.isfinite(al[ix]).all()) and bool(torch.isfinite(be[ix]).all())
    assert bool(torch.isfinite(runs[0][2].view(torch.float32)).all())


# ----------------------------------------------------------------------------- fp32 mode

@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_tiny_fp32(gpu_lib, mode):
    say(f"tiny fp32 {mode}")
    full_check(gpu_lib, workload_inputs("tiny-f32"), mode=mode)


@pytest.mark.parametrize("mode,tile,tpw", [("tiled", (32, 16), 3), ("tiled", (64, 32), 0),
                                           ("untiled", (32, 16), 0), ("tiled", (20, 7), 2)])
def test_fp32_ragged_multitile(gpu_lib, mode, tile, tpw):
    inp = make_inputs(3, 75, 41, 300, 48, 40, 64, dtype="f32", seed=41, t_range=(20, 75),
                      u_range=(0, 41), bias_std=0.3)
    say(f"fp32 ragged B=3 T=75 U=41 V=300 {mode} tile={tile} tpw={tpw}")
    full_check(gpu_lib, inp, mode=mode, tile=tile, tpw=tpw)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_fp32_small_workload_shapes(gpu_lib, mode):
    """fp32 mode at the small workload's shapes (B=8, T=250, U=64, V=1024, H_A=H_L=512, H=640, ragged
    lengths), costs to 1e-5 relative and every gradient to 1e-4 of max-abs. alpha and beta reach
    thousands of nats here: held in fp32 their spacing (~2.4e-4) alone would put the occupancies
    exp(alpha + beta - ln P) outside 1e-4, so fp32 mode carries the lattice in fp64."""
    inp = make_inputs(8, 250, 64, 1024, 512, 512, 640, dtype="f32", seed=12, t_range=(150, 250),
                      u_range=(32, 64))
    say(f"fp32 small-workload shapes {mode}")
    ref = oracle.loss_and_grads(inp)
    costs, grads = run_gpu(gpu_lib, inp, mode=mode)
    check_costs(inp, costs, ref.costs)
    for k in GRADS:
        rel = float(np.max(np.abs(grads[k] - ref.grads[k])) / np.max(np.abs(ref.grads[k])))
        say(f"  {k} err / max-abs {rel:.2e}")
        assert rel <= TOL["f32"][1], f"{k}: {rel:.3e} of max-abs"
    for b in range(len(inp.T_len)):
        assert np.all(grads["dhA"][b, inp.T_len[b]:] == 0) and np.all(grads["dhL"][b, inp.U_len[b] + 1:] == 0)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_fp32_long_lattice(gpu_lib, mode):
    """fp32 mode on lattices as long as the 40 s workload's (T_b up to 1000) with more label rows
    than the fp64 sweep's workgroup has threads (U_b in 257..300), V and H kept narrow so the oracle
    stays quick. Costs reach ~3.4e3 nats: costs to 1e-5 relative, gradients to 1e-4 of max-abs."""
    inp = make_inputs(3, 1000, 300, 48, 32, 32, 32, dtype="f32", seed=17, t_range=(700, 1000),
                      u_range=(257, 300))
    say(f"fp32 long lattice B=3 T=1000 U=300 V=48 {mode}")
    full_check(gpu_lib, inp, mode=mode)


# ----------------------------------------------------------------------------- bf16 mode

@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_bf16_reduced(gpu_lib, mode):
    inp = make_inputs(4, 100, 30, 1000, 128, 96, 128, dtype="bf16", seed=51, t_range=(40, 100),
                      u_range=(0, 30), bias_std=0.1)
    say(f"bf16 reduced B=4 T=100 U=30 V=1000 {mode}")
    full_check(gpu_lib, inp, mode=mode, tile=(32, 16), tpw=5)


def test_bf16_weighted_dcosts(gpu_lib):
    """Per-sample upstream gradients of mixed sign and size (a weighted, partly negated sum): every
    gradient term carries the sample's g_b, including the blank / label terms of dh."""
    inp = make_inputs(5, 60, 18, 400, 64, 48, 96, dtype="bf16", seed=57, t_range=(10, 60), u_range=(0, 18),
                      bias_std=0.1)
    dc = np.array([0.5, -1.25, 2.0, 0.0, 1.0 / 3.0])
    say("bf16 weighted dcosts B=5 T=60 U=18 V=400")
    ref = oracle.loss_and_grads(inp, dcosts=dc)
    costs, grads = run_gpu(gpu_lib, inp, tile=(32, 8), tpw=3, dcosts=dc)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


@pytest.mark.parametrize("H", [320, 448])
def test_bf16_dwo_column_tiles(gpu_lib, H):
    """dW^O / db^O output tilings: H = 320 leaves a 64-column remainder (512 x 128 tiles over
    V = 700, the last one partial in V), H = 448 a 192-column one (a partial 256 x 256 tile)."""
    inp = make_inputs(3, 70, 24, 700, 64, 96, H, dtype="bf16", seed=81 + H, t_range=(20, 70),
                      u_range=(0, 24), bias_std=0.1)
    say(f"bf16 dW^O tiles B=3 T=70 U=24 V=700 H={H}")
    full_check(gpu_lib, inp, mode="tiled", tile=(32, 16), tpw=4)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_small_full(gpu_lib, mode):
    say(f"small full bf16 {mode}")
    full_check(gpu_lib, workload_inputs("small-bf16"), mode=mode)


@pytest.mark.timeout(400)
def test_sample_wise_waves_from_budget(gpu_lib):
    """Whole-sample tiles ([N] section "Sample-wise method") with the wave size
    chosen from a memory budget: a few samples per wave."""
    rl = gpu_lib
    inp = workload_inputs("small-bf16")
    B, T, HA = inp.hA.shape
    U = inp.hL.shape[1] - 1
    V, H = inp.WO.shape
    tile = (T, U + 1)
    one = rl.make_desc(B, T, U, V, HA, inp.hL.shape[2], H, tile=tile, tiles_per_wave=1)
    s1, w1 = rl.rnnt_loss_query(one, inp.T_len, inp.U_len)
    d = rl.make_desc(B, T, U, V, HA, inp.hL.shape[2], H, tile=tile)
    n = rl.rnnt_waves_for_budget(d, inp.T_len, inp.U_len, int((s1 + w1) * 1.6))
    assert 1 < n < B
    say(f"sample-wise tiles {tile}, {n} samples per wave")
    full_check(rl, inp, tile=tile, tpw=n)


def closed_form_costs(rl, inp, **kw):
    """W^O = 0 and b^O = 0 (every softmax row uniform, 1/V): every alignment has probability
    V^-(T_b + U_b), so cost_b = (T_b + U_b) ln V - ln C(T_b + U_b - 1, U_b), for every sample of
    the batch, at the workload's full size ("Neural transducer training ...", Eqs. (8)-(9))."""
    import dataclasses

    inp0 = dataclasses.replace(inp, WO=np.zeros_like(inp.WO), bO=np.zeros_like(inp.bO))
    c0, _ = run_gpu(rl, inp0, **kw)
    V = inp.WO.shape[0]
    for b in range(len(inp0.T_len)):
        Tb, Ub = int(inp0.T_len[b]), int(inp0.U_len[b])
        want = (Tb + Ub) * math.log(V) - lnC(Tb + Ub - 1, Ub)
        assert abs(c0[b] - want) <= 1e-5 * want, (b, c0[b], want)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("mode", ["tiled", "untiled"])
def test_20s_closed_form_every_sample(gpu_lib, mode):
    say(f"20s full bf16 {mode}, W^O = 0: closed-form cost for every sample")
    closed_form_costs(gpu_lib, workload_inputs("20s-bf16"), mode=mode)


@pytest.mark.timeout(400)
def test_20s_untiled_sampled(gpu_lib):
    inp = workload_inputs("20s-bf16")
    say("20s full bf16 untiled, sampled oracle")
    sampled_check(gpu_lib, inp, [0], mode="untiled")


@pytest.mark.timeout(400)
def test_20s_sampled_tiled_and_untiled(gpu_lib):
    inp = workload_inputs("20s-bf16")
    say("20s full bf16 tiled 64x32, sampled oracle")
    ct = sampled_check(gpu_lib, inp, [0, 17])
    say("20s untiled vs tiled")
    cu, gu = run_gpu(gpu_lib, inp, mode="untiled")
    c2, g2 = run_gpu(gpu_lib, inp)
    say("20s tiled twice: bitwise")
    c3, g3 = run_gpu(gpu_lib, inp)
    # ordered reductions only (no float atomics): a second run gives the same bits
    assert np.array_equal(c2, c3)
    for k in GRADS:
        assert np.array_equal(g2[k], g3[k]), k
    # same equations; the tiled forward accumulates the per-V-tile (max, sum)
    # block by block, the untiled one per 256-score tile, so only the
    # summation order differs
    assert np.allclose(cu, c2, rtol=1e-5, atol=0), np.max(np.abs(cu - c2) / np.abs(c2))
    for k in GRADS:
        assert np.max(np.abs(gu[k] - g2[k])) <= 1e-2 * np.max(np.abs(g2[k])), k


@pytest.mark.timeout(600)
def test_vocab4096_tile_sweep(gpu_lib):
    inp = workload_inputs("vocab4096-bf16")
    results = {}
    for tile in ((32, 16), (64, 32), (128, 64)):
        say(f"vocab4096 bf16 tile {tile}")
        results[tile] = run_gpu(gpu_lib, inp, tile=tile)
    base_c, base_g = results[(64, 32)]
    for tile, (c, g) in results.items():
        assert np.array_equal(c, base_c), tile  # costs do not depend on the tile size
        for k in GRADS:
            assert np.max(np.abs(g[k] - base_g[k])) <= 1e-2 * np.max(np.abs(base_g[k])), (tile, k)
    say("vocab4096 sampled oracle")
    sampled_check(gpu_lib, inp, [3], tile=(32, 16))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tile,sample", [((64, 32), 8), ((128, 64), 13)])
def test_vocab4096_tiles_sampled(gpu_lib, tile, sample):
    inp = workload_inputs("vocab4096-bf16")
    say(f"vocab4096 bf16 tile {tile}, sampled oracle")
    sampled_check(gpu_lib, inp, [sample], tile=tile)


@pytest.mark.timeout(400)
def test_vocab4096_closed_form_every_sample(gpu_lib):
    say("vocab4096 full bf16, W^O = 0: closed-form cost for every sample")
    closed_form_costs(gpu_lib, workload_inputs("vocab4096-bf16"), tile=(64, 32))


@pytest.mark.timeout(600)
def test_40s_b256_closed_form_and_sample(gpu_lib):
    inp = workload_inputs("40s-b256-bf16")
    say("40s-b256 full, W^O = 0: closed-form cost for every sample")
    closed_form_costs(gpu_lib, inp)
    say("40s-b256 full, sampled oracle")
    sampled_check(gpu_lib, inp, [11])


@pytest.mark.timeout(600)
def test_40s_b256_untiled_closed_form_and_sample(gpu_lib):
    """Untiled mode at the 40 s x 256 workload: the scores and z of all 31 M rows are kept
    (about 98 GB of `saved`, which one GPU's HBM holds), the backward forms dh from them."""
    import torch

    inp = workload_inputs("40s-b256-bf16")
    say("40s-b256 full untiled, W^O = 0: closed-form cost for every sample")
    closed_form_costs(gpu_lib, inp, mode="untiled")
    torch.cuda.empty_cache()
    say("40s-b256 full untiled, sampled oracle")
    sampled_check(gpu_lib, inp, [11], mode="untiled")
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode,fp8", [("tiled", False), ("untiled", False), ("tiled", True)])
def test_40s_b256_bitwise_repeats(gpu_lib, mode, fp8):
    """Two fwd+bwd passes over the 40 s x 256 workload give the same bits in every cost and gradient.
    Every reduction is ordered, so they must; and at this size every CU is busy, so a load or store
    whose result depended on timing would show here first (the lattice sweep's bitwise test makes the
    same check for the sweep alone)."""
    import torch

    inp = workload_inputs("40s-b256-bf16")
    say(f"40s-b256 {mode}{' fp8' if fp8 else ''}: two passes, bitwise")
    prob = gpu_lib.Problem(inp, mode=mode, fp8=fp8)
    dc = torch.tensor(np.random.default_rng(5).uniform(0.5, 1.5, len(inp.T_len)).astype(np.float32),
                      device=prob.device)
    runs = []
    for _ in range(2):
        c = prob.forward().clone()
        g = {k: v.clone() for k, v in prob.backward(dc).items()}
        torch.cuda.synchronize()
        runs.append((c, g))
    bits = lambda t: t.contiguous().view(torch.int32)
    assert torch.equal(bits(runs[0][0]), bits(runs[1][0])), "costs differ between the passes"
    for k in GRADS:
        a, b = bits(runs[0][1][k]), bits(runs[1][1][k])
        if not torch.equal(a, b):
            diff = (a != b).flatten()
            raise AssertionError(f"{k}: {int(diff.sum())} entries differ, first at flat index "
                                 f"{int(diff.nonzero()[0])}")
    assert bool(torch.isfinite(runs[0][0]).all())
    for k in GRADS:
        assert bool(torch.isfinite(runs[0][1][k]).all()), k
    del prob, runs
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- structure

@pytest.mark.timeout(400)
def test_device_memory_is_the_callers_buffers_and_tile_bounded(gpu_lib):
    """Tiled mode on a 40 s-like family (B=32, tile 64x32, 64 tiles per wave, T x U from 250 x 50 to
    1000 x 200): a fwd+bwd takes no device memory beyond the caller's buffers (free device memory is
    unchanged across the calls), and the workspace minus the O(B (T+U+1) H) gradient accumulators is the
    same for every lattice size, so the V- and H-proportional working set is set by the tile."""
    import torch

    rl = gpu_lib
    B, V, HA, HL, H = 32, 1024, 512, 512, 640
    rest = set()
    for T, U in ((250, 50), (500, 100), (1000, 200)):
        inp = make_inputs(B, T, U, V, HA, HL, H, dtype="bf16", seed=90 + T, t_range=(T // 2, T),
                          u_range=(U // 2, U))
        say(f"device memory B={B} T={T} U={U}")
        prob = rl.Problem(inp, mode="tiled", tile=(64, 32), tiles_per_wave=64)
        prob.forward()
        prob.backward()  # first calls: code objects and runtime state are set up here
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        costs = prob.forward().clone()
        prob.backward()
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        # the clone above is the only new allocation (served by torch's cache or one new block)
        assert free0 - free1 <= 2 * 1024 * 1024, (free0, free1)
        assert bool(torch.isfinite(costs).all())
        rest.add(prob.ws_bytes - 4 * H * B * (T + U + 1))
        del prob
        torch.cuda.empty_cache()
    assert max(rest) - min(rest) <= 4096, rest


@pytest.mark.parametrize("dtype,mode", [("bf16", "tiled"), ("bf16", "untiled"), ("f32", "tiled"),
                                        ("f32", "untiled")])
def test_padding_poison_is_ignored(gpu_lib, dtype, mode):
    """NaN in every padded row of h^A and h^L and out-of-range labels past U_b: the padded rows are
    read by the pre-projection products but must not reach any cost or gradient."""
    inp = make_inputs(3, 60, 20, 257, 64, 64, 64, dtype=dtype, seed=61, t_range=(10, 60), u_range=(0, 20))
    say(f"padding poison {dtype} {mode}")
    c0, g0 = run_gpu(gpu_lib, inp, mode=mode, tile=(32, 16))
    c1, g1 = run_gpu(gpu_lib, poison_padding(inp), mode=mode, tile=(32, 16))
    assert np.array_equal(c0, c1)
    for k in GRADS:
        assert np.array_equal(g0[k], g1[k]), k


@pytest.mark.parametrize("dtype,mode,H", [("bf16", "tiled", 640), ("bf16", "untiled", 640), ("bf16", "tiled", 128),
                                          ("bf16", "untiled", 128), ("f32", "tiled", 64), ("f32", "untiled", 64),
                                          ("fp8", "tiled", 640)])
def test_large_output_biases(gpu_lib, dtype, mode, H):
    """Output biases far beyond exp's fp32 range (+-100 nats): every cell's softmax is dominated by
    them, and rows that are no cell (a tile's t extent padded to 32 rows, the rows after a wave's
    last cell) must still contribute exactly nothing, so costs and gradients match the oracle."""
    import dataclasses

    import torch

    fp8 = dtype == "fp8"
    inp = make_inputs(3, 45, 12, 300, 64, 48, H, dtype="bf16" if fp8 else dtype, seed=67, t_range=(17, 45),
                      u_range=(0, 12), bias_std=0.1)
    bO = inp.bO.copy()
    bO[[3, 150, 299]] = [100.0, 95.0, -100.0]
    inp = dataclasses.replace(inp, bO=bO)
    say(f"large output biases {dtype} {mode} H={H}")
    prob = gpu_lib.Problem(inp, mode=mode, tile=(20, 7), tiles_per_wave=2, fp8=fp8)
    costs = prob.forward().clone().cpu().numpy().astype(np.float64)
    grads = {k: v.cpu().numpy().astype(np.float64) for k, v in prob.backward().items()}
    torch.cuda.synchronize()
    ref = oracle.loss_and_grads(inp, fp8_scores=fp8)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


@pytest.mark.parametrize("dtype,mode", [("f32", "tiled"), ("bf16", "tiled"), ("bf16", "untiled")])
def test_longest_label_sequence(gpu_lib, dtype, mode):
    """U + 1 = 1024, the library's limit (the lattice sweep on sixteen waves), and a long utterance
    (T = 3000) in one batch, against the oracle."""
    inp = make_inputs(3, 3000, 1023, 40, 32, 32, 64, dtype=dtype, seed=79, t_range=(2, 12), u_range=(900, 1023),
                      bias_std=0.3)
    inp.U_len[1] = 1023
    inp.T_len[2], inp.U_len[2] = 3000, 7
    say(f"U + 1 = 1024 and T = 3000, {dtype} {mode}: T_len={list(inp.T_len)} U_len={list(inp.U_len)}")
    costs, grads = run_gpu(gpu_lib, inp, mode=mode, tile=(64, 32))
    ref = oracle.loss_and_grads(inp)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


@pytest.mark.parametrize("dtype,mode,H", [("f32", "tiled", 32), ("bf16", "tiled", 32), ("bf16", "tiled", 640),
                                          ("bf16", "untiled", 640)])
def test_smallest_vocabulary(gpu_lib, dtype, mode, H):
    """V = 2 (the blank and one label), the library's smallest vocabulary: one 256-score V tile
    holding 254 scores past V."""
    inp = make_inputs(3, 20, 5, 2, 16, 24, H, dtype=dtype, seed=83, t_range=(1, 20), u_range=(0, 5), bias_std=0.5)
    say(f"V = 2 {dtype} {mode} H={H}")
    costs, grads = run_gpu(gpu_lib, inp, mode=mode, tile=(16, 4))
    ref = oracle.loss_and_grads(inp)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


@pytest.mark.parametrize("dtype,mode,tpw", [("f32", "tiled", 0), ("bf16", "tiled", 0), ("bf16", "tiled", 100),
                                            ("bf16", "untiled", 0)])
def test_large_batch_of_short_lattices(gpu_lib, dtype, mode, tpw):
    """B = 1024 lattices of at most 10 x 5 cells: a wave of a thousand one-tile samples (or waves of
    100), a thousand reduction groups of each kind, the lattice sweep on 2048 workgroups."""
    inp = make_inputs(1024, 10, 4, 60, 16, 16, 64 if dtype == "f32" else 512, dtype=dtype, seed=85, t_range=(1, 10),
                      u_range=(0, 4), bias_std=0.3)
    say(f"B = 1024 short lattices {dtype} {mode} tpw={tpw}")
    costs, grads = run_gpu(gpu_lib, inp, mode=mode, tile=(16, 8), tpw=tpw)
    ref = oracle.loss_and_grads(inp)
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


def test_deterministic_repeats(gpu_lib):
    inp = workload_inputs("small-bf16")
    say("determinism small")
    a = run_gpu(gpu_lib, inp)
    b = run_gpu(gpu_lib, inp)
    assert np.array_equal(a[0], b[0])
    for k in GRADS:
        assert np.array_equal(a[1][k], b[1][k]), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(gpu_lib, dtype):
    """U_b = 0, T_b = 1, a transcript label equal to the blank id, blank != 0,
    one tile per wave, V not a multiple of 64."""
    inp = make_inputs(5, 9, 4, 70, 16, 24, 32, dtype=dtype, seed=71, bias_std=0.5)
    inp.T_len[:] = [1, 9, 3, 9, 1]
    inp.U_len[:] = [0, 0, 4, 2, 3]
    inp.blank = 69
    inp.labels[:, 0] = 69
    for b in range(5):
        inp.labels[b, inp.U_len[b] + 1:] = 69
    inp.labels[2, 2] = 69  # a label that is the blank id
    say(f"edge cases {dtype}")
    full_check(gpu_lib, inp, tile=(32, 2), tpw=1)
    full_check(gpu_lib, inp, mode="untiled")


@pytest.mark.parametrize("dtype,mode", [("f32", "tiled"), ("bf16", "tiled"), ("bf16", "untiled"), ("fp8", "tiled")])
def test_largest_vocabulary(gpu_lib, dtype, mode):
    """V = 65536, the library's limit (256 V tiles of 256 scores), on a small ragged lattice with
    labels near the top of the vocabulary and the blank id at V - 1."""
    import torch

    inp = make_inputs(2, 20, 5, 65536, 64, 40, 64, dtype="f32" if dtype == "f32" else "bf16", seed=73,
                      t_range=(9, 20), u_range=(2, 5), bias_std=0.3, blank=65535)
    inp.labels[0, 1] = 65534
    inp.labels[1, 2] = 1
    say(f"V = 65536 {dtype} {mode}")
    prob = gpu_lib.Problem(inp, mode=mode, tile=(16, 4), tiles_per_wave=3, fp8=dtype == "fp8")
    costs = prob.forward().clone().cpu().numpy().astype(np.float64)
    grads = {k: v.cpu().numpy().astype(np.float64) for k, v in prob.backward().items()}
    torch.cuda.synchronize()
    ref = oracle.loss_and_grads(inp, fp8_scores=dtype == "fp8")
    check_costs(inp, costs, ref.costs)
    check_grads(inp, grads, ref.grads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_out_of_range_labels_are_counted_and_contained(gpu_lib, dtype):
    """Labels outside [0, V) in the transcript: the forward's checked copy replaces them with the
    blank id (so no kernel indexes the output layer with them), and the first two int32 of saved
    report how many there were and the flat index of the first. Results equal those of the same
    batch with the blank id written in their place."""
    import dataclasses

    import torch

    rl = gpu_lib
    inp = make_inputs(3, 40, 10, 300, 64, 48, 64, dtype=dtype, seed=67, t_range=(10, 40), u_range=(4, 10),
                      bias_std=0.2)
    U1, V = inp.labels.shape[1], inp.WO.shape[0]
    bad = inp.labels.copy()
    bad[1, 3] = V + 5
    bad[2, 1] = -3
    bad[0, inp.U_len[0] + 1:] = V + 1000  # past U_b: never read, not counted
    fixed = bad.copy()
    fixed[1, 3] = fixed[2, 1] = inp.blank
    fixed[0, inp.U_len[0] + 1:] = inp.blank
    say(f"out-of-range labels {dtype}")
    prob = rl.Problem(dataclasses.replace(inp, labels=bad), tile=(32, 8))
    c_bad = prob.forward().clone()
    g_bad = {k: v.clone() for k, v in prob.backward().items()}
    torch.cuda.synchronize()
    status = prob.saved[:8].view(torch.int32).cpu().tolist()
    assert status == [2, 1 * U1 + 3], status
    c_fix, g_fix = run_gpu(rl, dataclasses.replace(inp, labels=fixed), tile=(32, 8))
    assert np.array_equal(c_bad.cpu().numpy().astype(np.float64), c_fix)
    for k in GRADS:
        assert np.array_equal(g_bad[k].cpu().numpy().astype(np.float64), g_fix[k]), k
    # in-range labels leave the status words at (0, -1)
    prob = rl.Problem(inp, tile=(32, 8))
    prob.forward()
    torch.cuda.synchronize()
    assert prob.saved[:8].view(torch.int32).cpu().tolist() == [0, -1]
