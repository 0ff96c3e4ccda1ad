"""Pins for the fp64 oracle: results fixed by the mathematics, not by the oracle.

Each check is independent of the oracle's own formulas:
  * brute force: summing every monotone alignment path (tiny lattices);
  * alpha/beta identity: both recursions give the same total probability;
  * closed forms with W^O = 0 (every alignment then has the same probability,
    so the cost is a binomial count and the occupancy a ratio of binomials);
  * torch's fp64 log_softmax for the softmax-denominator step;
  * flow invariants (each frame is left by exactly one blank, each label is
    emitted exactly once) and dh row sums = 0;
  * central finite differences of the loss for every input and parameter;
  * an independent torch fp64 autograd implementation written cell by cell.
The mutation tests at the end plant plausible mistakes into the oracle and
check that these pins catch every one of them.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import rnnt_oracle as ro
from rnnt_inputs import diagonal_band, make_inputs, poison_padding, workload_inputs


def tiny(B=2, T=5, U=3, V=6, H=4, HA=3, HL=5, seed=0, t_range=None, u_range=None, bias_std=0.3,
         enc="normal0.5", weights="normal0.5"):
    return make_inputs(B, T, U, V, HA, HL, H, dtype="f32", seed=seed, enc=enc, weights=weights,
                       t_range=t_range, u_range=u_range, bias_std=bias_std)


def lnC(n, k):
    return math.lgamma(n + 1) - math.lgamma(k + 1) - math.lgamma(n - k + 1)


# ----------------------------------------------------------------------------- brute force

LATTICES = [(6, 3), (1, 0), (1, 4), (5, 0), (3, 3), (4, 5), (7, 2)]


@pytest.mark.parametrize("Tb,Ub", LATTICES)
def test_dp_equals_brute_force(Tb, Ub):
    inp = tiny(B=1, T=Tb, U=Ub, seed=Tb * 10 + Ub)
    r = oracle.loss_and_grads(inp, want_grads=False)
    s = r.samples[0]
    bf = oracle.brute_force_cost(s.phi, s.psi)
    assert abs(bf - r.costs[0]) <= 1e-12 * abs(bf)


def test_tiny_brute_force():
    inp = workload_inputs("tiny-f32")
    r = oracle.loss_and_grads(inp, want_grads=False)
    for b, s in enumerate(r.samples):
        assert abs(oracle.brute_force_cost(s.phi, s.psi) - r.costs[b]) <= 1e-12 * abs(r.costs[b])


def test_label_equal_to_blank_inside_transcript():
    inp = tiny(B=1, T=4, U=3, seed=3)
    inp.labels[0, 2] = inp.blank  # a transcript label that is the blank id
    r = oracle.loss_and_grads(inp)
    s = r.samples[0]
    assert abs(oracle.brute_force_cost(s.phi, s.psi) - r.costs[0]) <= 1e-12 * abs(r.costs[0])
    fd_check(inp, names=("WO", "bO"))


def test_alpha_beta_identity_ragged():
    inp = tiny(B=4, T=9, U=5, seed=7, t_range=(1, 9), u_range=(0, 5))
    r = oracle.loss_and_grads(inp, want_grads=False)
    for s in r.samples:
        assert abs(s.beta[0, 0] - s.lnP) <= 1e-12 * max(1.0, abs(s.lnP))


def test_alpha_beta_identity_small_sample():
    inp = workload_inputs("small-bf16", B=1)
    inp = make_inputs(1, 40, 12, 64, 32, 32, 48, dtype="bf16", seed=2, t_range=(25, 40), u_range=(6, 12))
    r = oracle.loss_and_grads(inp, want_grads=False)
    s = r.samples[0]
    assert abs(s.beta[0, 0] - s.lnP) <= 1e-12 * abs(s.lnP)


# ----------------------------------------------------------------------------- closed forms

def zero_output_weights(inp, bias=None):
    inp.WO[:] = 0.0
    inp.bO[:] = 0.0 if bias is None else bias
    return inp


def test_closed_form_uniform_tiny_lattice():
    """W^O = 0, b^O = 0: every p = 1/V, cost = (T_b+U_b) ln V - ln C(T_b+U_b-1, U_b)."""
    inp = zero_output_weights(workload_inputs("tiny-f32"))
    r = oracle.loss_and_grads(inp, want_grads=False)
    for b in range(2):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        want = (Tb + Ub) * math.log(5) - lnC(Tb + Ub - 1, Ub)
        assert abs(r.costs[b] - want) <= 1e-13 * want
    # the worked value for a 6 x 4 lattice with V = 5
    assert abs(r.costs[0] - 10.459589521171752) < 1e-12


@pytest.mark.parametrize("Tb,Ub,V", [(6, 3, 5), (250, 64, 1024), (1000, 200, 1024), (400, 150, 4096), (1, 0, 7)])
def test_closed_form_bias_only(Tb, Ub, V):
    """W^O = 0: cost = -[T_b ln p_blank + sum_u ln p_{y_u} + ln C(T_b+U_b-1, U_b)], p = softmax(b^O)."""
    inp = make_inputs(1, Tb, Ub, V, 4, 4, 4, dtype="f32", seed=V + Tb)
    rng = np.random.default_rng(Tb)
    bO = rng.normal(0, 1.5, V).astype(np.float32)
    inp = zero_output_weights(inp, bO)
    r = oracle.loss_and_grads(inp, want_grads=False)
    b64 = bO.astype(np.float64)
    logp = b64 - (b64.max() + np.log(np.exp(b64 - b64.max()).sum()))
    y = inp.labels[0, 1:Ub + 1]
    want = -(Tb * logp[0] + logp[y].sum() + lnC(Tb + Ub - 1, Ub))
    assert abs(r.costs[0] - want) <= 1e-12 * abs(want)


@pytest.mark.parametrize("bias", [False, True])
def test_occupancy_closed_form(bias):
    """W^O = 0: all alignments equally likely, occ(t,u) = C(t+u,u) C(T-1-t+U-u, U-u) / C(T-1+U, U)."""
    Tb, Ub = 7, 4
    inp = tiny(B=1, T=Tb, U=Ub, V=6, seed=11)
    inp = zero_output_weights(inp, np.linspace(-1, 1, 6).astype(np.float32) if bias else None)
    r = oracle.loss_and_grads(inp, keep_flows=True)
    s = r.samples[0]
    for t in range(Tb):
        for u in range(Ub + 1):
            want = math.exp(lnC(t + u, u) + lnC(Tb - 1 - t + Ub - u, Ub - u) - lnC(Tb - 1 + Ub, Ub))
            assert abs(s.occ[t, u] - want) <= 1e-12


# ----------------------------------------------------------------------------- library cross-check

def test_log_softmax_matches_torch():
    rng = np.random.default_rng(5)
    h = rng.normal(0, 3, size=(7, 5, 33))
    y = np.array([0, 3, 9, 32, 1])
    lse = oracle.log_softmax_denominator(h)
    phi, psi = oracle.two_log_probs(h, lse, y, 4, 0)
    ref = torch.log_softmax(torch.from_numpy(h), dim=-1).numpy()
    assert np.max(np.abs(phi - ref[..., 0])) <= 1e-14 * 10
    for u in range(4):
        assert np.max(np.abs(psi[:, u] - ref[:, u, y[u + 1]])) <= 1e-13
    assert np.all(np.isneginf(psi[:, 4]))


# ----------------------------------------------------------------------------- invariants

def test_flow_invariants_and_row_sums():
    inp = tiny(B=3, T=8, U=5, V=7, seed=21, t_range=(2, 8), u_range=(0, 5))
    r = oracle.loss_and_grads(inp, keep_flows=True)
    for b, s in enumerate(r.samples):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        assert np.allclose(s.bflow.sum(axis=1), 1.0, atol=1e-12, rtol=0)  # one blank leaves each frame
        if Ub:
            assert np.allclose(s.lflow[:, :Ub].sum(axis=0), 1.0, atol=1e-12, rtol=0)  # each label once
        assert abs(s.bflow[Tb - 1, Ub] - 1.0) < 1e-12  # final blank
        assert abs(s.occ.sum() - (Tb + Ub)) < 1e-10
        assert np.allclose(s.occ, s.bflow + s.lflow, atol=1e-12, rtol=0)
        h = rng_logits(Tb, Ub, 7, seed=b)
        dh = oracle.dlogits(h, inp.labels[b], Ub, 0, g=1.7)
        assert np.max(np.abs(dh.sum(axis=-1))) <= 1e-12


def rng_logits(Tb, Ub, V, seed):
    return np.random.default_rng(seed).normal(0, 2, size=(Tb, Ub + 1, V))


# ----------------------------------------------------------------------------- finite differences

@pytest.mark.parametrize("Tb,Ub", [(4, 3), (1, 2), (3, 0)])
def test_fd_logits(Tb, Ub):
    V = 5
    h = rng_logits(Tb, Ub, V, seed=Tb + 7 * Ub)
    y = np.array([0, 2, 4, 1])[: Ub + 1]
    dh = oracle.dlogits(h, y, Ub, 0)
    eps = 1e-6
    fd = np.zeros_like(h)
    for idx in np.ndindex(*h.shape):
        hp = h.copy(); hp[idx] += eps
        hm = h.copy(); hm[idx] -= eps
        fd[idx] = (oracle.lattice_from_logits(hp, y, Ub, 0)[0] - oracle.lattice_from_logits(hm, y, Ub, 0)[0]) / (2 * eps)
    assert np.max(np.abs(fd - dh)) <= 1e-7 * max(1.0, np.max(np.abs(dh)))


def total_loss(inp, g, band=None):
    r = oracle.loss_and_grads(inp, want_grads=False, band=band)
    return float(np.dot(g, r.costs))


def fd_check(inp, names=("hA", "hL", "WA", "WL", "bZ", "WO", "bO"), g=None, eps=1e-6, tol=1e-7, band=None):
    """Central differences of sum_b g_b cost_b for every element of the named arrays."""
    B = len(inp.T_len)
    g = np.linspace(0.5, 1.5, B) if g is None else g
    r = oracle.loss_and_grads(inp, dcosts=g, band=band)
    key = dict(hA="dhA", hL="dhL", WA="dWA", WL="dWL", bZ="dbZ", WO="dWO", bO="dbO")
    for name in names:
        arr = getattr(inp, name)
        # perturb in float64 so eps is not lost to float32 rounding
        base = arr.astype(np.float64)
        setattr(inp, name, base)
        grad = r.grads[key[name]]
        fd = np.zeros_like(base)
        for idx in np.ndindex(*base.shape):
            if name == "hA" and idx[1] >= inp.T_len[idx[0]]:
                continue
            if name == "hL" and idx[1] > inp.U_len[idx[0]]:
                continue
            old = base[idx]
            base[idx] = old + eps
            lp = total_loss(inp, g, band)
            base[idx] = old - eps
            lm = total_loss(inp, g, band)
            base[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        setattr(inp, name, arr)
        err = np.max(np.abs(fd - grad))
        assert err <= tol * max(1.0, np.max(np.abs(grad))), (name, err)


def test_fd_every_parameter_tiny():
    fd_check(workload_inputs("tiny-f32"))


def test_fd_ragged_batch_with_biases():
    fd_check(tiny(B=3, T=5, U=3, seed=13, t_range=(1, 5), u_range=(0, 3)))


# ----------------------------------------------------------------------------- pruned lattice

def brute_force_band_cost(phi, psi, lo, S):
    """-log of the summed probability of the alignments whose every cell lies in the band
    lo[t] <= u < lo[t] + S, by enumeration with an explicit membership test on each visited
    cell (the unpruned log-probs phi, psi; independent of the oracle's masking)."""
    import itertools

    Tb, U1 = phi.shape
    Ub = U1 - 1
    n = Tb - 1 + Ub
    inb = lambda t, u: lo[t] <= u < lo[t] + S
    logps = []
    for label_steps in itertools.combinations(range(n), Ub):
        ls = set(label_steps)
        t = u = 0
        lp, ok = 0.0, True
        for step in range(n):
            ok = ok and inb(t, u)
            if step in ls:
                lp += psi[t, u]
                u += 1
            else:
                lp += phi[t, u]
                t += 1
        ok = ok and inb(Tb - 1, Ub)
        if ok:
            logps.append(lp + phi[Tb - 1, Ub])
    logps = np.array(logps)
    m = logps.max()
    return -(m + np.log(np.sum(np.exp(logps - m)))), len(logps)


@pytest.mark.parametrize("Tb,Ub,S", [(6, 3, 2), (7, 5, 3), (5, 4, 2), (8, 0, 1), (4, 6, 4)])
def test_pruned_cost_equals_band_brute_force(Tb, Ub, S):
    inp = tiny(B=1, T=Tb, U=Ub, seed=100 + Tb * 10 + Ub)
    lo = diagonal_band(inp.T_len, inp.U_len, Tb, S)
    full = oracle.loss_and_grads(inp, want_grads=False)
    pruned = oracle.loss_and_grads(inp, want_grads=False, band=(lo, S))
    bf, n_paths = brute_force_band_cost(full.samples[0].phi, full.samples[0].psi, lo[0], S)
    assert n_paths >= 1
    assert abs(bf - pruned.costs[0]) <= 1e-12 * abs(bf)
    # pruning removes alignments: the cost can only grow
    assert pruned.costs[0] >= full.costs[0] - 1e-12


def test_pruned_wide_band_is_the_full_loss():
    inp = tiny(B=3, T=7, U=4, seed=41, t_range=(2, 7), u_range=(0, 4))
    S = 5  # every row of every frame
    lo = np.zeros((3, 7), dtype=np.int32)
    a = oracle.loss_and_grads(inp)
    b = oracle.loss_and_grads(inp, band=(lo, S))
    assert np.array_equal(a.costs, b.costs)
    for k, v in a.grads.items():
        assert np.array_equal(v, b.grads[k]), k


def test_pruned_fd_every_parameter():
    """Central differences of the pruned loss for every input and parameter (ragged batch)."""
    inp = tiny(B=2, T=6, U=4, seed=43, t_range=(4, 6), u_range=(2, 4))
    lo = diagonal_band(inp.T_len, inp.U_len, 6, 2)
    fd_check(inp, band=(lo, 2))


def test_pruned_cells_get_no_gradient():
    inp = tiny(B=1, T=6, U=4, seed=47)
    S = 2
    lo = diagonal_band(inp.T_len, inp.U_len, 6, S)
    r = oracle.loss_and_grads(inp, band=(lo, S), keep_flows=True)
    s = r.samples[0]
    out = ~ro.band_mask(lo[0], S, 6, 5)
    assert np.all(s.occ[out] == 0) and np.all(s.bflow[out] == 0) and np.all(s.lflow[out] == 0)
    assert abs(s.occ.sum() - (6 + 4)) < 1e-10  # every alignment still visits T_b + U_b cells


# ----------------------------------------------------------------------------- independent autograd

def torch_loss(inp, g):
    """Cell-by-cell RNN-T loss in torch fp64; gradients by autograd. Independent of the oracle."""
    P = {k: torch.tensor(np.asarray(getattr(inp, k), dtype=np.float64), requires_grad=True)
         for k in ("hA", "hL", "WA", "WL", "bZ", "WO", "bO")}
    total = torch.zeros((), dtype=torch.float64)
    for b in range(len(inp.T_len)):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        y = [int(v) for v in inp.labels[b]]
        logp = {}
        for t in range(Tb):
            for u in range(Ub + 1):
                pre = P["WA"] @ P["hA"][b, t] + P["WL"] @ P["hL"][b, u] + P["bZ"]
                logits = P["WO"] @ torch.tanh(pre) + P["bO"]
                logp[t, u] = torch.log_softmax(logits, dim=0)
        alpha = {}
        for t in range(Tb):
            for u in range(Ub + 1):
                if t == 0 and u == 0:
                    alpha[t, u] = torch.zeros((), dtype=torch.float64)
                    continue
                terms = []
                if t > 0:
                    terms.append(alpha[t - 1, u] + logp[t - 1, u][inp.blank])
                if u > 0:
                    terms.append(alpha[t, u - 1] + logp[t, u - 1][y[u]])
                alpha[t, u] = torch.logsumexp(torch.stack(terms), dim=0)
        lnP = alpha[Tb - 1, Ub] + logp[Tb - 1, Ub][inp.blank]
        total = total - float(g[b]) * lnP
    total.backward()
    grads = {"d" + k: P[k].grad.numpy() for k in P}
    return float(total), grads


def autograd_check(inp, g=None, tol=1e-12, **oracle_kw):
    B = len(inp.T_len)
    g = np.linspace(1.3, 0.7, B) if g is None else g
    r = oracle.loss_and_grads(inp, dcosts=g, **oracle_kw)
    L, tg = torch_loss(inp, g)
    assert abs(L - float(np.dot(g, r.costs))) <= tol * abs(L)
    for k in ("dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO"):
        ref = tg[k]
        err = np.max(np.abs(r.grads[k] - ref))
        assert err <= tol * max(1.0, np.max(np.abs(ref))), (k, err)


def test_autograd_tiny():
    autograd_check(workload_inputs("tiny-f32"))


def test_autograd_reduced_small():
    # small-workload structure (bf16 values, Xavier weights, ragged lengths) at a size autograd can walk
    inp = make_inputs(2, 9, 5, 40, 12, 10, 16, dtype="bf16", seed=2, t_range=(5, 9), u_range=(2, 5),
                      bias_std=0.2)
    autograd_check(inp, tol=1e-11)


def test_autograd_one_row_per_block():
    """The oracle's blocking over t rows (which only bounds host memory) pinned to the independent
    autograd implementation: with a byte budget of 1 every block holds a single t row, so each
    sample's forward and backward run over T_b blocks, ragged lengths included."""
    inp = make_inputs(3, 8, 4, 30, 12, 10, 16, dtype="bf16", seed=29, t_range=(3, 8), u_range=(0, 4),
                      bias_std=0.2)
    autograd_check(inp, tol=1e-11, mem_budget=1)


def test_blocking_does_not_change_results():
    """One t row per block against the default single block, on a ragged batch at the small
    workload's widths: costs and every gradient agree to 1e-13 (only summation order differs)."""
    inp = make_inputs(3, 40, 12, 300, 64, 48, 80, dtype="bf16", seed=33, t_range=(10, 40),
                      u_range=(0, 12), bias_std=0.2)
    a = oracle.loss_and_grads(inp)
    b = oracle.loss_and_grads(inp, mem_budget=1)
    assert np.max(np.abs(a.costs - b.costs) / np.abs(a.costs)) <= 1e-13
    for k, v in a.grads.items():
        assert np.max(np.abs(v - b.grads[k])) <= 1e-13 * max(1.0, np.max(np.abs(v))), k


# ----------------------------------------------------------------------------- padding / batch structure

def test_padding_invariance():
    inp = tiny(B=3, T=7, U=4, seed=17, t_range=(2, 7), u_range=(0, 4))
    r0 = oracle.loss_and_grads(inp)
    r1 = oracle.loss_and_grads(poison_padding(inp))
    assert np.array_equal(r0.costs, r1.costs)
    for k, v in r0.grads.items():
        assert np.array_equal(v, r1.grads[k]), k
    for b in range(3):
        assert np.all(r1.grads["dhA"][b, inp.T_len[b]:] == 0)
        assert np.all(r1.grads["dhL"][b, inp.U_len[b] + 1:] == 0)


def test_gradients_linear_in_dcosts():
    """Gradient with one-hot dcosts = that sample's own gradient; they sum to the full one."""
    inp = tiny(B=3, T=6, U=3, seed=19, t_range=(3, 6), u_range=(1, 3))
    full = oracle.loss_and_grads(inp, dcosts=np.array([0.5, 2.0, -1.0]))
    acc = {k: np.zeros_like(v) for k, v in full.grads.items()}
    for b, gb in enumerate([0.5, 2.0, -1.0]):
        e = np.zeros(3); e[b] = gb
        part = oracle.loss_and_grads(inp, dcosts=e, samples=[b])
        for k in acc:
            acc[k] += part.grads[k]
    for k in acc:
        assert np.allclose(acc[k], full.grads[k], atol=1e-13, rtol=1e-12), k


# ----------------------------------------------------------------------------- planted mistakes

def pin_suite():
    """Run the fast pins; return the names of those that fail."""
    failed = []
    checks = {
        "brute": lambda: test_tiny_brute_force(),
        "identity": lambda: test_alpha_beta_identity_ragged(),
        "closed_uniform": lambda: test_closed_form_uniform_tiny_lattice(),
        "closed_bias": lambda: test_closed_form_bias_only(6, 3, 5),
        "flows": lambda: test_flow_invariants_and_row_sums(),
        "autograd": lambda: (autograd_check(workload_inputs("tiny-f32")), autograd_check(_square_biased())),
    }
    for name, fn in checks.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def _square_biased():
    # tiny-workload dimensions (H = H_A = H_L) with non-zero biases and ragged lengths
    return make_inputs(3, 6, 3, 5, 8, 8, 8, dtype="f32", seed=23, enc="normal0.5", weights="normal0.5",
                       t_range=(2, 6), u_range=(0, 3), bias_std=0.4)


def test_pin_suite_passes_on_oracle():
    assert pin_suite() == []


def _two_log_probs_wrong_label(h, lse, y_b, U_b, blank):
    phi, psi = _orig["two_log_probs"](h, lse, np.concatenate([[y_b[0]], y_b[:-1]]), U_b, blank)
    return phi, psi


def _beta_missing_terminal(phi, psi):
    b = _orig["beta_recursion"](phi, psi - 0.0)
    return b - phi[-1, -1]


def _logits_grad_label_sign(h, lse, occ, bflow, lflow, y_b, U_b, blank, g):
    return _orig["logits_grad"](h, lse, occ, bflow, -lflow, y_b, U_b, blank, g)


def _alpha_no_label_moves(phi, psi):
    return _orig["alpha_recursion"](phi, np.full_like(psi, -np.inf))


def _joint_no_bias(hA_b, hL_b, WA, WL, bZ):
    return _orig["joint"](hA_b, hL_b, WA, WL, 0 * np.asarray(bZ))


def _output_transposed_bias(z, WO, bO):
    return _orig["output_layer"](z, WO, np.asarray(bO)[::-1])


_orig = {k: getattr(ro, k) for k in ("two_log_probs", "beta_recursion", "logits_grad",
                                      "alpha_recursion", "joint", "output_layer")}

MUTANTS = {
    "psi reads y[u] instead of y[u+1]": ("two_log_probs", _two_log_probs_wrong_label),
    "beta drops the final blank": ("beta_recursion", _beta_missing_terminal),
    "dh label correction has the wrong sign": ("logits_grad", _logits_grad_label_sign),
    "alpha forgets label moves": ("alpha_recursion", _alpha_no_label_moves),
    "joint drops b^Z": ("joint", _joint_no_bias),
    "b^O indexed backwards": ("output_layer", _output_transposed_bias),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ro, attr, fn)
    assert pin_suite(), f"no pin caught: {name}"


def test_pins_catch_band_off_by_one(monkeypatch):
    orig = ro.band_mask
    monkeypatch.setattr(ro, "band_mask", lambda lo, S, Tb, U1: orig(lo, S - 1, Tb, U1) | orig(lo, 1, Tb, U1))
    with pytest.raises(AssertionError):
        test_pruned_cost_equals_band_brute_force(6, 3, 2)


def test_pins_catch_wrong_dtanh(monkeypatch):
    monkeypatch.setattr(ro, "tanh_grad", lambda z: 1.0 - z)
    assert "autograd" in pin_suite()


def test_pins_catch_transposed_encoder_weight(monkeypatch):
    # the tiny workload has H = H_A = H_L = 8, so a transposed W^A is shape-valid
    monkeypatch.setattr(ro, "encoding_grad", lambda g, W: g @ W.T)
    assert "autograd" in pin_suite()


# ----------------------------------------------------------------------------- fp8 (E4M3) output layer

def e4m3_decode(code):
    """Value of an OCP FP8 E4M3 byte from the format's definition: sign, 4 exponent bits (bias 7),
    3 fraction bits; exponent field 0 holds the subnormals m/8 2^-6; S.1111.111 is NaN (None)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def e4m3_table():
    """{value: code} over every finite code, non-negative values only."""
    return {e4m3_decode(c): c for c in range(128) if e4m3_decode(c) is not None}


def test_e4m3_table_fixed_points_and_ties():
    tab = e4m3_table()
    vals = np.array(sorted(tab))
    assert len(vals) == 127 and vals[-1] == 448.0 and vals[1] == 2.0 ** -9
    # every finite value (both signs) rounds to itself
    assert np.array_equal(ro.e4m3_round(vals), vals)
    assert np.array_equal(ro.e4m3_round(-vals), -vals)
    # the midpoint of two neighbours goes to the one with an even code; just off it, to the nearer
    mid = (vals[:-1] + vals[1:]) / 2
    even = np.array([lo if tab[lo] % 2 == 0 else hi for lo, hi in zip(vals[:-1], vals[1:])])
    assert np.array_equal(ro.e4m3_round(mid), even)
    gap = vals[1:] - vals[:-1]
    assert np.array_equal(ro.e4m3_round(mid - gap / 64), vals[:-1])
    assert np.array_equal(ro.e4m3_round(mid + gap / 64), vals[1:])


def test_e4m3_round_matches_torch_float8():
    """Against torch's float8_e4m3fn conversion (a library routine) on float32 values: random
    magnitudes over the whole range and every midpoint of neighbouring values."""
    rng = np.random.default_rng(5)
    x = (rng.choice([-1.0, 1.0], 20000) * 2.0 ** rng.uniform(-12, np.log2(448), 20000)).astype(np.float32)
    vals = np.array(sorted(e4m3_table()))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([0.0, 448.0, -448.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ro.e4m3_round(x.astype(np.float64)), ref)


@pytest.mark.parametrize("amax", [448.0, 224.0, 447.0, 449.0, 0.875, 0.87, 0.88, 0.0604, 1.0, 3e-3, 7.0])
def test_wo_scale_exponent(amax):
    W = np.array([[0.5 * amax, -amax], [0.0, 0.25 * amax]])
    e = ro.wo_scale_exp(W)
    assert amax * 2.0 ** e <= 448.0 < amax * 2.0 ** (e + 1)


def torch_fp8_loss(inp, g):
    """Cell-by-cell loss in torch fp64 whose scores are the product of E4M3-rounded operands (z by
    2^8, W^O by 2^e), rounded by torch's float8_e4m3fn conversion, while autograd differentiates the
    unrounded product (the value of the rounded one is added as a constant). Independent of the
    oracle; the scale exponent from log2."""
    P = {k: torch.tensor(np.asarray(getattr(inp, k), dtype=np.float64), requires_grad=True)
         for k in ("hA", "hL", "WA", "WL", "bZ", "WO", "bO")}
    amax = float(np.max(np.abs(np.asarray(inp.WO, dtype=np.float64))))
    ew = math.floor(math.log2(448.0 / amax))
    q = lambda x, e: x.detach().mul(2.0 ** e).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
    wq = q(P["WO"], ew)
    total = torch.zeros((), dtype=torch.float64)
    for b in range(len(inp.T_len)):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        y = [int(v) for v in inp.labels[b]]
        logp = {}
        for t in range(Tb):
            for u in range(Ub + 1):
                z = torch.tanh(P["WA"] @ P["hA"][b, t] + P["WL"] @ P["hL"][b, u] + P["bZ"])
                exact = P["WO"] @ z
                rounded = (wq @ q(z, 8)) * 2.0 ** -(8 + ew)
                logits = exact + (rounded - exact).detach() + P["bO"]
                logp[t, u] = torch.log_softmax(logits, dim=0)
        alpha = {}
        for t in range(Tb):
            for u in range(Ub + 1):
                if t == 0 and u == 0:
                    alpha[t, u] = torch.zeros((), dtype=torch.float64)
                    continue
                terms = []
                if t > 0:
                    terms.append(alpha[t - 1, u] + logp[t - 1, u][inp.blank])
                if u > 0:
                    terms.append(alpha[t, u - 1] + logp[t, u - 1][y[u]])
                alpha[t, u] = torch.logsumexp(torch.stack(terms), dim=0)
        total = total - float(g[b]) * (alpha[Tb - 1, Ub] + logp[Tb - 1, Ub][inp.blank])
    total.backward()
    return float(total), {"d" + k: P[k].grad.numpy() for k in P}


@pytest.mark.parametrize("which", ["tiny", "reduced"])
def test_fp8_scores_against_independent_autograd(which):
    if which == "tiny":
        inp = workload_inputs("tiny-f32")
    else:
        inp = make_inputs(2, 9, 5, 40, 12, 10, 16, dtype="bf16", seed=2, t_range=(5, 9), u_range=(2, 5),
                          bias_std=0.2)
    g = np.linspace(1.3, 0.7, len(inp.T_len))
    r = oracle.loss_and_grads(inp, dcosts=g, fp8_scores=True)
    L, tg = torch_fp8_loss(inp, g)
    assert abs(L - float(np.dot(g, r.costs))) <= 1e-12 * abs(L)
    for k in ("dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO"):
        err = np.max(np.abs(r.grads[k] - tg[k]))
        assert err <= 1e-11 * max(1.0, np.max(np.abs(tg[k]))), (k, err)
    # the rounding is not a no-op: the plain loss differs
    plain = oracle.loss_and_grads(inp, dcosts=g, want_grads=False)
    assert np.max(np.abs(plain.costs - r.costs)) > 1e-6


def test_fp8_scores_zero_projection_is_the_closed_form():
    """W^O = 0 rounds to 0, so the fp8 loss is the bias-only closed form at any lattice size."""
    inp = make_inputs(2, 30, 7, 9, 8, 8, 8, dtype="f32", seed=3, t_range=(20, 30), u_range=(3, 7),
                      bias_std=0.4)
    inp = dataclasses.replace(inp, WO=np.zeros_like(inp.WO))
    a = oracle.loss_and_grads(inp, want_grads=False, fp8_scores=True)
    b = oracle.loss_and_grads(inp, want_grads=False)
    assert np.allclose(a.costs, b.costs, rtol=1e-14, atol=0)


def test_fp8_pins_catch_ties_away_from_zero(monkeypatch):
    def away(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        _, e = np.frexp(a)
        k = np.maximum(e - 1, -6)
        return np.copysign(np.ldexp(np.floor(np.ldexp(a, 3 - k) + 0.5), k - 3), x)

    monkeypatch.setattr(ro, "e4m3_round", away)
    with pytest.raises(AssertionError):
        test_e4m3_table_fixed_points_and_ties()


def test_fp8_pins_catch_unscaled_projection_weights(monkeypatch):
    # without its scale W^O (|w| < 0.5 here) falls partly into the subnormals
    monkeypatch.setattr(ro, "wo_scale_exp", lambda WO: 0)
    with pytest.raises(AssertionError):
        test_fp8_scores_against_independent_autograd("reduced")
