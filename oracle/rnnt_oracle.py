"""fp64 CPU oracle for the RNN-T joint network, output layer and loss.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP library; its only shared dependency is
the seeded input generator in `rnnt_inputs`, which holds no transducer
arithmetic.

What it computes, per sample b (the sample-wise loop of "Neural transducer
training: reduced memory consumption with sample-wise computation", section
"Sample-wise method", Algorithm 1, whose per-sample result is identical to the
batched one), in float64 from the same dtype-rounded input values the GPU sees:

  joint network f^J   (section "Transducer training", Eqs. (3)-(4))
      z[t,u] = tanh(W^A h^A[t] + W^L h^L[u] + b^Z)
      The extracted text lost Eq. (4); tanh and the single bias b^Z are the
      reading used throughout this project.
  output layer f^O    (Eqs. (5)-(6))
      h[t,u] = W^O z[t,u] + b^O
  softmax denominator f^W_1 (Eq. (7)), kept in the log domain
      lse[t,u] = log sum_v exp(h[t,u,v])
  the two log-probs the loss needs ("Flash RNN-T: making room to train speech
  recognition", section "Compute it, use it, make room")
      phi[t,u] = h[t,u,blank] - lse[t,u]
      psi[t,u] = h[t,u,y[u+1]] - lse[t,u]      (u < U_b; y has blank in col 0)
  forward/backward variables f^W_2 (Eq. (8)), log domain
      alpha(0,0) = 0
      alpha(t,u) = logaddexp(alpha(t-1,u) + phi(t-1,u), alpha(t,u-1) + psi(t,u-1))
      beta(T_b-1,U_b) = phi(T_b-1,U_b)
      beta(t,u)  = logaddexp(phi(t,u) + beta(t+1,u), psi(t,u) + beta(t,u+1))
      (terms outside the lattice are -inf; a path ends with a blank at
      (T_b-1, U_b))
  loss f^W_3 (Eq. (9))
      cost_b = -(alpha(T_b-1,U_b) + phi(T_b-1,U_b)),  L = sum_b cost_b
  output-score gradient f^W_4 (Eq. (10)), with g_b = dL/dcost_b
      dh[t,u,v] = g_b * (occ*softmax_v - [v=blank]*bflow - [v=y[u+1]]*lflow)
      occ   = exp(alpha(t,u) + beta(t,u) - lnP)
      bflow = exp(alpha(t,u) + phi(t,u) + beta(t+1,u) - lnP), beta(T_b,U_b) := 0
      lflow = exp(alpha(t,u) + psi(t,u) + beta(t,u+1) - lnP)
  backward through output layer and joint network (Algorithm 1's gradient
  accumulation), summed over samples in order b = 0..B-1:
      dz = W^O^T dh;  dW^O += dh z^T;  db^O += dh;  ds = dz * (1 - z^2)
      gA[t] = sum_u ds[t,u];  gL[u] = sum_t ds[t,u]
      dW^A += gA h^A^T;  db^Z += sum_t gA;  dh^A = W^A^T gA
      dW^L += gL h^L^T;  dh^L = W^L^T gL
  Padded positions (t >= T_b, u > U_b) take no part; their gradient rows are 0.

Evaluation order: the forward and backward recursions are evaluated one
anti-diagonal t+u = d at a time (every cell on a diagonal depends only on the
previous one), which is the recursion itself, vectorised. The joint/output
steps are evaluated over blocks of t rows only to bound host memory; each
cell's value is the same function of its own inputs whatever the block.

Pruned lattice (the pruning named in "Neural transducer training ...",
Introduction and Conclusion, and the title of its reference 14; the pages
give no definition, so this is the reading implemented): given a band of S
label positions per frame, lo[t] <= u < lo[t] + S, cells outside the band are
removed from the lattice: their two log-probs are taken as -inf, so the loss
sums the probability of the alignments whose every cell lies in the band,
and such cells get no gradient (their occupancy and flows are 0). The band
is an input (where it comes from is outside the method on these pages).

Reduced-precision output layer ("Neural transducer training ...",
Introduction, reduced precision among the ways to cut memory, and its
Conclusion, mixed precision as future work; the pages do not define it, so
this is the reading implemented): with fp8_scores, the product W^O z of the
output layer takes its two operands rounded to the OCP FP8 E4M3 format
(1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest finite value
448, round to nearest with ties to even) after power-of-two scaling: z by
2^8 (|z| <= 1), W^O by 2^e_w with e_w the largest integer for which
max|W^O| 2^e_w <= 448; the exact product of the rounded values is scaled
back by 2^-(8 + e_w) and b^O added. Everything else is unchanged: lse, phi,
psi and dh come from these scores (the forward and the backward's), and the
two backward products dz = W^O^T dh and dW^O = dh z^T take the unrounded
W^O and z, as does 1 - z^2.

Pins (tests/test_oracle_pins.py): brute-force enumeration of every monotone
alignment on tiny lattices, the alpha/beta identity, closed forms with
W^O = 0, occupancy closed form, torch fp64 log_softmax, flow and row-sum
invariants, central finite differences of every input and parameter, and an
independent torch fp64 autograd implementation.
"""
from __future__ import annotations

import dataclasses

import numpy as np

NEG_INF = -np.inf


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def logaddexp(a, b):
    """log(exp(a) + exp(b)) elementwise; -inf if both are -inf (never NaN)."""
    return np.logaddexp(a, b)


def joint(hA_b, hL_b, WA, WL, bZ):
    """Eqs. (3)-(4): z[t,u] = tanh(W^A h^A[t] + W^L h^L[u] + b^Z) -> [T_b,U_b+1,H].

    W^A h^A[t] + b^Z depends on t alone and W^L h^L[u] on u alone; their sum
    is formed per (t,u) before tanh.
    """
    a = _f64(hA_b) @ _f64(WA).T + _f64(bZ)  # [T_b, H]
    l = _f64(hL_b) @ _f64(WL).T  # [U_b+1, H]
    return np.tanh(a[:, None, :] + l[None, :, :])


def tanh_grad(z):
    """d tanh(s)/ds expressed through z = tanh(s): 1 - z^2."""
    return 1.0 - z * z


def encoding_grad(g, W):
    """Rows of W^T g for each row g[i] of g (dh^A = W^A^T gA, dh^L = W^L^T gL)."""
    return g @ W


def output_layer(z, WO, bO):
    """Eqs. (5)-(6): h[t,u] = W^O z[t,u] + b^O -> [..., V]."""
    return z @ _f64(WO).T + _f64(bO)


E4M3_MAX = 448.0
Z_SCALE_EXP = 8  # z in [-1, 1] is scaled by 2^8 before rounding


def e4m3_round(x):
    """Nearest OCP FP8 E4M3 value of each element (ties to even), as fp64.

    The format's normal numbers have exponents -6..8 and 3 fraction bits, so
    in the binade [2^k, 2^(k+1)) the spacing is 2^(k-3); below 2^-6 the
    subnormals keep the spacing 2^-9. Rounding the value divided by its
    spacing to the nearest integer (ties to even) is rounding to the
    format. Magnitudes above 448 are outside what this oracle uses.
    """
    x = _f64(x)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value beyond the E4M3 range")
    _, e = np.frexp(a)  # a = m 2^e with m in [0.5, 1): binade exponent e - 1
    k = np.maximum(e - 1, -6)
    q = np.ldexp(np.round(np.ldexp(a, 3 - k)), k - 3)
    return np.copysign(q, x)


def wo_scale_exp(WO):
    """Largest integer e with max|W^O| 2^e <= 448 (0 for an all-zero W^O)."""
    amax = float(np.max(np.abs(_f64(WO)))) if np.size(WO) else 0.0
    if amax == 0.0:
        return 0
    m, e = np.frexp(amax)  # amax = m 2^e, m in [0.5, 1); 448 = 0.875 2^9
    return int(9 - e if m <= 0.875 else 8 - e)


def output_layer_fp8(z, WO, bO):
    """Eqs. (5)-(6) with the product on E4M3-rounded, power-of-two scaled operands."""
    ew = wo_scale_exp(WO)
    zq = e4m3_round(np.ldexp(_f64(z), Z_SCALE_EXP))
    wq = e4m3_round(np.ldexp(_f64(WO), ew))
    return np.ldexp(zq @ wq.T, -(Z_SCALE_EXP + ew)) + _f64(bO)


def log_softmax_denominator(h):
    """Eq. (7) in the log domain: lse = m + log(sum_v exp(h_v - m)), m = max_v h_v."""
    m = np.max(h, axis=-1)
    return m + np.log(np.sum(np.exp(h - m[..., None]), axis=-1))


def two_log_probs(h, lse, y_b, U_b, blank):
    """phi = h[blank] - lse on every cell; psi = h[y[u+1]] - lse for u < U_b (else -inf)."""
    phi = h[..., blank] - lse
    psi = np.full(phi.shape, NEG_INF)
    if U_b > 0:
        lab = np.asarray(y_b[1:U_b + 1], dtype=np.int64)  # label emitted from row u
        psi[:, :U_b] = np.take_along_axis(h[:, :U_b, :], lab[None, :, None], axis=2)[..., 0] - lse[:, :U_b]
    return phi, psi


def alpha_recursion(phi, psi):
    """Eq. (8) forward variables over the T_b x (U_b+1) lattice, by anti-diagonals."""
    Tb, U1 = phi.shape
    alpha = np.full((Tb, U1), NEG_INF)
    alpha[0, 0] = 0.0
    for d in range(1, Tb + U1 - 1):
        t = np.arange(max(0, d - U1 + 1), min(Tb - 1, d) + 1)
        u = d - t
        from_t = np.full(t.shape, NEG_INF)  # arrive by blank from (t-1, u)
        m = t > 0
        from_t[m] = alpha[t[m] - 1, u[m]] + phi[t[m] - 1, u[m]]
        from_u = np.full(t.shape, NEG_INF)  # arrive by label from (t, u-1)
        m = u > 0
        from_u[m] = alpha[t[m], u[m] - 1] + psi[t[m], u[m] - 1]
        alpha[t, u] = logaddexp(from_t, from_u)
    return alpha


def beta_recursion(phi, psi):
    """Eq. (8) backward variables; beta(T_b-1,U_b) = phi(T_b-1,U_b), by anti-diagonals."""
    Tb, U1 = phi.shape
    beta = np.full((Tb, U1), NEG_INF)
    beta[Tb - 1, U1 - 1] = phi[Tb - 1, U1 - 1]
    for d in range(Tb + U1 - 3, -1, -1):
        t = np.arange(max(0, d - U1 + 1), min(Tb - 1, d) + 1)
        u = d - t
        by_blank = np.full(t.shape, NEG_INF)  # leave by blank to (t+1, u)
        m = t + 1 < Tb
        by_blank[m] = phi[t[m], u[m]] + beta[t[m] + 1, u[m]]
        by_label = np.full(t.shape, NEG_INF)  # leave by label to (t, u+1)
        m = u + 1 < U1
        by_label[m] = psi[t[m], u[m]] + beta[t[m], u[m] + 1]
        beta[t, u] = logaddexp(by_blank, by_label)
    return beta


def flows(alpha, beta, phi, psi, lnP):
    """occ, bflow, lflow (unscaled) per cell; beta(T_b, U_b) := 0 for the final blank."""
    Tb, U1 = phi.shape
    beta_next_t = np.full((Tb, U1), NEG_INF)  # beta(t+1, u)
    beta_next_t[:-1, :] = beta[1:, :]
    beta_next_t[Tb - 1, U1 - 1] = 0.0
    beta_next_u = np.full((Tb, U1), NEG_INF)  # beta(t, u+1)
    beta_next_u[:, :-1] = beta[:, 1:]
    occ = np.exp(alpha + beta - lnP)
    bflow = np.exp(alpha + phi + beta_next_t - lnP)
    lflow = np.exp(alpha + psi + beta_next_u - lnP)
    return occ, bflow, lflow


def logits_grad(h, lse, occ, bflow, lflow, y_b, U_b, blank, g):
    """Eq. (10): dh = g*(occ*softmax - [v=blank]*bflow - [v=y[u+1]]*lflow) on a block of rows.

    h, lse, occ, bflow, lflow cover rows t of the lattice (all U_b+1 columns).
    When y[u+1] is the blank id both corrections land on that column.
    """
    p = np.exp(h - lse[..., None])  # softmax
    dh = occ[..., None] * p
    dh[:, :, blank] -= bflow
    if U_b > 0:
        lab = np.asarray(y_b[1:U_b + 1], dtype=np.int64)
        tt, uu = np.meshgrid(np.arange(h.shape[0]), np.arange(U_b), indexing="ij")
        dh[tt, uu, lab[uu]] -= lflow[:, :U_b]
    return g * dh


def lattice_from_logits(h, y_b, U_b, blank):
    """Loss pieces from a sample's logits h [T_b, U_b+1, V] (Eqs. (7)-(9)).

    Returns (cost, lse, phi, psi, alpha, beta).
    """
    lse = log_softmax_denominator(h)
    phi, psi = two_log_probs(h, lse, y_b, U_b, blank)
    alpha = alpha_recursion(phi, psi)
    beta = beta_recursion(phi, psi)
    Tb = h.shape[0]
    return -(alpha[Tb - 1, U_b] + phi[Tb - 1, U_b]), lse, phi, psi, alpha, beta


def dlogits(h, y_b, U_b, blank, g=1.0):
    """dcost/dh for a sample's full logits h [T_b, U_b+1, V] (Eq. (10))."""
    cost, lse, phi, psi, alpha, beta = lattice_from_logits(h, y_b, U_b, blank)
    occ, bflow, lflow = flows(alpha, beta, phi, psi, -cost)
    return logits_grad(h, lse, occ, bflow, lflow, y_b, U_b, blank, g)


@dataclasses.dataclass
class SampleResult:
    cost: float
    lnP: float
    lse: np.ndarray  # [T_b, U_b+1]
    phi: np.ndarray
    psi: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    grads: dict | None = None  # per-sample gradients (see loss_and_grads)
    occ: np.ndarray | None = None
    bflow: np.ndarray | None = None
    lflow: np.ndarray | None = None


def _rows_per_block(U1, V, H, budget_bytes):
    return max(1, int(budget_bytes // max(1, U1 * (V + 2 * H) * 8)))


def band_mask(lo_b, S, Tb, U1):
    """In-band cells of a pruned lattice: lo[t] <= u < lo[t] + S, [T_b, U_b+1] booleans."""
    u = np.arange(U1)[None, :]
    lo = np.asarray(lo_b[:Tb], dtype=np.int64)[:, None]
    return (u >= lo) & (u < lo + S)


def sample_forward_backward(inp, b, g=1.0, *, want_grads=True, keep_flows=False,
                            mem_budget=512 << 20, band=None, fp8_scores=False):
    """Loss and gradients of sample b alone (Algorithm 1's loop body).

    g is dL/dcost_b. band: None, or (lo [T] int array of this sample, S) for
    the pruned lattice (cells outside lo[t] <= u < lo[t] + S removed).
    fp8_scores: the output layer's product on E4M3-rounded operands
    (output_layer_fp8); the backward products keep the unrounded ones.
    Returns a SampleResult whose grads dict holds this sample's contributions:
    dWO, dbO, dWA, dWL, dbZ (parameter shaped) and dhA_b [T_b, HA],
    dhL_b [U_b+1, HL].
    """
    Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
    if Tb < 1 or Ub < 0:
        raise ValueError("need T_b >= 1 and U_b >= 0")
    U1 = Ub + 1
    blank = int(inp.blank)
    WA, WL, bZ = _f64(inp.WA), _f64(inp.WL), _f64(inp.bZ)
    WO, bO = _f64(inp.WO), _f64(inp.bO)
    V, H = WO.shape
    hA_b = _f64(inp.hA[b, :Tb])
    hL_b = _f64(inp.hL[b, :U1])
    y_b = np.asarray(inp.labels[b])
    rows = _rows_per_block(U1, V, H, mem_budget)
    scores = output_layer_fp8 if fp8_scores else output_layer

    # forward: per-cell lse, phi, psi (z and h are discarded per block)
    lse = np.empty((Tb, U1))
    phi = np.empty((Tb, U1))
    psi = np.empty((Tb, U1))
    for t0 in range(0, Tb, rows):
        t1 = min(Tb, t0 + rows)
        z = joint(hA_b[t0:t1], hL_b, WA, WL, bZ)
        h = scores(z, WO, bO)
        lse[t0:t1] = log_softmax_denominator(h)
        phi[t0:t1], psi[t0:t1] = two_log_probs(h, lse[t0:t1], y_b, Ub, blank)
    if band is not None:
        # pruned lattice: no emission leaves a cell outside the band
        out = ~band_mask(band[0], band[1], Tb, U1)
        phi[out] = NEG_INF
        psi[out] = NEG_INF

    alpha = alpha_recursion(phi, psi)
    beta = beta_recursion(phi, psi)
    lnP = alpha[Tb - 1, Ub] + phi[Tb - 1, Ub]
    res = SampleResult(cost=-lnP, lnP=lnP, lse=lse, phi=phi, psi=psi, alpha=alpha, beta=beta)
    if not want_grads and not keep_flows:
        return res
    occ, bflow, lflow = flows(alpha, beta, phi, psi, lnP)
    if keep_flows:
        res.occ, res.bflow, res.lflow = occ, bflow, lflow
    if not want_grads:
        return res

    dWO = np.zeros((V, H))
    dbO = np.zeros(V)
    gA = np.zeros((Tb, H))
    gL = np.zeros((U1, H))
    for t0 in range(0, Tb, rows):
        t1 = min(Tb, t0 + rows)
        z = joint(hA_b[t0:t1], hL_b, WA, WL, bZ)
        h = scores(z, WO, bO)
        dh = logits_grad(h, lse[t0:t1], occ[t0:t1], bflow[t0:t1], lflow[t0:t1],
                         y_b, Ub, blank, g)
        dz = dh @ WO  # [t, U1, H]
        dWO += dh.reshape(-1, V).T @ z.reshape(-1, H)
        dbO += dh.sum(axis=(0, 1))
        ds = dz * tanh_grad(z)
        gA[t0:t1] = ds.sum(axis=1)
        gL += ds.sum(axis=0)
    res.grads = dict(
        dWO=dWO, dbO=dbO,
        dWA=gA.T @ hA_b, dbZ=gA.sum(axis=0), dhA_b=encoding_grad(gA, WA),
        dWL=gL.T @ hL_b, dhL_b=encoding_grad(gL, WL),
        gA=gA, gL=gL,
    )
    return res


@dataclasses.dataclass
class BatchResult:
    costs: np.ndarray  # [B] fp64
    grads: dict | None  # dhA [B,T,HA], dhL [B,U+1,HL], dWA, dWL, dbZ, dWO, dbO
    samples: list  # SampleResult per computed sample (None if skipped)


def loss_and_grads(inp, dcosts=None, *, samples=None, want_grads=True, keep_flows=False,
                   mem_budget=512 << 20, band=None, fp8_scores=False):
    """Batch loss and gradients: per-sample results summed over b in order.

    dcosts: [B] upstream gradient (None = all ones, i.e. L = sum of costs).
    samples: optional subset of sample indices to compute; the others get
    cost NaN and contribute nothing to the gradients (so the gradients equal
    the full-batch ones when dcosts is zero outside the subset).
    band: None, or (lo [B, T] int array, S) for the pruned lattice.
    fp8_scores: the output layer's product on E4M3-rounded operands.
    """
    d = inp.dims
    B, T, U, V, HA, HL, H = (d[k] for k in ("B", "T", "U", "V", "HA", "HL", "H"))
    g = np.ones(B) if dcosts is None else _f64(dcosts)
    which = range(B) if samples is None else samples
    costs = np.full(B, np.nan)
    out = [None] * B
    grads = None
    if want_grads:
        grads = dict(dhA=np.zeros((B, T, HA)), dhL=np.zeros((B, U + 1, HL)),
                     dWA=np.zeros((H, HA)), dWL=np.zeros((H, HL)), dbZ=np.zeros(H),
                     dWO=np.zeros((V, H)), dbO=np.zeros(V))
    for b in which:
        r = sample_forward_backward(inp, b, float(g[b]), want_grads=want_grads,
                                    keep_flows=keep_flows, mem_budget=mem_budget,
                                    band=None if band is None else (band[0][b], band[1]),
                                    fp8_scores=fp8_scores)
        costs[b] = r.cost
        out[b] = r
        if want_grads:
            sg = r.grads
            Tb, U1 = int(inp.T_len[b]), int(inp.U_len[b]) + 1
            grads["dhA"][b, :Tb] = sg["dhA_b"]
            grads["dhL"][b, :U1] = sg["dhL_b"]
            for k in ("dWA", "dWL", "dbZ", "dWO", "dbO"):
                grads[k] += sg[k]
    return BatchResult(costs=costs, grads=grads, samples=out)


def brute_force_cost(phi, psi):
    """-log of the summed probability of every monotone alignment path.

    A path from (0,0) makes T_b-1 blank moves (t+1) and U_b label moves (u+1)
    in some order, then the final blank at (T_b-1, U_b); its log-probability
    is the sum of phi/psi at the cells it leaves. Enumerates all
    C(T_b-1+U_b, U_b) orders; for tiny lattices only.
    """
    import itertools

    Tb, U1 = phi.shape
    Ub = U1 - 1
    n = Tb - 1 + Ub
    logps = []
    for label_steps in itertools.combinations(range(n), Ub):
        ls = set(label_steps)
        t = u = 0
        lp = 0.0
        for step in range(n):
            if step in ls:
                lp += psi[t, u]
                u += 1
            else:
                lp += phi[t, u]
                t += 1
        lp += phi[Tb - 1, Ub]
        logps.append(lp)
    logps = np.array(logps)
    m = logps.max()
    return -(m + np.log(np.sum(np.exp(logps - m))))
