"""Seeded synthetic inputs for the RNN-T joint + loss path.

This module only draws numbers. It holds none of the transducer arithmetic
and is the single source of inputs shared by the fp64 oracle and by the HIP
library's tests and benchmark, so both sides see identical values.

Shapes follow "Neural transducer training: reduced memory consumption with
sample-wise computation" (section "Transducer training"): acoustic encodings
h^A [B,T,H_A], label encodings h^L [B,U+1,H_L], labels [B,U+1] with the blank
id prepended in column 0, joint weights W^A [H,H_A], W^L [H,H_L], b^Z [H] and
output layer W^O [V,H], b^O [V].

Draw order is fixed: lengths, labels, h^A, h^L, W^A, W^L, W^O, then biases.
Float values are rounded once to the working dtype (bf16 round-to-nearest-even
when dtype == "bf16") and returned as float32 arrays holding exactly those
values, so either side can widen them without loss.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLANK = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    """Dimensions and value distributions of one synthetic workload."""

    name: str
    B: int
    T: int
    U: int
    V: int
    HA: int
    HL: int
    H: int
    dtype: str  # "f32" or "bf16"
    enc: str  # "normal0.5" (the tiny workload) or "normal1"
    weights: str  # "normal0.5" or "xavier"
    labels: str  # "uniform" or "zipf1.1"
    t_range: tuple  # inclusive integer range for T_b
    u_range: tuple  # inclusive integer range for U_b
    seed: int
    tiles: tuple = ((64, 32),)  # tile sizes (t x u) this workload is run with


def _frac_range(lo_frac: float, n: int) -> tuple:
    return (int(math.ceil(lo_frac * n)), n)


# The five workloads: a tiny fp32 lattice for brute force, then bf16 batches
# shaped like ~10 s, ~20 s and ~40 s utterances at 40 ms frames, plus a
# 4096-token vocabulary case. Lengths are integer-uniform over the ranges.
WORKLOADS = {
    "tiny-f32": Workload("tiny-f32", 2, 6, 3, 5, 8, 8, 8, "f32", "normal0.5", "normal0.5",
                "uniform", (6, 6), (3, 3), seed=1, tiles=((64, 32),)),
    "small-bf16": Workload("small-bf16", 8, 250, 64, 1024, 512, 512, 640, "bf16", "normal1",
                "xavier", "uniform", (150, 250), (32, 64), seed=2,
                tiles=((64, 32),)),
    "20s-bf16": Workload("20s-bf16", 32, 500, 120, 1024, 512, 512, 640, "bf16", "normal1",
                "xavier", "uniform", _frac_range(0.6, 500), _frac_range(0.6, 120),
                seed=3, tiles=((64, 32),)),
    "vocab4096-bf16": Workload("vocab4096-bf16", 16, 400, 150, 4096, 640, 640, 640, "bf16",
                "normal1", "xavier", "zipf1.1", _frac_range(0.6, 400),
                _frac_range(0.6, 150), seed=4, tiles=((32, 16), (64, 32), (128, 64))),
    "40s-b256-bf16": Workload("40s-b256-bf16", 256, 1000, 200, 1024, 512, 512, 640, "bf16",
                "normal1", "xavier", "uniform", _frac_range(0.5, 1000),
                _frac_range(0.5, 200), seed=5, tiles=((64, 32),)),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    NaN stays NaN and infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def _zipf_labels(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """Truncated Zipf(s) on 1..V-1 by inverse CDF over the finite support."""
    k = np.arange(1, V, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]
    u = rng.random(n)
    return (np.searchsorted(cdf, u, side="left") + 1).astype(np.int32)


def _draw_lengths(rng: np.random.Generator, B: int, T: int, U: int, t_range, u_range):
    """The first draws of every batch: T_b, then U_b, integer-uniform over the inclusive ranges."""
    t_lo, t_hi = t_range if t_range is not None else (T, T)
    u_lo, u_hi = u_range if u_range is not None else (U, U)
    if not (1 <= t_lo <= t_hi <= T and 0 <= u_lo <= u_hi <= U):
        raise ValueError("bad length ranges")
    T_len = rng.integers(t_lo, t_hi + 1, size=B).astype(np.int32)
    U_len = rng.integers(u_lo, u_hi + 1, size=B).astype(np.int32)
    return T_len, U_len


def workload_lengths(cfg: str, *, seed: int | None = None):
    """(T_len, U_len) of a named workload's batch without drawing the rest (the lengths are the
    first draws, so they equal workload_inputs(cfg).T_len / .U_len)."""
    w = WORKLOADS[cfg]
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    return _draw_lengths(rng, w.B, w.T, w.U, w.t_range, w.u_range)


@dataclasses.dataclass
class Inputs:
    """One batch of inputs. Float arrays are float32 holding dtype-exact values."""

    dtype: str
    blank: int
    T_len: np.ndarray  # int32 [B]
    U_len: np.ndarray  # int32 [B]
    labels: np.ndarray  # int32 [B, U+1], column 0 = blank, past U_b = blank
    hA: np.ndarray  # [B, T, HA]
    hL: np.ndarray  # [B, U+1, HL]
    WA: np.ndarray  # [H, HA]
    WL: np.ndarray  # [H, HL]
    bZ: np.ndarray  # [H]
    WO: np.ndarray  # [V, H]
    bO: np.ndarray  # [V]

    @property
    def dims(self):
        B, T, HA = self.hA.shape
        U1, HL = self.hL.shape[1], self.hL.shape[2]
        V, H = self.WO.shape
        return dict(B=B, T=T, U=U1 - 1, V=V, HA=HA, HL=HL, H=H)

    @property
    def valid_cells(self) -> int:
        return int(np.sum(self.T_len.astype(np.int64) * (self.U_len.astype(np.int64) + 1)))

    @property
    def padded_cells(self) -> int:
        d = self.dims
        return d["B"] * d["T"] * (d["U"] + 1)


def make_inputs(B: int, T: int, U: int, V: int, HA: int, HL: int, H: int, *,
                dtype: str = "f32", seed: int = 0, enc: str = "normal1",
                weights: str = "xavier", labels: str = "uniform",
                t_range=None, u_range=None, bias_std: float = 0.0,
                blank: int = BLANK) -> Inputs:
    """Draw a batch with the given dimensions and distributions.

    enc/weights: "normal1" = N(0,1); "normal0.5" = N(0, sd 0.5); "xavier" =
    U(-sqrt(6/(fan_in+fan_out)), +sqrt(...)) per weight matrix. Labels are
    uniform on the non-blank ids or truncated Zipf(1.1) on 1..V-1 (blank must
    be 0 for the label draws to avoid it). bias_std > 0 draws N(0, bias_std)
    biases instead of zeros (used by tests that need non-zero biases).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    # 1. lengths
    T_len, U_len = _draw_lengths(rng, B, T, U, t_range, u_range)
    # 2. labels (blank-prepended; entries past U_b are blank)
    if V < 2:
        raise ValueError("need V >= 2")
    n_lab = B * U
    if labels == "uniform":
        lab = rng.integers(1, V, size=n_lab).astype(np.int32)
    elif labels == "zipf1.1":
        lab = _zipf_labels(rng, n_lab, V, 1.1)
    else:
        raise ValueError(labels)
    if blank != 0:
        # keep labels off the blank id by mapping it to 0 (the id it displaced)
        lab = np.where(lab == blank, 0, lab).astype(np.int32)
    lab = lab.reshape(B, U)
    y = np.full((B, U + 1), blank, dtype=np.int32)
    y[:, 1:] = lab
    for b in range(B):
        y[b, 1 + U_len[b]:] = blank

    def enc_draw(shape):
        if enc == "normal1":
            return rng.standard_normal(shape, dtype=np.float32)
        if enc == "normal0.5":
            return 0.5 * rng.standard_normal(shape, dtype=np.float32)
        raise ValueError(enc)

    def w_draw(rows, cols):
        if weights == "xavier":
            bound = math.sqrt(6.0 / (rows + cols))
            return rng.uniform(-bound, bound, size=(rows, cols)).astype(np.float32)
        if weights == "normal0.5":
            return 0.5 * rng.standard_normal((rows, cols), dtype=np.float32)
        if weights == "normal1":
            return rng.standard_normal((rows, cols), dtype=np.float32)
        raise ValueError(weights)

    # 3.-7. encodings and weights
    hA = enc_draw((B, T, HA))
    hL = enc_draw((B, U + 1, HL))
    WA = w_draw(H, HA)
    WL = w_draw(H, HL)
    WO = w_draw(V, H)
    # 8. biases
    if bias_std > 0:
        bZ = bias_std * rng.standard_normal(H, dtype=np.float32)
        bO = bias_std * rng.standard_normal(V, dtype=np.float32)
    else:
        bZ = np.zeros(H, dtype=np.float32)
        bO = np.zeros(V, dtype=np.float32)
    cv = lambda a: _as_dtype(a, dtype)
    return Inputs(dtype=dtype, blank=blank, T_len=T_len, U_len=U_len, labels=y,
                  hA=cv(hA), hL=cv(hL), WA=cv(WA), WL=cv(WL), bZ=cv(bZ),
                  WO=cv(WO), bO=cv(bO))


def workload_inputs(cfg: str, *, seed: int | None = None, dtype: str | None = None,
                    B: int | None = None) -> Inputs:
    """Inputs for one of the five named workloads (seed defaults to the workload's own).

    B overrides the batch size (the first B samples' lengths then differ from
    the full-batch draw, since lengths are drawn per batch).
    """
    w = WORKLOADS[cfg]
    return make_inputs(B if B is not None else w.B, w.T, w.U, w.V, w.HA, w.HL, w.H,
                       dtype=dtype or w.dtype, seed=w.seed if seed is None else seed,
                       enc=w.enc, weights=w.weights, labels=w.labels,
                       t_range=w.t_range, u_range=w.u_range)


def poison_padding(inp: Inputs) -> Inputs:
    """Copy of inp with every padded position set to NaN (labels to V+7).

    Padded positions are h^A rows t >= T_b, h^L rows u > U_b and label
    columns past U_b. Results must not depend on them.
    """
    hA = inp.hA.copy()
    hL = inp.hL.copy()
    y = inp.labels.copy()
    V = inp.WO.shape[0]
    for b in range(len(inp.T_len)):
        hA[b, inp.T_len[b]:] = np.nan
        hL[b, inp.U_len[b] + 1:] = np.nan
        y[b, inp.U_len[b] + 1:] = V + 7
    return dataclasses.replace(inp, hA=hA, hL=hL, labels=y)


def diagonal_band(T_len, U_len, T: int, S: int) -> np.ndarray:
    """Label-position bands of width S for a pruned lattice, lo [B, T] int32: per frame t
    the band lo[t] <= u < lo[t] + S is centred on the straight line from (0, 0) to
    (T_b - 1, U_b), clipped to [0, U_b], with lo[0] = 0, lo non-decreasing, steps of at
    most S - 1 and the last frame's band reaching U_b (so the band holds an alignment).
    Frames past T_b get 0. A synthetic stand-in for bounds that come from a model."""
    B = len(T_len)
    lo = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        Tb, Ub = int(T_len[b]), int(U_len[b])
        top = max(0, Ub - S + 1)
        prev = 0
        for t in range(Tb):
            c = (t * Ub) // max(1, Tb - 1)
            v = min(max(c - (S - 1) // 2, 0), top)
            v = min(max(v, prev), prev + S - 1)
            lo[b, t] = v
            prev = v
        if lo[b, Tb - 1] + S - 1 < Ub:
            raise ValueError(f"band width {S} too narrow for sample {b} (T_b={Tb}, U_b={Ub})")
    return lo
