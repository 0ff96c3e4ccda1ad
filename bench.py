"""Benchmark: RNN-T fwd+bwd lattice cells/s (B*T*(U+1)) at V=1024 and peak HBM bytes.

One step = rnnt_loss_fwd + rnnt_loss_bwd over one batch of the workload, with
inputs already resident in HBM. K steps are timed after W warm-up steps.
Prints one JSON line. The headline ms_per_step and value come from a timed
pass with nothing but the library's launches; a second pass over the same K
steps brackets every launch with a hipEvent pair on its stream (the library's
launch timing) for the per-kernel durations, the roofline object of the
dominant kernel and t_fwd / t_bwd. The fp64 CPU oracle is timed on a bounded
sample of the same workload as cpu_baseline, one sample per worker process,
before the GPU is initialised.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--workload 40s-b256-bf16]
    python bench.py --calibrate-copy BYTES   # counter calibration only
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "fp8": 5000.0}  # MI355X dense MFMA
FP8_KERNELS = ("scores_fwd", "scores_bwd")  # the products on E4M3 operands with --fp8
PEAK_HBM_GBS = 8000.0
GEMM_KERNELS = ("joint_fwd", "joint_bwd", "scores_fwd", "scores_bwd", "dz", "dWO_gemm", "dz_dwo")
# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled
# by a 1 GiB device copy: x2.000 / x1.000) on the 40 s x 256 workload; the
# figure applies only while the kernel's sources hash to `src` (else null).
# The kernel's sources: whole files, or (file, "struct Name") for one struct's definition in a
# shared header (the argument structs the kernel takes).
TRAFFIC = {
    "dz_dwo": {"bytes": 4.120e9, "src": "8684baf37b16b2b7",
               "files": ("rnn_loss_joint_amd/csrc/dz_dwo.hip", "rnn_loss_joint_amd/csrc/mfma_core.hpp",
                         "rnn_loss_joint_amd/csrc/common.hpp", "rnn_loss_joint_amd/csrc/common_host.hpp",
                         ("rnn_loss_joint_amd/csrc/kernels.hpp", "struct DzArgs"),
                         ("rnn_loss_joint_amd/csrc/kernels.hpp", "struct DwoArgs")),
               "profile": "profiles/hbm_traffic_40s_b256_bf16.md", "workload": "40s-b256-bf16"},
}


def source_hash(files):
    """First 16 hex digits of the sha256 over the listed sources (see TRAFFIC)."""
    import hashlib

    h = hashlib.sha256()
    for f in files:
        path, struct = (f, None) if isinstance(f, str) else f
        with open(os.path.join(ROOT, path), "rb") as fh:
            text = fh.read()
        if struct is not None:
            i = text.index(struct.encode() + b" {")
            text = text[i:text.index(b"\n};", i) + 3]
        h.update(text)
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """Measured HBM bytes per launch if the kernel's sources are unchanged."""
    t = TRAFFIC.get(kernel)
    if t is None or t["workload"] != workload:
        return None
    return t["bytes"] if source_hash(t["files"]) == t["src"] else None


FLOP_FORMULA = {"dz_dwo": "4*H*V*valid_cells", "preproj_gemm": "2*H*(rows_a*HA + rows_l*HL)",
                "dh_enc_gemm": "2*H*(rows_a*HA + rows_l*HL)", "dW_enc_gemm": "2*H*(rows_a*HA + rows_l*HL)"}


def band_cells(inp, band):
    """Lattice cells inside a pruned lattice's bands: per frame t < T_b, the label positions
    lo[b, t] <= u < lo[b, t] + S that are at most U_b."""
    lo, S = band
    n = 0
    for b in range(len(inp.T_len)):
        Tb, Ub = int(inp.T_len[b]), int(inp.U_len[b])
        l = lo[b, :Tb].astype(np.int64)
        n += int(np.sum(np.minimum(l + S, Ub + 1) - l))
    return n


def mfma_flops(inp, cells=None):
    """Algorithmic FLOP of each MFMA kernel class over one step (valid cells only, or the given
    count of computed lattice cells: the in-band cells of a pruned lattice)."""
    d = inp.dims
    H, V, HA, HL = d["H"], d["V"], d["HA"], d["HL"]
    Nc = inp.valid_cells if cells is None else cells
    rows_a = int(np.sum(inp.T_len))
    rows_l = int(np.sum(inp.U_len + 1))
    pre = 2.0 * H * (rows_a * HA + rows_l * HL)
    return {
        "joint_fwd": 2.0 * H * V * Nc,   # scores for every valid cell (fp32 path)
        "joint_bwd": 2.0 * H * V * Nc,   # recomputed scores (fp32 path)
        "scores_fwd": 2.0 * H * V * Nc,  # scores for every valid cell (bf16 path)
        "scores_bwd": 2.0 * H * V * Nc,  # recomputed scores (bf16 path)
        "dz": 2.0 * H * V * Nc,          # dz = dh W^O (fp32 path)
        "dz_dwo": 4.0 * H * V * Nc,      # dz = dh W^O and dW^O = dh^T z in one launch (bf16 path)
        "dWO_gemm": 2.0 * H * V * Nc,    # dW^O = dh^T z
        "preproj_gemm": pre,             # a = W^A h^A, l = W^L h^L
        "dh_enc_gemm": pre,              # dh^A, dh^L
        "dW_enc_gemm": pre,              # dW^A, dW^L
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_one_sample(args):
    """Pool worker: the oracle's fwd + bwd of one sample (BLAS limited to one thread)."""
    inp, b = args
    import oracle
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.loss_and_grads(inp, samples=[0])
        return b, time.perf_counter() - t0


def _one_sample_inputs(inp, b):
    """The batch's sample b alone (B = 1, the same padded shapes), for shipping to a worker."""
    import dataclasses

    return dataclasses.replace(inp, T_len=inp.T_len[b:b + 1].copy(), U_len=inp.U_len[b:b + 1].copy(),
                               labels=inp.labels[b:b + 1].copy(), hA=inp.hA[b:b + 1].copy(),
                               hL=inp.hL[b:b + 1].copy())


def cpu_baseline(inp, budget_s: float, workers: int | None = None):
    """Time the oracle (as it stands) on the host cores: one sample per worker process, BLAS at one
    thread per worker, over a bounded sample of the workload's batch.

    Samples are taken in a fixed shuffled order (seed 0) so the sample's length mix follows the
    batch's; new samples are started until budget_s of wall time has passed, and the samples in
    flight are finished. The rate is the completed samples' valid cells over the wall time,
    reported with the padded numerator like the GPU figure (x padded / valid cells of the batch).
    Run before the GPU is initialised (the workers are fresh processes)."""
    import multiprocessing as mp

    n_cpu = len(os.sched_getaffinity(0))
    workers = workers or max(1, min(16, n_cpu))
    B = len(inp.T_len)
    order = [int(b) for b in np.random.default_rng(0).permutation(B)]
    env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved_env = {k: os.environ.get(k) for k in env_keys}
    for k in env_keys:
        os.environ[k] = "1"
    ctx = mp.get_context("spawn")
    done, cells = [], 0
    try:
        with ctx.Pool(workers) as pool:
            t0 = time.perf_counter()
            pending = []
            it = iter(order)
            for _ in range(workers):  # one sample per worker to start
                b = next(it, None)
                if b is not None:
                    pending.append(pool.apply_async(_oracle_one_sample, ((_one_sample_inputs(inp, b), b),)))
            while pending:
                r = pending.pop(0)
                b, _ = r.get()
                done.append(b)
                cells += int(inp.T_len[b]) * (int(inp.U_len[b]) + 1)
                if time.perf_counter() - t0 < budget_s:
                    nb = next(it, None)
                    if nb is not None:
                        pending.append(pool.apply_async(_oracle_one_sample, ((_one_sample_inputs(inp, nb), nb),)))
            wall = time.perf_counter() - t0
    finally:
        for k, v in saved_env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    valid_rate = cells / wall
    return {
        "value": valid_rate * inp.padded_cells / inp.valid_cells,
        "unit": "cells/s",
        "cores": int(workers),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle fwd+bwd, one sample per worker process ({workers} processes, BLAS at 1 "
                   f"thread each, {_cpu_model()}, {n_cpu} cores visible) on {len(done)} of the batch's {B} "
                   f"samples in a fixed shuffled order ({cells} valid cells, {wall:.1f} s wall); rate = valid "
                   f"cells/s x padded/valid cells of the batch ({inp.padded_cells}/{inp.valid_cells})"),
        "valid_cells_per_s": valid_rate,
        "cpu_model": _cpu_model(),
    }


def reference_gemm(torch, w, rows=524288):
    """Vendor bf16 GEMM (torch.matmul -> hipBLASLt) on the three product shapes of one wave of
    `rows` lattice cells: scores z W^O^T, dz = dh W^O, dW^O = dh^T z. Context for the fused kernels'
    MFMA fractions; these plain products fuse nothing."""
    R, H, V = rows, w.H, w.V
    g = torch.Generator(device="cuda").manual_seed(0)
    z = torch.randn(R, H, device="cuda", dtype=torch.bfloat16, generator=g)
    wo = torch.randn(V, H, device="cuda", dtype=torch.bfloat16, generator=g)
    dh = torch.randn(R, V, device="cuda", dtype=torch.bfloat16, generator=g)
    wot, dht = wo.t().contiguous(), dh.t().contiguous()
    out = {}
    for name, f in (("scores z W^O^T", lambda: torch.matmul(z, wot)), ("dz dh W^O", lambda: torch.matmul(dh, wo)),
                    ("dW^O dh^T z", lambda: torch.matmul(dht, z))):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        tf = 2.0 * R * H * V / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_TFLOPS["bf16"], 4)}
    print(json.dumps({"reference_gemm": out, "rows": R, "H": H, "V": V}))


def unfused_baseline(torch, rl, inp, steps, warmup):
    """Comparator for the fused, tiled path: an unfused batched RNN-T loss over the materialised
    [B, T, U+1, V] scores, as a warp-transducer style implementation computes it ("Neural transducer
    training ...", section "Transducer training", f^W_1..4 as separate passes): torch GEMMs,
    log_softmax and elementwise ops over the padded batch, this library's lattice kernel for alpha /
    beta. Benchmark only. Returns (ms per fwd+bwd, peak bytes, costs, {gradient name: tensor})."""
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    B, T, HA = inp.hA.shape
    U1, HL = inp.hL.shape[1], inp.hL.shape[2]
    U = U1 - 1
    V, H = inp.WO.shape
    blank = int(inp.blank)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(bf)
    hA, hL, WA, WL, bZ, WO, bO = map(up, (inp.hA, inp.hL, inp.WA, inp.WL, inp.bZ, inp.WO, inp.bO))
    # right operands of every product contiguous (transposed views in batched bf16 products are avoided)
    WAt, WLt, WOt = WA.t().contiguous(), WL.t().contiguous(), WO.t().contiguous()
    WAf, WLf = WA.float(), WL.float()
    lab = torch.from_numpy(np.ascontiguousarray(inp.labels[:, 1:], dtype=np.int64)).to(dev)  # [B, U]
    Tl = torch.from_numpy(np.ascontiguousarray(inp.T_len, dtype=np.int32)).to(dev)
    Ul = torch.from_numpy(np.ascontiguousarray(inp.U_len, dtype=np.int32)).to(dev)
    # the lattice arrays' layout: groups of four anti-diagonals per row
    NQ, US = (T + U1 - 1 + 3) // 4, (U1 + 31) // 32 * 32
    bi, ti, ui = torch.arange(B, device=dev), torch.arange(T, device=dev), torch.arange(U1, device=dev)
    dg = ti[None, :, None] + ui[None, None, :]
    diag = (((bi[:, None, None] * NQ + dg // 4) * US + ui[None, None, :]) * 4 + dg % 4).reshape(-1)
    desc = rl.make_desc(B, T, U, V, HA, HL, H)
    lab_idx = lab[:, None, :, None].expand(B, T, U, 1)
    neg = float("-inf")

    def fwd_bwd():
        a = torch.matmul(hA, WAt).float() + bZ.float()                     # [B, T, H]
        l = torch.matmul(hL, WLt).float()                                  # [B, U+1, H]
        z = torch.tanh(a[:, :, None, :] + l[:, None, :, :]).to(bf)         # [B, T, U+1, H]
        h = torch.matmul(z, WOt) + bO                                      # [B, T, U+1, V]
        logp = torch.log_softmax(h.float(), dim=-1)
        del h
        phi = logp[..., blank].contiguous()
        psi = torch.zeros_like(phi)
        psi[:, :, :U] = logp[:, :, :U, :].gather(-1, lab_idx)[..., 0]
        phid = torch.zeros(B * NQ * US * 4, device=dev)
        psid = torch.zeros_like(phid)
        phid[diag] = phi.reshape(-1)
        psid[diag] = psi.reshape(-1)
        ald = torch.full_like(phid, neg)
        bed = torch.full_like(phid, neg)
        costs = torch.zeros(B, device=dev)
        rl.rnnt_lattice(desc, Tl, Ul, phid, psid, ald, bed, costs)
        alpha, beta = ald[diag].view(B, T, U1), bed[diag].view(B, T, U1)   # -inf outside each lattice
        lnP = -costs[:, None, None]
        bt1 = torch.full_like(beta, neg)
        bt1[:, :-1] = beta[:, 1:]
        bt1[bi, Tl.long() - 1, Ul.long()] = 0.0                            # the terminal blank
        bu1 = torch.full_like(beta, neg)
        bu1[:, :, :-1] = beta[:, :, 1:]
        occ = torch.exp(alpha + beta - lnP)
        bflow = torch.exp(alpha + phi + bt1 - lnP)
        lflow = torch.exp(alpha + psi + bu1 - lnP)
        dh = torch.exp(logp) * occ[..., None]                              # d cost / d scores
        del logp
        dh[..., blank] -= bflow
        dh[:, :, :U, :].scatter_add_(-1, lab_idx, -lflow[:, :, :U, None])
        dh = dh.to(bf)
        dz = torch.matmul(dh, WO).float()                                  # [B, T, U+1, H]
        zf = z.float()
        ds = dz * (1.0 - zf * zf)
        del dz, zf
        gA, gL = ds.sum(2), ds.sum(1)
        del ds
        dhf = dh.reshape(-1, V)
        dWO = torch.matmul(dhf.t().contiguous(), z.reshape(-1, H)).float()
        dbO = dhf.float().sum(0)
        dhA, dhL = torch.matmul(gA, WAf), torch.matmul(gL, WLf)
        dWA = torch.matmul(gA.reshape(-1, H).t().contiguous(), hA.reshape(-1, HA).float())
        dWL = torch.matmul(gL.reshape(-1, H).t().contiguous(), hL.reshape(-1, HL).float())
        dbZ = gA.sum((0, 1))
        return costs, dict(dhA=dhA, dhL=dhL, dWA=dWA, dWL=dWL, dbZ=dbZ, dWO=dWO, dbO=dbO)

    for _ in range(warmup):
        out = fwd_bwd()
    del out
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        out = fwd_bwd()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, torch.cuda.max_memory_allocated(), out[0], out[1]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="40s-b256-bf16",
                    help="tiny-f32 | small-bf16 | 20s-bf16 | vocab4096-bf16 | 40s-b256-bf16")
    ap.add_argument("--mode", default="tiled", choices=["tiled", "untiled"])
    ap.add_argument("--tile", default="64x32", help="TxU, or 'sample' for whole-sample tiles (T x (U+1))")
    ap.add_argument("--tiles-per-wave", type=int, default=0)
    ap.add_argument("--budget", type=float, default=0, metavar="BYTES",
                    help="pick tiles_per_wave as the largest whose saved + workspace bytes fit (tiled mode)")
    ap.add_argument("--prune-width", type=int, default=0, metavar="S",
                    help="pruned lattice: a band of S label positions per frame around the diagonal (0 = full lattice)")
    ap.add_argument("--fp8", action="store_true",
                    help="bf16 workloads: the output layer's score products on OCP E4M3 operands (an approximation)")
    ap.add_argument("--graph", action="store_true",
                    help="time the headline pass as replays of one fwd+bwd captured into a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget; 0 = skip")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes three times (counter calibration)")
    ap.add_argument("--reference-gemm", action="store_true",
                    help="only time the vendor GEMM (torch.matmul) on this workload's three product shapes")
    ap.add_argument("--unfused-baseline", action="store_true",
                    help="also time an unfused batched loss over materialised [B,T,U+1,V] scores (comparator; "
                         "prints its own JSON line after checking it against this library)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library computes one GPU's share of a batch sharded by sample)", file=sys.stderr)
        sys.exit(2)

    from rnnt_inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    inp = None
    cpu = None
    side_runs = args.calibrate_copy or args.reference_gemm or args.unfused_baseline
    if not side_runs:
        print(f"# generating {w.name} inputs", file=sys.stderr, flush=True)
        inp = workload_inputs(args.workload)
        if args.cpu_seconds > 0 and args.prune_width == 0 and not args.fp8:
            # the oracle's worker processes start before this process touches the GPU
            print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
            cpu = cpu_baseline(inp, args.cpu_seconds)

    import torch

    import rnn_loss_joint_amd as rl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        # a plain copy kernel of known size: FETCH_SIZE / WRITE_SIZE of one
        # dispatch against these bytes give the counters' scale
        n = args.calibrate_copy // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 4 * n}))
        return
    if args.reference_gemm:
        reference_gemm(torch, w)
        return
    rl.load()
    tile = (w.T, w.U + 1) if args.tile == "sample" else tuple(int(x) for x in args.tile.split("x"))
    if inp is None:
        print(f"# generating {w.name} inputs", file=sys.stderr, flush=True)
        inp = workload_inputs(args.workload)
    if args.budget > 0:
        d = rl.make_desc(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, dtype=w.dtype, tile=tile)
        args.tiles_per_wave = rl.rnnt_waves_for_budget(d, inp.T_len, inp.U_len, int(args.budget))
        print(f"# budget {args.budget:.3g} B -> {args.tiles_per_wave} tiles per wave", file=sys.stderr, flush=True)
    band = None
    if args.prune_width > 0:
        from rnnt_inputs import diagonal_band

        band = (diagonal_band(inp.T_len, inp.U_len, w.T, args.prune_width), args.prune_width)
    prob = rl.Problem(inp, mode=args.mode, tile=tile, tiles_per_wave=args.tiles_per_wave, band=band, fp8=args.fp8)
    stream = torch.cuda.current_stream()

    print("# warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        prob.forward()
        prob.backward()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    graph = None
    if args.graph:
        # one fwd+bwd captured into a graph (warm-up on a side stream first)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            prob.forward()
            prob.backward()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            prob.forward()
            prob.backward()
        graph.replay()
        torch.cuda.synchronize()
        print("# captured one fwd+bwd into a graph", file=sys.stderr, flush=True)

    # timed pass 1 (the headline figure): K steps, nothing but the library's launches
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            prob.forward()
            prob.backward()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    peak = torch.cuda.max_memory_allocated()
    print(f"# timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s)", file=sys.stderr, flush=True)

    # timed pass 2 (the breakdown): the same K steps with every launch bracketed by a hipEvent
    # pair on its stream (the library's launch timing), and the forward and backward separately
    rl.rnnt_profile_start()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        prob.forward()
        e[1].record(stream)
        prob.backward()
        e[2].record(stream)
    torch.cuda.synchronize()
    prof = rl.rnnt_profile_stop()
    t_fwd = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    t_bwd = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    print(f"# profiled pass: fwd {t_fwd:.3f} + bwd {t_bwd:.3f} ms/step", file=sys.stderr, flush=True)

    cells = inp.valid_cells if band is None else band_cells(inp, band)
    cell_name = "valid_cells" if band is None else "band_cells"
    flops = mfma_flops(inp, cells)
    dtype = inp.dtype
    kernels = {}
    for name, (launches, tot) in prof.items():
        k = {"launches": launches // args.steps, "ms_per_step": tot / args.steps}
        if name in flops and tot > 0:
            k["tflops"] = flops[name] * args.steps / (tot * 1e-3) / 1e12
        if name == "lattice" and tot > 0:
            k["gbs"] = 24.0 * inp.valid_cells * args.steps / (tot * 1e-3) / 1e9  # the sweep visits every cell
        kernels[name] = k
    mfma_names = [n for n in kernels if n in flops and n in GEMM_KERNELS]
    dom = max(mfma_names, key=lambda n: kernels[n]["ms_per_step"])
    dk = kernels[dom]
    ach = dk["tflops"]
    peak_of = lambda name: PEAK_TFLOPS["fp8" if args.fp8 and name in FP8_KERNELS else dtype]
    for name, k in kernels.items():
        if "tflops" in k and name in GEMM_KERNELS:
            k["frac"] = k["tflops"] / peak_of(name)
    roof = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": peak_of(dom), "unit": "TFLOP/s",
            "frac": ach / peak_of(dom), "traffic": measured_traffic(dom, w.name),
            "per_launch": (f"{FLOP_FORMULA.get(dom, '2*H*V*valid_cells').replace('valid_cells', cell_name)} / launches = "
                           f"{flops[dom] / max(1, dk['launches']):.4g} FLOP"),
            "launch_ms": dk["ms_per_step"] / max(1, dk["launches"]),
            "timing": "mean launch duration from hipEvent pairs on the launch stream over the profiled pass"}

    d = inp.dims
    value = inp.padded_cells / (ms * 1e-3)
    # device inputs: h^A, h^L, W^A, W^L, b^Z, W^O, b^O in the mode dtype, labels int32
    esz = 2 if dtype == "bf16" else 4
    input_bytes = (esz * (d["B"] * d["T"] * d["HA"] + d["B"] * (d["U"] + 1) * d["HL"] + d["H"] * (d["HA"] + d["HL"] + 1)
                          + d["V"] * (d["H"] + 1)) + 4 * d["B"] * (d["U"] + 1))
    out = {
        "metric": "RNN-T fwd+bwd lattice cells/s (B*T*(U+1)) at V=1024; peak HBM bytes",
        "value": value,
        "unit": "cells/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16" if args.fp8 else dtype,
        "data": "synthetic",
        "peak_hbm_bytes": int(peak),
        "input_bytes": int(input_bytes),
        "peak_hbm_minus_inputs_bytes": int(peak - input_bytes),
        "valid_cells_per_s": inp.valid_cells / (ms * 1e-3),
        "t_fwd_ms": t_fwd,
        "t_bwd_ms": t_bwd,
        "ms_per_step_profiled": t_fwd + t_bwd,
        "config": {"workload": w.name, "B": d["B"], "T": d["T"], "U": d["U"],
                   "V": d["V"], "HA": d["HA"], "HL": d["HL"], "H": d["H"], "mode": args.mode,
                   "tile": list(tile), "tiles_per_wave": args.tiles_per_wave, "prune_width": args.prune_width,
                   "fp8_scores": bool(args.fp8), "graph_replay": graph is not None,
                   "padded_cells": inp.padded_cells, "valid_cells": inp.valid_cells,
                   "band_cells": None if band is None else cells,
                   "saved_bytes": prob.saved_bytes, "workspace_bytes": prob.ws_bytes},
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    if args.unfused_baseline:
        unfused_line(torch, rl, inp, prob, w.name, ms, peak, args)
        return
    print(json.dumps(out))


def unfused_line(torch, rl, inp, prob, name, ms, peak, args):
    """Time the unfused comparator after checking it against this library's results."""
    costs_f = prob.forward().clone()
    grads = prob.backward()
    torch.cuda.synchronize()
    ref = {"costs": costs_f.cpu().numpy().astype(np.float64),
           "dWO": grads["dWO"].cpu().numpy().astype(np.float64), "dhA": grads["dhA"].cpu().numpy().astype(np.float64)}
    del prob, grads, costs_f
    torch.cuda.empty_cache()
    print("# unfused comparator", file=sys.stderr, flush=True)
    ms_u, peak_u, cu, gu = unfused_baseline(torch, rl, inp, args.steps, max(1, args.warmup))
    got = {"costs": cu.cpu().numpy().astype(np.float64), "dWO": gu["dWO"].cpu().numpy().astype(np.float64),
           "dhA": gu["dhA"].cpu().numpy().astype(np.float64)}
    agree = {"costs_max_rel": float(np.max(np.abs(got["costs"] - ref["costs"]) / np.abs(ref["costs"])))}
    for k in ("dWO", "dhA"):
        agree[f"{k}_err_of_max_abs"] = float(np.max(np.abs(got[k] - ref[k])) / np.max(np.abs(ref[k])))
    ok = agree["costs_max_rel"] <= 2e-3 and agree["dWO_err_of_max_abs"] <= 2e-2 and agree["dhA_err_of_max_abs"] <= 2e-2
    print(json.dumps({"comparator": "unfused batched loss over materialised [B,T,U+1,V] scores", "workload": name,
                      "steps": args.steps, "fused": {"ms_per_step": ms, "peak_hbm_bytes": int(peak)},
                      "unfused": {"ms_per_step": ms_u, "peak_hbm_bytes": int(peak_u)},
                      "unfused_over_fused_time": ms_u / ms, "unfused_over_fused_peak": peak_u / peak,
                      "agreement": agree, "agrees": bool(ok)}))
    if not ok:
        sys.exit(3)


if __name__ == "__main__":
    main()
