"""Host replay of the persistent score kernels' item and address mapping (no launch).

tests/host/replay_scores3.cpp is built with g++ against the library's own plan code and
the constexpr mapping the kernel compiles (rnn_loss_joint_amd/csrc/scores3_map.hpp). For
every wave of every plan below, every workgroup, stage and item of the forward and backward
launches, it checks that the cell tile and V tile indices are in range and that every dma
source and epilogue store byte range lies inside the buffer region the layout reserves.
Covered: the four bf16 workloads at their lengths with the tile sizes they are run with and
more, default, single-tile, small and whole-batch waves, whole-sample tiles, ragged or
degenerate length sets, untiled mode (the forward's z rows and stored scores in `saved`),
the fp8 output layer and pruned lattices.
"""
import os
import subprocess

import numpy as np
import pytest

import rnn_loss_joint_amd as rl
from rnnt_inputs import WORKLOADS, diagonal_band, workload_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rnn_loss_joint_amd", "csrc")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def replay(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("replay") / "replay_scores3")
    # AddressSanitizer and UBSan on the host code (the library's plan.cpp included)
    cmd = ["g++", "-O2", "-std=c++17", *SANITIZE, f"-I{CSRC}", os.path.join(ROOT, "tests", "host", "replay_scores3.cpp"),
           os.path.join(CSRC, "plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return exe


def case_line(B, T, U, V, HA, HL, H, tile, tpw, T_len, U_len, bf16=True, untiled=False, band=None, fp8=False):
    vals = [B, T, U, V, HA, HL, H, 2 if fp8 else int(bf16), int(untiled), tile[0], tile[1], tpw]
    vals += list(map(int, T_len)) + list(map(int, U_len))
    if band is not None:
        vals += [int(band[1])] + list(map(int, np.asarray(band[0]).reshape(-1)))
    return " ".join(map(str, vals))


def run(exe, lines):
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=600)
    out = r.stdout.strip().splitlines()
    assert len(out) == len(lines), r.stdout + r.stderr
    return r.returncode, out


@pytest.mark.parametrize("name", ["small-bf16", "20s-bf16", "vocab4096-bf16", "40s-b256-bf16"])
def test_workload_plans_stay_in_bounds(replay, name):
    w = WORKLOADS[name]
    T_len, U_len = workload_lengths(name)
    tiles = sorted(set(w.tiles) | {(64, 32), (32, 16), (128, 64), (32, 8), (96, 40), (w.T, w.U + 1)})
    lines = []
    for tile in tiles:
        for tpw in (0, 1, 3, w.B, 4 * w.B):
            lines.append(case_line(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, tile, tpw, T_len, U_len))
    rc, out = run(replay, lines)
    bad = [(l.split()[:12], o) for l, o in zip(lines, out) if not o.startswith("ok")]
    assert rc == 0 and not bad, bad[:3]


def test_ragged_and_degenerate_plans_stay_in_bounds(replay):
    rng = np.random.default_rng(7)
    lines = []
    for _ in range(40):
        B = int(rng.integers(1, 40))
        T = int(rng.integers(1, 700))
        U = int(rng.integers(0, 300))
        V = int(rng.choice([300, 1000, 1024, 1025, 4096, 5000]))
        H = int(rng.choice([512, 576, 640, 768]))
        T_len = rng.integers(1, T + 1, B)
        U_len = rng.integers(0, U + 1, B)
        tile = (int(rng.integers(1, 200)), int(rng.integers(1, 80)))
        tpw = int(rng.choice([0, 1, 2, 7, B]))
        lines.append(case_line(B, T, U, V, 64, 64, H, tile, tpw, T_len, U_len))
    # every sample of length 1 x 1, one sample, a single full tile
    lines.append(case_line(5, 9, 4, 1024, 64, 64, 640, (32, 2), 1, [1] * 5, [0] * 5))
    lines.append(case_line(1, 1000, 200, 1024, 512, 512, 640, (64, 32), 0, [1000], [200]))
    lines.append(case_line(3, 64, 31, 256, 64, 64, 512, (64, 32), 0, [64] * 3, [31] * 3))
    rc, out = run(replay, lines)
    bad = [(l.split()[:12], o) for l, o in zip(lines, out) if o.startswith("FAIL")]
    assert rc == 0 and not bad, bad[:3]
    assert sum(o.startswith("ok") for o in out) >= 30


def test_untiled_plans_stay_in_bounds(replay):
    """Untiled bf16 mode runs the forward score kernel with a store of the scores: one wave
    of every row, its z rows read from `saved` (the last cell tile reads into the padding
    rows kept there) and the scores of the wave's rows stored into `saved`."""
    lines = []
    for name in ("small-bf16", "20s-bf16", "vocab4096-bf16"):
        w = WORKLOADS[name]
        T_len, U_len = workload_lengths(name)
        for tile in ((64, 32), (32, 16), (w.T, w.U + 1)):
            lines.append(case_line(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, tile, 0, T_len, U_len, untiled=True))
    rng = np.random.default_rng(13)
    for _ in range(20):
        B, T, U = int(rng.integers(1, 20)), int(rng.integers(1, 300)), int(rng.integers(0, 120))
        H = int(rng.choice([512, 576, 640, 768]))
        V = int(rng.choice([300, 1000, 1024, 4096]))
        tile = (int(rng.integers(1, 100)), int(rng.integers(1, 40)))
        lines.append(case_line(B, T, U, V, 64, 64, H, tile, 0, rng.integers(1, T + 1, B), rng.integers(0, U + 1, B),
                               untiled=True))
    rc, out = run(replay, lines)
    bad = [(l.split()[:12], o) for l, o in zip(lines, out) if not o.startswith("ok")]
    assert rc == 0 and not bad, bad[:3]


def test_fp8_plans_stay_in_bounds(replay):
    """The fp8 output layer's score kernels read E4M3 rows of H8 bytes (H_pad rounded up to
    128, at least 640) with three bias buffers: the bf16 workloads' plans and small hidden
    sizes (rows padded to 640) at several tiles and wave sizes."""
    lines = []
    for name in ("small-bf16", "20s-bf16", "vocab4096-bf16", "40s-b256-bf16"):
        w = WORKLOADS[name]
        T_len, U_len = workload_lengths(name)
        for tile in sorted(set(w.tiles) | {(64, 32), (32, 8)}):
            for tpw in (0, 1, 3):
                lines.append(case_line(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, tile, tpw, T_len, U_len, fp8=True))
    rng = np.random.default_rng(11)
    for _ in range(20):
        B, T, U = int(rng.integers(1, 20)), int(rng.integers(1, 300)), int(rng.integers(0, 120))
        H = int(rng.choice([64, 128, 256, 512, 640, 768]))
        V = int(rng.choice([300, 1000, 1024, 4096]))
        tile = (int(rng.integers(1, 100)), int(rng.integers(1, 40)))
        lines.append(case_line(B, T, U, V, 64, 64, H, tile, int(rng.choice([0, 1, 5])), rng.integers(1, T + 1, B),
                               rng.integers(0, U + 1, B), fp8=True))
    rc, out = run(replay, lines)
    bad = [(l.split()[:12], o) for l, o in zip(lines, out) if not o.startswith("ok")]
    assert rc == 0 and not bad, bad[:3]


def test_fp8_is_tiled_only():
    d = rl.make_desc(2, 8, 2, 64, 64, 64, 64, dtype="bf16-fp8", mode="untiled")
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_loss_query(d, np.full(2, 8), np.full(2, 2))
    assert e.value.status == rl.RNNT_E_UNSUPPORTED
    d = rl.make_desc(2, 8, 2, 64, 64, 64, 64, dtype="bf16-fp8")
    s, w = rl.rnnt_loss_query(d, np.full(2, 8), np.full(2, 2))
    d16 = rl.make_desc(2, 8, 2, 64, 64, 64, 64, dtype="bf16")
    s16, w16 = rl.rnnt_loss_query(d16, np.full(2, 8), np.full(2, 2))
    assert s == s16 and w > w16  # same saved state; the E4M3 operand rows in the workspace


def test_plan_rows_beyond_32_bits_are_refused():
    """A tiny tile_t pads every tile's t extent to 32 rows: 400 samples x 1000 frames with
    1 x 201 tiles need ~2.6e9 rows, which the 32-bit row numbers cannot address. The query
    refuses it (host only, nothing launched)."""
    B, T, U = 400, 1000, 200
    d = rl.make_desc(B, T, U, 1024, 512, 512, 640, tile=(1, 201))
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_loss_query(d, np.full(B, T), np.full(B, U))
    assert e.value.status == rl.RNNT_E_UNSUPPORTED
    assert "rows" in str(e.value)
    # the same batch with 32-row tiles fits
    d = rl.make_desc(B, T, U, 1024, 512, 512, 640, tile=(32, 201))
    s, w = rl.rnnt_loss_query(d, np.full(B, T), np.full(B, U))
    assert s > 0 and w > 0


@pytest.mark.parametrize("S", [8, 32, 64])
def test_pruned_plans_stay_in_bounds_and_skip_tiles(replay, S):
    """Pruned lattices at the 40 s x 256 lengths (bands around the diagonal): every wave's
    mapping stays in bounds, and the plan keeps fewer tiles than the full lattice's."""
    name = "40s-b256-bf16"
    w = WORKLOADS[name]
    T_len, U_len = workload_lengths(name)
    lo = diagonal_band(T_len, U_len, w.T, S)
    lines = [case_line(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, (64, 32), 0, T_len, U_len),
             case_line(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, (64, 32), 0, T_len, U_len, band=(lo, S)),
             case_line(w.B, w.T, w.U, w.V, w.HA, w.HL, w.H, (32, 16), 0, T_len, U_len, band=(lo, S))]
    rc, out = run(replay, lines)
    assert rc == 0 and all(o.startswith("ok") for o in out), out
    full, pruned = int(out[0].split()[-1]), int(out[1].split()[-1])
    assert pruned < full
    # a band of S label positions per frame keeps about S / (U_b + 1) of the cells; 64 x 32 tiles
    # straddle the band, so at most S/32 + 2 of a sample's ~7 tile columns survive per tile row
    assert pruned <= full * min(1.0, (S / 32 + 2) / 5)


def test_pruned_band_validation():
    B, T, U = 3, 20, 6
    T_len, U_len = np.array([20, 12, 5]), np.array([6, 3, 0])
    d = rl.make_desc(B, T, U, 64, 64, 64, 128)
    lo = diagonal_band(T_len, U_len, T, 3)
    s_ok, w_ok = rl.rnnt_loss_query_pruned(d, T_len, U_len, lo, 3)
    assert s_ok > 0 and w_ok > 0
    bad = []
    x = lo.copy(); x[0, 0] = 1; bad.append((x, 3))                   # first frame must start at 0
    x = lo.copy(); x[0, 5] = x[0, 4] - 1 if x[0, 4] > 0 else -1; bad.append((x, 3))  # decreasing / negative
    x = lo.copy(); x[0, 16:] = 6; bad.append((x, 3))                 # a step of 3 > width - 1
    bad.append((lo, 0))                                              # width 0
    x = lo.copy(); x[1, :] = 0; bad.append((x, 3))                   # the last frame's band misses U_b
    for lo_bad, S in bad:
        with pytest.raises(rl.RnntError) as e:
            rl.rnnt_loss_query_pruned(d, T_len, U_len, lo_bad, S)
        assert e.value.status == rl.RNNT_E_INVALID
    # frames past T_b are not read
    x = lo.copy(); x[2, 5:] = -7
    assert rl.rnnt_loss_query_pruned(d, T_len, U_len, x, 3) == (s_ok, w_ok)
