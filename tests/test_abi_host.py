"""Host-only checks of the C ABI: exports, argument validation, buffer sizes.

Nothing here launches GPU work: rnnt_loss_query is pure host code, and the
fwd/bwd calls below fail validation before any launch.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import rnn_loss_joint_amd as rl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "rnnt.h")).read()
    return sorted(set(re.findall(r"^(?:rnnt_status|const char\*)\s+(rnnt_\w+)\(", src, re.M)))


def test_library_exports_every_declared_function():
    lib = rl.load()
    names = header_functions()
    assert set(names) == set(rl.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_header_is_c_and_host_calls_work_from_c(tmp_path):
    """include/rnnt.h compiles as C99 on its own; a C client (tests/host/abi_c_client.c) links to
    the library and calls the host-only entry points."""
    import subprocess

    exe = str(tmp_path / "abi_c_client")
    lib_dir = os.path.dirname(rl.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
                        os.path.join(ROOT, "tests", "host", "abi_c_client.c"), f"-L{lib_dir}", "-lrnnt_mi355",
                        f"-Wl,-rpath,{lib_dir}", "-o", exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_status_strings():
    assert rl.rnnt_status_string(0) == "ok"
    assert "workspace" in rl.rnnt_status_string(-2)


def q(B=4, T=100, U=20, V=256, HA=64, HL=64, H=64, T_len=None, U_len=None, **kw):
    d = rl.make_desc(B, T, U, V, HA, HL, H, **kw)
    T_len = np.full(B, T) if T_len is None else T_len
    U_len = np.full(B, U) if U_len is None else U_len
    return rl.rnnt_loss_query(d, T_len, U_len)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), rl.RNNT_E_INVALID),
    (dict(V=1), rl.RNNT_E_INVALID),
    (dict(blank=256), rl.RNNT_E_INVALID),
    (dict(blank=-1), rl.RNNT_E_INVALID),
    (dict(tile=(0, 32)), rl.RNNT_E_INVALID),
    (dict(tile=(64, 0)), rl.RNNT_E_INVALID),
    (dict(tiles_per_wave=-1), rl.RNNT_E_INVALID),
    (dict(H=60), rl.RNNT_E_UNSUPPORTED),
    (dict(HA=12), rl.RNNT_E_UNSUPPORTED),
    (dict(H=776), rl.RNNT_E_UNSUPPORTED),
    (dict(U=1100, U_len=np.full(4, 5)), rl.RNNT_E_UNSUPPORTED),
])
def test_query_rejects_bad_descriptors(kw, status):
    with pytest.raises(rl.RnntError) as e:
        q(**kw)
    assert e.value.status == status


@pytest.mark.parametrize("T_len,U_len", [
    ([100, 0, 5, 5], [3, 3, 3, 3]),      # T_b = 0
    ([100, 101, 5, 5], [3, 3, 3, 3]),    # T_b > T
    ([10, 10, 10, 10], [3, -1, 3, 3]),   # U_b < 0
    ([10, 10, 10, 10], [3, 21, 3, 3]),   # U_b > U
])
def test_query_rejects_bad_lengths(T_len, U_len):
    with pytest.raises(rl.RnntError) as e:
        q(T_len=np.array(T_len), U_len=np.array(U_len))
    assert e.value.status == rl.RNNT_E_INVALID


def test_bad_dtype_and_mode_and_reserved():
    d = rl.make_desc(2, 8, 2, 16, 8, 8, 8)
    for field, val in (("dtype", 7), ("mode", 3), ("reserved", 1)):
        d2 = rl.RnntDesc.from_buffer_copy(d)
        setattr(d2, field, val)
        with pytest.raises(rl.RnntError) as e:
            rl.rnnt_loss_query(d2, np.full(2, 8), np.full(2, 2))
        assert e.value.status == rl.RNNT_E_INVALID


class FakeTensor:
    """Stands in for a device tensor: the calls below fail validation before use."""

    def __init__(self, nbytes, ptr=0x1000):
        self._n, self._p = nbytes, ptr

    def data_ptr(self):
        return self._p

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_fwd_bwd_reject_small_buffers_before_launch():
    d = rl.make_desc(2, 8, 2, 16, 8, 8, 8, dtype="f32")
    T, U = np.full(2, 8), np.full(2, 2)
    s, w = rl.rnnt_loss_query(d, T, U)
    x = FakeTensor(1 << 20)
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_loss_fwd(d, x, x, x, T, U, x, x, x, x, x, x, FakeTensor(s - 1), None, stream=0)
    assert e.value.status == rl.RNNT_E_WORKSPACE
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_loss_bwd(d, x, x, x, T, U, x, x, x, x, x, None, FakeTensor(s), FakeTensor(w - 1),
                         x, x, x, x, x, x, x, stream=0)
    assert e.value.status == rl.RNNT_E_WORKSPACE
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_loss_fwd(d, None, x, x, T, U, x, x, x, x, x, x, FakeTensor(s), None, stream=0)
    assert e.value.status == rl.RNNT_E_INVALID


def test_lattice_entry_rejects_null_and_large_U():
    d = rl.make_desc(2, 8, 2, 16, 8, 8, 8)
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_lattice(d, None, None, None, None, None, None, None, stream=0)
    assert e.value.status == rl.RNNT_E_INVALID
    d = rl.make_desc(2, 8, 1500, 16, 8, 8, 8)
    x = FakeTensor(16)
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_lattice(d, x, x, x, x, x, x, x, stream=0)
    assert e.value.status == rl.RNNT_E_UNSUPPORTED
    # the lattice arrays move as 16-byte pieces: a misaligned one is rejected before any launch
    d = rl.make_desc(2, 8, 2, 16, 8, 8, 8)
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_lattice(d, x, x, x, FakeTensor(16, 4), x, x, x, stream=0)
    assert e.value.status == rl.RNNT_E_INVALID
    # (T + U) * US per sample beyond 2^29 entries
    d = rl.make_desc(1, 600000, 1000, 16, 8, 8, 8)
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_lattice(d, x, x, x, x, x, x, x, stream=0)
    assert e.value.status == rl.RNNT_E_UNSUPPORTED


def test_tile_working_set_independent_of_lattice_size():
    """At a fixed tile and tiles_per_wave, workspace minus the O(B*T*H) gradient
    accumulators does not depend on T or U (tiled mode)."""
    B, V, HA, HL, H = 32, 1024, 512, 512, 640
    seen = set()
    for T in (250, 500, 1000):
        for U in (50, 100, 200):
            d = rl.make_desc(B, T, U, V, HA, HL, H, tile=(64, 32), tiles_per_wave=64)
            _, w = rl.rnnt_loss_query(d, np.full(B, T), np.full(B, U))
            accum = 4 * H * B * (T + U + 1)
            seen.add(w - accum)
    assert len(seen) <= 2, seen  # only 256-byte alignment slack may differ
    assert max(seen) - min(seen) <= 4096


def test_tiled_working_set_scales_with_tile_not_lattice():
    B, T, U, V, HA, HL, H = 16, 400, 150, 4096, 640, 640, 640
    ws = []
    for tile in ((32, 16), (64, 32), (128, 64)):
        d = rl.make_desc(B, T, U, V, HA, HL, H, tile=tile, tiles_per_wave=B)
        ws.append(rl.rnnt_loss_query(d, np.full(B, T), np.full(B, U))[1])
    assert ws[0] < ws[1] < ws[2]
    du = rl.make_desc(B, T, U, V, HA, HL, H, mode="untiled")
    dt = rl.make_desc(B, T, U, V, HA, HL, H, tiles_per_wave=B)
    su, _ = rl.rnnt_loss_query(du, np.full(B, T), np.full(B, U))
    st, _ = rl.rnnt_loss_query(dt, np.full(B, T), np.full(B, U))
    cells = B * T * (U + 1)
    assert su - st >= cells * (V + H) * 2  # untiled keeps scores and z for every cell


# ----------------------------------------------------------------------------- wave size from a budget

def _total(d, T_len, U_len):
    s, w = rl.rnnt_loss_query(d, T_len, U_len)
    return s + w


@pytest.mark.parametrize("tile", [(64, 32), (500, 121)])
def test_waves_for_budget_is_the_largest_fit(tile):
    B, T, U, V, HA, HL, H = 32, 500, 120, 1024, 512, 512, 640
    rng = np.random.default_rng(3)
    T_len, U_len = rng.integers(300, T + 1, B), rng.integers(72, U + 1, B)
    d = rl.make_desc(B, T, U, V, HA, HL, H, tile=tile)
    lo = _total(rl.make_desc(B, T, U, V, HA, HL, H, tile=tile, tiles_per_wave=1), T_len, U_len)
    prev = 0
    for budget in (lo, int(lo * 1.3), int(lo * 2), int(lo * 4), 1 << 40):
        n = rl.rnnt_waves_for_budget(d, T_len, U_len, budget)
        assert n >= max(prev, 1)  # monotone in the budget
        prev = n
        at = rl.make_desc(B, T, U, V, HA, HL, H, tile=tile, tiles_per_wave=n)
        assert _total(at, T_len, U_len) <= budget
        above = rl.make_desc(B, T, U, V, HA, HL, H, tile=tile, tiles_per_wave=n + 1)
        n_tiles_reached = _total(above, T_len, U_len) == _total(at, T_len, U_len)
        assert n_tiles_reached or _total(above, T_len, U_len) > budget
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_waves_for_budget(d, T_len, U_len, lo - 1)
    assert e.value.status == rl.RNNT_E_WORKSPACE
    with pytest.raises(rl.RnntError) as e:
        rl.rnnt_waves_for_budget(rl.make_desc(B, T, U, V, HA, HL, H, mode="untiled"), T_len, U_len, 1 << 40)
    assert e.value.status == rl.RNNT_E_INVALID


def test_sample_wise_working_set_independent_of_batch():
    """Whole-sample tiles, a fixed number of samples per wave: saved is a fixed
    amount per sample (the lattice scalars and the a / l rows), and the
    workspace minus the gA / gL accumulators does not grow with the batch."""
    T, U, V, HA, HL, H = 500, 120, 1024, 512, 512, 640
    saved_per_sample, ws_rest = set(), []
    for B in (8, 32, 128):
        d = rl.make_desc(B, T, U, V, HA, HL, H, tile=(T, U + 1), tiles_per_wave=4)
        s, w = rl.rnnt_loss_query(d, np.full(B, T), np.full(B, U))
        saved_per_sample.add(round(s / B, -3))
        ws_rest.append(w - 4 * H * (T + U + 1) * B)
    assert len(saved_per_sample) == 1, saved_per_sample  # plan records aside
    assert ws_rest[0] <= ws_rest[1] and abs(ws_rest[2] - ws_rest[1]) <= 64 * 1024, ws_rest
