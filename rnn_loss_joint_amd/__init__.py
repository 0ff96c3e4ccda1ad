"""Python binding of librnnt_mi355.so, the gfx950 RNN-T joint + loss library.

The functions here only marshal arguments (torch device tensors and host
int32 length arrays) into the C ABI declared in include/rnnt.h and raise
RnntError on a non-OK status. Every step of the computation runs in the HIP
kernels of the shared library; there is no fallback path: if the library is
missing, load() raises.

Problem is a convenience that allocates the device buffers (inputs, saved,
workspace, outputs) with torch for one batch and calls the entry points.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librnnt_mi355.so")

RNNT_OK, RNNT_E_INVALID, RNNT_E_WORKSPACE, RNNT_E_HIP, RNNT_E_UNSUPPORTED = 0, -1, -2, -3, -4
RNNT_F32, RNNT_BF16, RNNT_BF16_FP8 = 0, 1, 2
RNNT_TILED, RNNT_UNTILED = 0, 1

_lib = None


class RnntError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"rnnt status {status}: {msg}")
        self.status = status


class RnntBand(ctypes.Structure):
    _fields_ = [("lo_host", ctypes.POINTER(ctypes.c_int32)), ("width", ctypes.c_int32)]


class RnntDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "T", "U", "V", "HA", "HL", "H", "blank", "dtype", "mode", "tile_t", "tile_u",
        "tiles_per_wave", "reserved")]


EXPORTS = ("rnnt_loss_query", "rnnt_waves_for_budget", "rnnt_loss_fwd", "rnnt_loss_fwd_noalloc", "rnnt_loss_bwd",
           "rnnt_loss_query_pruned", "rnnt_loss_fwd_pruned", "rnnt_loss_bwd_pruned",
           "rnnt_lattice", "rnnt_profile_start", "rnnt_profile_stop", "rnnt_profile_get", "rnnt_status_string",
           "rnnt_last_error")
NOALLOC_SCRATCH_BYTES = 256 << 20  # RNNT_NOALLOC_SCRATCH_BYTES


def load(path: str = LIB_PATH):
    """Load the shared library (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} not found: build it with `python -m rnn_loss_joint_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32P, SZ, SZP = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)
    DP = ctypes.POINTER(RnntDesc)
    lib.rnnt_loss_query.argtypes = [DP, I32P, I32P, SZP, SZP]
    lib.rnnt_loss_fwd.argtypes = [DP, P, P, P, I32P, I32P, P, P, P, P, P, P, P, SZ, P, SZ, P]
    lib.rnnt_loss_fwd_noalloc.argtypes = [DP, P, P, P, I32P, I32P, P, P, P, P, P, P, P, SZ, P]
    BP = ctypes.POINTER(RnntBand)
    lib.rnnt_loss_query_pruned.argtypes = [DP, I32P, I32P, BP, SZP, SZP]
    lib.rnnt_loss_fwd_pruned.argtypes = [DP, P, P, P, I32P, I32P, BP, P, P, P, P, P, P, P, SZ, P, SZ, P]
    lib.rnnt_loss_bwd_pruned.argtypes = [DP, P, P, P, I32P, I32P, BP, P, P, P, P, P, P, P, SZ, P, SZ,
                                         P, P, P, P, P, P, P, P]
    lib.rnnt_loss_bwd.argtypes = [DP, P, P, P, I32P, I32P, P, P, P, P, P, P, P, SZ, P, SZ,
                                  P, P, P, P, P, P, P, P]
    lib.rnnt_lattice.argtypes = [DP, P, P, P, P, P, P, P, P]
    lib.rnnt_waves_for_budget.argtypes = [DP, I32P, I32P, SZ, I32P]
    for f in ("rnnt_loss_query", "rnnt_waves_for_budget", "rnnt_loss_fwd", "rnnt_loss_fwd_noalloc", "rnnt_loss_bwd",
              "rnnt_loss_query_pruned", "rnnt_loss_fwd_pruned", "rnnt_loss_bwd_pruned", "rnnt_lattice"):
        getattr(lib, f).restype = ctypes.c_int
    lib.rnnt_profile_start.argtypes = []
    lib.rnnt_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.rnnt_profile_get.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_double)]
    for f in ("rnnt_profile_start", "rnnt_profile_stop", "rnnt_profile_get"):
        getattr(lib, f).restype = ctypes.c_int
    lib.rnnt_status_string.argtypes = [ctypes.c_int]
    lib.rnnt_status_string.restype = ctypes.c_char_p
    lib.rnnt_last_error.argtypes = []
    lib.rnnt_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != RNNT_OK:
        lib = load()
        raise RnntError(status, (lib.rnnt_last_error() or b"").decode())


_DTYPES = {"f32": RNNT_F32, "bf16": RNNT_BF16, "bf16-fp8": RNNT_BF16_FP8}


def make_desc(B, T, U, V, HA, HL, H, *, blank=0, dtype="bf16", mode="tiled", tile=(64, 32),
              tiles_per_wave=0) -> RnntDesc:
    """dtype: "f32", "bf16", or "bf16-fp8" (bf16 inputs, the output layer's score product on E4M3)."""
    return RnntDesc(B, T, U, V, HA, HL, H, blank, _DTYPES[dtype],
                    RNNT_UNTILED if mode == "untiled" else RNNT_TILED, tile[0], tile[1], tiles_per_wave, 0)


def _lens(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch

        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream)


def rnnt_status_string(status: int) -> str:
    return load().rnnt_status_string(status).decode()


def rnnt_last_error() -> str:
    return (load().rnnt_last_error() or b"").decode()


def rnnt_loss_query(desc: RnntDesc, T_len, U_len):
    """(saved_bytes, workspace_bytes) for this descriptor and host lengths."""
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    s, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.rnnt_loss_query(ctypes.byref(desc), tp, up, ctypes.byref(s), ctypes.byref(w)))
    return s.value, w.value


def make_band(lo, width):
    """An rnnt_band over a host int32 [B, T] array (keep the returned array alive with the struct)."""
    lo = np.ascontiguousarray(np.asarray(lo, dtype=np.int32))
    return RnntBand(lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(width)), lo


def rnnt_loss_query_pruned(desc: RnntDesc, T_len, U_len, lo, width):
    """(saved_bytes, workspace_bytes) of the pruned lattice with bands lo [B, T], width."""
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    band, keep = make_band(lo, width)
    s, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.rnnt_loss_query_pruned(ctypes.byref(desc), tp, up, ctypes.byref(band), ctypes.byref(s),
                                      ctypes.byref(w)))
    return s.value, w.value


def rnnt_loss_fwd_pruned(desc, hA, hL, labels, T_len, U_len, lo, width, WA, WL, bZ, WO, bO, costs, saved,
                         workspace=None, stream=None):
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    band, keep = make_band(lo, width)
    _check(lib.rnnt_loss_fwd_pruned(ctypes.byref(desc), _ptr(hA), _ptr(hL), _ptr(labels), tp, up, ctypes.byref(band),
                                    _ptr(WA), _ptr(WL), _ptr(bZ), _ptr(WO), _ptr(bO), _ptr(costs), _ptr(saved),
                                    saved.numel() * saved.element_size(), _ptr(workspace),
                                    0 if workspace is None else workspace.numel() * workspace.element_size(),
                                    _stream(stream)))


def rnnt_loss_bwd_pruned(desc, hA, hL, labels, T_len, U_len, lo, width, WA, WL, bZ, WO, bO, dcosts, saved,
                         workspace, dhA, dhL, dWA, dWL, dbZ, dWO, dbO, stream=None):
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    band, keep = make_band(lo, width)
    _check(lib.rnnt_loss_bwd_pruned(ctypes.byref(desc), _ptr(hA), _ptr(hL), _ptr(labels), tp, up, ctypes.byref(band),
                                    _ptr(WA), _ptr(WL), _ptr(bZ), _ptr(WO), _ptr(bO), _ptr(dcosts), _ptr(saved),
                                    saved.numel() * saved.element_size(), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _ptr(dhA), _ptr(dhL), _ptr(dWA),
                                    _ptr(dWL), _ptr(dbZ), _ptr(dWO), _ptr(dbO), _stream(stream)))


def rnnt_waves_for_budget(desc: RnntDesc, T_len, U_len, budget_bytes: int) -> int:
    """Largest tiles_per_wave whose saved + workspace bytes fit budget_bytes (tiled mode)."""
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    n = ctypes.c_int32(0)
    _check(lib.rnnt_waves_for_budget(ctypes.byref(desc), tp, up, int(budget_bytes), ctypes.byref(n)))
    return n.value


def rnnt_loss_fwd(desc, hA, hL, labels, T_len, U_len, WA, WL, bZ, WO, bO, costs, saved, workspace=None,
                  stream=None):
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    _check(lib.rnnt_loss_fwd(ctypes.byref(desc), _ptr(hA), _ptr(hL), _ptr(labels), tp, up, _ptr(WA),
                             _ptr(WL), _ptr(bZ), _ptr(WO), _ptr(bO), _ptr(costs), _ptr(saved),
                             saved.numel() * saved.element_size(), _ptr(workspace),
                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                             _stream(stream)))


def rnnt_loss_fwd_noalloc(desc, hA, hL, labels, T_len, U_len, WA, WL, bZ, WO, bO, costs, saved, stream=None):
    """rnnt_loss_fwd with the library's static scratch array as its workspace (no allocation)."""
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    _check(lib.rnnt_loss_fwd_noalloc(ctypes.byref(desc), _ptr(hA), _ptr(hL), _ptr(labels), tp, up, _ptr(WA),
                                     _ptr(WL), _ptr(bZ), _ptr(WO), _ptr(bO), _ptr(costs), _ptr(saved),
                                     saved.numel() * saved.element_size(), _stream(stream)))


def rnnt_loss_bwd(desc, hA, hL, labels, T_len, U_len, WA, WL, bZ, WO, bO, dcosts, saved, workspace,
                  dhA, dhL, dWA, dWL, dbZ, dWO, dbO, stream=None):
    lib = load()
    T_len, tp = _lens(T_len)
    U_len, up = _lens(U_len)
    _check(lib.rnnt_loss_bwd(ctypes.byref(desc), _ptr(hA), _ptr(hL), _ptr(labels), tp, up, _ptr(WA),
                             _ptr(WL), _ptr(bZ), _ptr(WO), _ptr(bO), _ptr(dcosts), _ptr(saved),
                             saved.numel() * saved.element_size(), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _ptr(dhA), _ptr(dhL),
                             _ptr(dWA), _ptr(dWL), _ptr(dbZ), _ptr(dWO), _ptr(dbO), _stream(stream)))


def rnnt_lattice(desc, T_len_dev, U_len_dev, phi, psi, alpha, beta, costs, stream=None):
    lib = load()
    _check(lib.rnnt_lattice(ctypes.byref(desc), _ptr(T_len_dev), _ptr(U_len_dev), _ptr(phi), _ptr(psi),
                            _ptr(alpha), _ptr(beta), _ptr(costs), _stream(stream)))


def rnnt_profile_start():
    _check(load().rnnt_profile_start())


def rnnt_profile_stop():
    """Stop launch timing; returns {kernel name: (launches, total_ms)}."""
    lib = load()
    n = ctypes.c_int32(0)
    _check(lib.rnnt_profile_stop(ctypes.byref(n)))
    out = {}
    for i in range(n.value):
        name, cnt, ms = ctypes.c_char_p(), ctypes.c_int32(), ctypes.c_double()
        _check(lib.rnnt_profile_get(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)))
        out[name.value.decode()] = (cnt.value, ms.value)
    return out


class Problem:
    """Device buffers for one batch and the calls that fill them.

    inputs: any object with dtype, blank, T_len, U_len, labels, hA, hL, WA, WL,
    bZ, WO, bO (numpy, float values exact in the dtype), e.g. rnnt_inputs.Inputs.
    """

    def __init__(self, inputs, *, mode="tiled", tile=(64, 32), tiles_per_wave=0, device="cuda:0", band=None,
                 fp8=False):
        """fp8: bf16 inputs with the output layer's score product on E4M3 operands (RNNT_BF16_FP8)."""
        import torch

        self.torch = torch
        self.inputs = inputs
        tdt = torch.bfloat16 if inputs.dtype == "bf16" else torch.float32
        B, T, HA = inputs.hA.shape
        U = inputs.hL.shape[1] - 1
        HL = inputs.hL.shape[2]
        V, H = inputs.WO.shape
        if fp8 and inputs.dtype != "bf16":
            raise ValueError("the fp8 output layer takes bf16 inputs")
        self.desc = make_desc(B, T, U, V, HA, HL, H, blank=int(inputs.blank),
                              dtype="bf16-fp8" if fp8 else inputs.dtype, mode=mode, tile=tile,
                              tiles_per_wave=tiles_per_wave)
        self.T_len = np.ascontiguousarray(inputs.T_len, dtype=np.int32)
        self.U_len = np.ascontiguousarray(inputs.U_len, dtype=np.int32)
        dev = torch.device(device)
        self.device = dev
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(tdt)
        self.hA, self.hL = up(inputs.hA), up(inputs.hL)
        self.WA, self.WL, self.bZ = up(inputs.WA), up(inputs.WL), up(inputs.bZ)
        self.WO, self.bO = up(inputs.WO), up(inputs.bO)
        self.labels = torch.from_numpy(np.ascontiguousarray(inputs.labels, dtype=np.int32)).to(dev)
        # band: None, or (lo [B, T], width) for the pruned lattice
        self.band = None if band is None else (np.ascontiguousarray(band[0], dtype=np.int32), int(band[1]))
        if self.band is None:
            self.saved_bytes, self.ws_bytes = rnnt_loss_query(self.desc, self.T_len, self.U_len)
        else:
            self.saved_bytes, self.ws_bytes = rnnt_loss_query_pruned(self.desc, self.T_len, self.U_len, *self.band)
        self.saved = torch.empty(max(self.saved_bytes, 1), dtype=torch.uint8, device=dev)
        self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.costs = torch.empty(B, dtype=torch.float32, device=dev)
        f = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)
        self.grads = dict(dhA=f(B, T, HA), dhL=f(B, U + 1, HL), dWA=f(H, HA), dWL=f(H, HL), dbZ=f(H),
                          dWO=f(V, H), dbO=f(V))

    def forward(self, stream=None):
        if self.band is None:
            rnnt_loss_fwd(self.desc, self.hA, self.hL, self.labels, self.T_len, self.U_len, self.WA, self.WL,
                          self.bZ, self.WO, self.bO, self.costs, self.saved, self.workspace, stream)
        else:
            rnnt_loss_fwd_pruned(self.desc, self.hA, self.hL, self.labels, self.T_len, self.U_len, *self.band, self.WA,
                                 self.WL, self.bZ, self.WO, self.bO, self.costs, self.saved, self.workspace, stream)
        return self.costs

    def backward(self, dcosts=None, stream=None):
        g = self.grads
        if self.band is None:
            rnnt_loss_bwd(self.desc, self.hA, self.hL, self.labels, self.T_len, self.U_len, self.WA, self.WL,
                          self.bZ, self.WO, self.bO, dcosts, self.saved, self.workspace, g["dhA"], g["dhL"],
                          g["dWA"], g["dWL"], g["dbZ"], g["dWO"], g["dbO"], stream)
        else:
            rnnt_loss_bwd_pruned(self.desc, self.hA, self.hL, self.labels, self.T_len, self.U_len, *self.band,
                                 self.WA, self.WL, self.bZ, self.WO, self.bO, dcosts, self.saved, self.workspace,
                                 g["dhA"], g["dhL"], g["dWA"], g["dWL"], g["dbZ"], g["dWO"], g["dbO"], stream)
        return g
