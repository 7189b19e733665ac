"""Python binding of the gfx950 gated diagonal linear-recurrence scans.

A thin ctypes layer over ``libssd.so`` (the C ABI declared in ``include/ssd.h``).
It only marshals arguments: checks tensor placement, dtype, shape and contiguity,
allocates outputs (and the scans' workspaces) with torch, and passes raw device
pointers plus torch's current HIP stream.  Every step of every scan runs in the
HIP kernels.  There is no CPU or eager fallback: importing works without a GPU,
but each call raises if the library is not built or no GPU is present.

Entry points (same names as the C ABI without the ``ssd_`` prefix):
    rglru_scan, rglru_scan_noalloc, rglru_scan_backward, rglru_update,
    minmax_scan, minmax_scan_backward, minmax_update,
    causal_conv1d, causal_conv1d_update,
    selective_scan, selective_scan_backward, selective_update,
    hgrn2_scan, hgrn2_scan_backward, hgrn2_update (gate_axis="value" or "key"), readout_norm,
    workspace_check, testing_lookback

Workspaces: the scans that pass partial results between workgroups take a caller-owned device
workspace (``ssd_*_workspace_bytes`` gives its size).  By default this module keeps one zero-filled
workspace per (device, stream, entry point), allocated through torch and grown on demand; a call may
instead pass its own zero-filled uint8 tensor as ``workspace=`` (used by that entry point only).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSD_LIBRARY names another build of the same library (for instance one whose host code carries a
# sanitizer); by default the in-tree libssd.so.
LIB_PATH = os.environ.get("SSD_LIBRARY") or os.path.join(_PKG, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE", 4: "SSD_ERR_ALIGN",
                5: "SSD_ERR_VALUE", 6: "SSD_ERR_ALIAS", 7: "SSD_ERR_HIP", 8: "SSD_ERR_TIMEOUT"}
SSD_ERR_HIP, SSD_ERR_TIMEOUT = 7, 8

# Every symbol include/ssd.h declares.
SCAN_CHUNK = 64  # SSD_SCAN_CHUNK of ssd.h

EXPORTS = ("ssd_status_str", "ssd_last_error", "ssd_version", "ssd_testing_lookback", "ssd_workspace_check",
           "ssd_rglru_scan", "ssd_rglru_scan_backward",
           "ssd_rglru_update",
           "ssd_selective_scan", "ssd_selective_update", "ssd_hgrn2_scan", "ssd_hgrn2_update", "ssd_minmax_scan",
           "ssd_minmax_update", "ssd_minmax_scan_backward", "ssd_causal_conv1d", "ssd_causal_conv1d_update",
           "ssd_selective_scan_backward", "ssd_hgrn2_scan_backward", "ssd_hgrn2_key_scan", "ssd_hgrn2_key_update",
           "ssd_readout_norm", "ssd_rglru_scan_workspace_bytes", "ssd_rglru_scan_backward_workspace_bytes",
           "ssd_minmax_scan_workspace_bytes", "ssd_minmax_scan_backward_workspace_bytes",
           "ssd_selective_scan_workspace_bytes", "ssd_selective_scan_backward_workspace_bytes",
           "ssd_hgrn2_scan_backward_workspace_bytes", "ssd_rglru_scan_noalloc")


class SSDError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {detail}")


class SSDValueError(SSDError, ValueError):
    pass


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_fp = ctypes.c_void_p
_sz = ctypes.c_size_t
_szp = ctypes.POINTER(ctypes.c_size_t)


def lib() -> ctypes.CDLL:
    """Load ``libssd.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m selective_state_space_diag_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.ssd_status_str.restype = ctypes.c_char_p
        L.ssd_status_str.argtypes = [ctypes.c_int]
        L.ssd_last_error.restype = ctypes.c_char_p
        L.ssd_last_error.argtypes = []
        L.ssd_version.restype = ctypes.c_int
        L.ssd_testing_lookback.argtypes = [ctypes.c_uint, ctypes.c_int]
        L.ssd_testing_lookback.restype = None
        L.ssd_workspace_check.argtypes = [_vp, _vp]
        L.ssd_rglru_scan.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _fp, ctypes.c_float,
                                     _fp, _vp, _vp, _fp, _fp, _vp, _sz, _vp]
        L.ssd_rglru_scan_noalloc.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _fp,
                                             ctypes.c_float, _fp, _vp, _vp, _fp, _fp, _vp]
        L.ssd_rglru_update.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _fp, ctypes.c_float, _vp,
                                       _fp, _vp, _vp]
        L.ssd_rglru_scan_backward.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _fp,
                                              ctypes.c_float, _fp, _vp, _fp, _vp, _fp, _vp, _vp, _vp, _fp, _fp, _vp,
                                              _vp, _sz, _vp]
        L.ssd_minmax_scan.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _fp, _vp, _vp, _fp, _fp,
                                      _vp, _sz, _vp]
        L.ssd_minmax_update.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _fp, _vp, _vp]
        L.ssd_minmax_scan_backward.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _fp, _vp, _fp,
                                               _vp, _fp, _vp, _vp, _fp, _vp, _vp, _sz, _vp]
        L.ssd_causal_conv1d.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _fp, _fp, _fp, _vp,
                                        _fp, _vp]
        L.ssd_causal_conv1d_update.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _fp, _fp, _fp, _vp,
                                               _vp]
        L.ssd_selective_scan.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _fp, _vp, _vp,
                                         _fp, _vp, _fp, ctypes.c_int, _vp, _i64, _fp, _vp, _fp, _vp, _sz, _vp]
        L.ssd_selective_scan_backward.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _fp,
                                                  _vp, _vp, _fp, _vp, _fp, ctypes.c_int, _vp, _i64, _fp, _vp, _fp,
                                                  _vp, _vp, _fp, _vp, _vp, _fp, _vp, _fp, _fp, _vp, _sz, _vp]
        L.ssd_selective_update.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _fp, _vp, _vp, _fp,
                                           _vp, _fp, ctypes.c_int, _fp, _vp, _vp]
        L.ssd_hgrn2_scan.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                     ctypes.c_float, _fp, _vp, _fp, _vp]
        L.ssd_hgrn2_update.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                       ctypes.c_float, _fp, _vp, _vp]
        L.ssd_hgrn2_key_scan.argtypes = L.ssd_hgrn2_scan.argtypes
        L.ssd_hgrn2_key_update.argtypes = L.ssd_hgrn2_update.argtypes
        L.ssd_readout_norm.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, _fp, _vp, _fp, _fp, ctypes.c_float, _vp,
                                       _vp]
        L.ssd_hgrn2_scan_backward.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp,
                                              ctypes.c_float, _fp, _fp, _vp, _fp, _vp, _vp, _vp, _vp, _fp, _vp, _sz,
                                              _vp]
        for q in ("rglru_scan", "rglru_scan_backward", "minmax_scan", "minmax_scan_backward"):
            getattr(L, f"ssd_{q}_workspace_bytes").argtypes = [_i64, _i64, _i64, _szp]
        L.ssd_selective_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _szp]
        L.ssd_selective_scan_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int, _szp]
        L.ssd_hgrn2_scan_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _szp]
        for name in EXPORTS[4:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _raise(status: int, fn: str):
    if status == 0:
        return
    detail = lib().ssd_last_error().decode(errors="replace")
    if status == 7:
        raise SSDError(status, fn, detail)
    raise SSDValueError(status, fn, detail)


# ----------------------------------------------------------------------------- torch marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: activations must be float32 or bfloat16")


def _out_code(out_dtype) -> int:
    torch = _torch()
    if out_dtype in (None, torch.float32):
        return SSD_F32
    if out_dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")


def _dev(t, name, shape=None, dtype=None):
    """Check a device tensor argument and return its data pointer (None for None)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ----------------------------------------------------------------------------- workspaces
# One zero-filled workspace per (device, stream, entry point), grown on demand.  torch allocates it on
# the current stream, so the zero fill is ordered before the call that first uses it; a replaced
# (smaller) one is freed to torch's caching allocator, which hands its memory only to later work on
# the same stream.
_workspaces = {}


def _workspace(entry: str, nbytes: int, device, workspace=None):
    """(pointer, size) of the workspace for one call of ``entry`` needing ``nbytes``."""
    if getattr(device, "type", None) != "cuda":
        raise ValueError("the inputs must be on the GPU")
    if nbytes == 0:
        return None, 0
    torch = _torch()
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on the GPU")
        return workspace.data_ptr(), workspace.numel()
    stream = torch.cuda.current_stream(device)
    key = (stream.device_index, stream.cuda_stream, entry)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 1 << 20)
        size = (size + 4095) // 4096 * 4096
        ws = torch.zeros(size, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws.data_ptr(), ws.numel()


def _ws_bytes(query: str, *args) -> int:
    n = ctypes.c_size_t(0)
    _raise(getattr(lib(), f"ssd_{query}_workspace_bytes")(*args, ctypes.byref(n)), f"{query}_workspace_bytes")
    return int(n.value)


def workspace_check(device=None):
    """Check every workspace this module keeps for ``device``'s current stream (waiting for the stream):
    raises SSDError with status SSD_ERR_TIMEOUT if a launch had a bounded wait between workgroups expire
    since the last check (the outputs that depended on it hold NaN)."""
    torch = _torch()
    stream = torch.cuda.current_stream(device)
    for (dev, sptr, entry), ws in list(_workspaces.items()):
        if dev == stream.device_index and sptr == stream.cuda_stream:
            _raise(lib().ssd_workspace_check(ws.data_ptr(), ctypes.c_void_p(sptr)), f"workspace_check({entry})")


def testing_lookback(spin_limit: int = 0, never_ready: bool = False):
    """Test hook of the timeout path (``ssd_testing_lookback``): later launches give up their bounded waits
    after ``spin_limit`` polls (0 = default), and with ``never_ready`` every wait expires."""
    lib().ssd_testing_lookback(int(spin_limit), int(bool(never_ready)))


def _act(ts, names):
    """All activation tensors share one dtype; returns its code."""
    code = None
    for t, n in zip(ts, names):
        if t is None:
            continue
        c = _dtype_code(t)
        if code is None:
            code = c
        elif c != code:
            raise TypeError(f"{n} has dtype {t.dtype}; all activations must share one dtype")
    return code


# ----------------------------------------------------------------------------- RG-LRU
def chunk_states_shape(B: int, L: int, D: int):
    """Shape of the ``chunk_states`` buffer of the state-size-1 scans: the state entering each chunk
    of SCAN_CHUNK steps."""
    return (B, (L + SCAN_CHUNK - 1) // SCAN_CHUNK, D)


def rglru_scan(x, r_logit, i_logit, a_log, c: float = 8.0, h0=None, return_last_state: bool = False,
               out_dtype=None, gate=None, chunk_states=None, workspace=None):
    """RG-LRU scan over [B, L, D] (see ``ssd_rglru_scan``); with ``gate``, y = gelu(gate) * h.
    ``chunk_states`` (fp32, ``chunk_states_shape``) receives the state entering each chunk, for
    ``rglru_scan_backward``.  Returns y, or (y, h_last)."""
    torch = _torch()
    B, L, D = x.shape
    code = _act([x, r_logit, i_logit, gate], ["x", "r_logit", "i_logit", "gate"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, L, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    h_last = torch.empty((B, D), device=x.device, dtype=torch.float32) if return_last_state else None
    wp, wn = _workspace("rglru_scan", _ws_bytes("rglru_scan", B, L, D), x.device, workspace)
    st = lib().ssd_rglru_scan(B, L, D, code, oc, _dev(x, "x"), _dev(r_logit, "r_logit", x.shape),
                              _dev(i_logit, "i_logit", x.shape), _dev(a_log, "a_log", (D,), torch.float32),
                              float(c), _dev(h0, "h0", (B, D), torch.float32), _dev(gate, "gate", x.shape),
                              _dev(y, "y"), _dev(h_last, "h_last"),
                              _dev(chunk_states, "chunk_states", chunk_states_shape(B, L, D), torch.float32),
                              wp, wn, _stream(x.device))
    _raise(st, "rglru_scan")
    return (y, h_last) if return_last_state else y


NOALLOC_SCRATCH_BYTES = 64 << 20  # SSD_NOALLOC_SCRATCH_BYTES of ssd.h


def rglru_scan_noalloc(x, r_logit, i_logit, a_log, c: float = 8.0, h0=None, return_last_state: bool = False,
                       out_dtype=None, gate=None, chunk_states=None, y=None, h_last=None):
    """``rglru_scan`` through ``ssd_rglru_scan_noalloc``: no workspace, the library's fixed per-GPU scratch
    (for callers that cannot allocate; calls that overlap on one GPU race).  ``y`` / ``h_last`` may be
    given preallocated.  Returns y, or (y, h_last)."""
    torch = _torch()
    B, L, D = x.shape
    code = _act([x, r_logit, i_logit, gate], ["x", "r_logit", "i_logit", "gate"])
    oc = _out_code(out_dtype)
    if y is None:
        y = torch.empty((B, L, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    if return_last_state and h_last is None:
        h_last = torch.empty((B, D), device=x.device, dtype=torch.float32)
    st = lib().ssd_rglru_scan_noalloc(B, L, D, code, oc, _dev(x, "x"), _dev(r_logit, "r_logit", x.shape),
                                      _dev(i_logit, "i_logit", x.shape), _dev(a_log, "a_log", (D,), torch.float32),
                                      float(c), _dev(h0, "h0", (B, D), torch.float32), _dev(gate, "gate", x.shape),
                                      _dev(y, "y", (B, L, D)), _dev(h_last, "h_last", (B, D), torch.float32),
                                      _dev(chunk_states, "chunk_states", chunk_states_shape(B, L, D), torch.float32),
                                      _stream(x.device))
    _raise(st, "rglru_scan_noalloc")
    return (y, h_last) if return_last_state else y


def rglru_update(x, r_logit, i_logit, a_log, c: float, state, out_dtype=None, gate=None):
    """One decode step; ``state`` [B, D] fp32 is updated in place.  Returns y [B, D]
    (gelu(gate) * h with a gate)."""
    torch = _torch()
    B, D = x.shape
    code = _act([x, r_logit, i_logit, gate], ["x", "r_logit", "i_logit", "gate"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    st = lib().ssd_rglru_update(B, D, code, oc, _dev(x, "x"), _dev(r_logit, "r_logit", x.shape),
                                _dev(i_logit, "i_logit", x.shape), _dev(a_log, "a_log", (D,), torch.float32),
                                float(c), _dev(gate, "gate", x.shape), _dev(state, "state", (B, D), torch.float32),
                                _dev(y, "y"), _stream(x.device))
    _raise(st, "rglru_update")
    return y


def rglru_scan_backward(x, r_logit, i_logit, a_log, c, dy, h0=None, gate=None, dh_last=None, out_dtype=None,
                        chunk_states=None, workspace=None):
    """Gradients of ``rglru_scan`` for the loss sum(dy * y) + sum(dh_last * h_last) (see
    ``ssd_rglru_scan_backward``); ``chunk_states`` from the forward call saves recomputing them.
    Returns a dict: dx, dr_logit, di_logit [B, L, D] (out dtype), da_log [D], dh0 [B, D] (fp32), and
    dgate when a gate is given."""
    torch = _torch()
    B, L, D = x.shape
    code = _act([x, r_logit, i_logit, gate, dy], ["x", "r_logit", "i_logit", "gate", "dy"])
    oc = _out_code(out_dtype)
    odt = torch.bfloat16 if oc == SSD_BF16 else torch.float32
    g = {n: torch.empty((B, L, D), device=x.device, dtype=odt) for n in ("dx", "dr_logit", "di_logit")}
    if gate is not None:
        g["dgate"] = torch.empty((B, L, D), device=x.device, dtype=odt)
    g["da_log"] = torch.empty((D,), device=x.device, dtype=torch.float32)
    g["dh0"] = torch.empty((B, D), device=x.device, dtype=torch.float32)
    wp, wn = _workspace("rglru_scan_backward", _ws_bytes("rglru_scan_backward", B, L, D), x.device, workspace)
    st = lib().ssd_rglru_scan_backward(
        B, L, D, code, oc, _dev(x, "x"), _dev(r_logit, "r_logit", x.shape), _dev(i_logit, "i_logit", x.shape),
        _dev(a_log, "a_log", (D,), torch.float32), float(c), _dev(h0, "h0", (B, D), torch.float32),
        _dev(gate, "gate", x.shape), _dev(chunk_states, "chunk_states", chunk_states_shape(B, L, D), torch.float32),
        _dev(dy, "dy", x.shape), _dev(dh_last, "dh_last", (B, D), torch.float32),
        _dev(g["dx"], "dx"), _dev(g["dr_logit"], "dr_logit"), _dev(g["di_logit"], "di_logit"),
        _dev(g["da_log"], "da_log"), _dev(g["dh0"], "dh0"), _dev(g.get("dgate"), "dgate"), wp, wn,
        _stream(x.device))
    _raise(st, "rglru_scan_backward")
    return g


# ----------------------------------------------------------------------------- MinMax
def minmax_scan(r, s, x0=None, gate=None, return_last_state: bool = False, out_dtype=None, chunk_states=None,
                workspace=None):
    """MinMax scan x_t = max(min(r_t, x_{t-1}), s_t) over [B, L, D] (see ``ssd_minmax_scan``);
    with ``gate``, y = x * gate; ``chunk_states`` as for ``rglru_scan``.  Returns y, or (y, x_last)."""
    torch = _torch()
    B, L, D = r.shape
    code = _act([r, s, gate], ["r", "s", "gate"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, L, D), device=r.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    x_last = torch.empty((B, D), device=r.device, dtype=torch.float32) if return_last_state else None
    wp, wn = _workspace("minmax_scan", _ws_bytes("minmax_scan", B, L, D), r.device, workspace)
    st = lib().ssd_minmax_scan(B, L, D, code, oc, _dev(r, "r"), _dev(s, "s", r.shape),
                               _dev(x0, "x0", (B, D), torch.float32), _dev(gate, "gate", r.shape), _dev(y, "y"),
                               _dev(x_last, "x_last"),
                               _dev(chunk_states, "chunk_states", chunk_states_shape(B, L, D), torch.float32),
                               wp, wn, _stream(r.device))
    _raise(st, "minmax_scan")
    return (y, x_last) if return_last_state else y


def minmax_update(r, s, state, gate=None, out_dtype=None):
    """One MinMax decode step; ``state`` [B, D] fp32 is updated in place.  Returns y [B, D]."""
    torch = _torch()
    B, D = r.shape
    code = _act([r, s, gate], ["r", "s", "gate"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, D), device=r.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    st = lib().ssd_minmax_update(B, D, code, oc, _dev(r, "r"), _dev(s, "s", r.shape), _dev(gate, "gate", r.shape),
                                 _dev(state, "state", (B, D), torch.float32), _dev(y, "y"), _stream(r.device))
    _raise(st, "minmax_update")
    return y


def minmax_scan_backward(r, s, dy, x0=None, gate=None, dx_last=None, out_dtype=None, chunk_states=None,
                         workspace=None):
    """Gradients of ``minmax_scan`` for the loss sum(dy * y) + sum(dx_last * x_last) (see
    ``ssd_minmax_scan_backward``).  Returns a dict: dr, ds [B, L, D] (out dtype), dx0 [B, D] (fp32),
    and dgate when a gate is given."""
    torch = _torch()
    B, L, D = r.shape
    code = _act([r, s, gate, dy], ["r", "s", "gate", "dy"])
    oc = _out_code(out_dtype)
    odt = torch.bfloat16 if oc == SSD_BF16 else torch.float32
    g = {n: torch.empty((B, L, D), device=r.device, dtype=odt) for n in ("dr", "ds")}
    if gate is not None:
        g["dgate"] = torch.empty((B, L, D), device=r.device, dtype=odt)
    g["dx0"] = torch.empty((B, D), device=r.device, dtype=torch.float32)
    wp, wn = _workspace("minmax_scan_backward", _ws_bytes("minmax_scan_backward", B, L, D), r.device, workspace)
    st = lib().ssd_minmax_scan_backward(
        B, L, D, code, oc, _dev(r, "r"), _dev(s, "s", r.shape), _dev(x0, "x0", (B, D), torch.float32),
        _dev(gate, "gate", r.shape), _dev(chunk_states, "chunk_states", chunk_states_shape(B, L, D), torch.float32),
        _dev(dy, "dy", r.shape), _dev(dx_last, "dx_last", (B, D), torch.float32),
        _dev(g["dr"], "dr"), _dev(g["ds"], "ds"), _dev(g["dx0"], "dx0"), _dev(g.get("dgate"), "dgate"), wp, wn,
        _stream(r.device))
    _raise(st, "minmax_scan_backward")
    return g


# ----------------------------------------------------------------------------- causal conv1d
def causal_conv1d(x, weight, bias=None, state_in=None, return_state: bool = False, out_dtype=None):
    """Causal depthwise convolution over [B, L, D] with weight [D, W] (see ``ssd_causal_conv1d``).
    ``state_in`` [B, D, W] fp32 supplies the inputs before t = 0.  Returns y, or (y, state_out)."""
    torch = _torch()
    B, L, D = x.shape
    W = int(weight.shape[1]) if weight.dim() == 2 else -1
    code = _act([x], ["x"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, L, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    st_out = torch.empty((B, D, max(W, 0)), device=x.device, dtype=torch.float32) if return_state else None
    st = lib().ssd_causal_conv1d(B, L, D, W, code, oc, _dev(x, "x"), _dev(weight, "weight", (D, W), torch.float32),
                                 _dev(bias, "bias", (D,), torch.float32),
                                 _dev(state_in, "state_in", (B, D, W), torch.float32), _dev(y, "y"),
                                 _dev(st_out, "state_out"), _stream(x.device))
    _raise(st, "causal_conv1d")
    return (y, st_out) if return_state else y


def causal_conv1d_update(x, weight, state, bias=None, out_dtype=None):
    """One convolution decode step; ``state`` [B, D, W] fp32 is updated in place.  Returns y [B, D]."""
    torch = _torch()
    B, D = x.shape
    W = int(weight.shape[1]) if weight.dim() == 2 else -1
    code = _act([x], ["x"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    st = lib().ssd_causal_conv1d_update(B, D, W, code, oc, _dev(x, "x"), _dev(weight, "weight", (D, W), torch.float32),
                                        _dev(bias, "bias", (D,), torch.float32),
                                        _dev(state, "state", (B, D, W), torch.float32), _dev(y, "y"),
                                        _stream(x.device))
    _raise(st, "causal_conv1d_update")
    return y


# ----------------------------------------------------------------------------- selective
def _cu_seqlens_device(cu_seqlens, L, device, check: bool):
    torch = _torch()
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
        dev = cu_seqlens
        host = cu_seqlens.cpu().numpy() if check else None
    else:
        host = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
        dev = torch.from_numpy(host).to(device)
    if dev.dtype != torch.int32 or dev.dim() != 1 or not dev.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    if host is not None:
        if host.size < 1 or host[0] != 0 or host[-1] != L or np.any(np.diff(host.astype(np.int64)) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at L")
    return dev


def selective_scan(x, dt, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, dt_softplus: bool = True,
                   cu_seqlens=None, h0=None, return_last_state: bool = False, out_dtype=None,
                   check_cu_seqlens: bool = True, workspace=None):
    """Multi-scale selective scan over [B, L, D] with N states (see ``ssd_selective_scan``).

    ``cu_seqlens`` (int32 [nseq + 1], host or device) packs nseq sequences into B = 1.
    Returns y, or (y, h_last) with h_last [B or nseq, D, N]."""
    torch = _torch()
    B, L, D = x.shape
    N = A.shape[1]
    code = _act([x, dt, Bm, Cm, z], ["x", "dt", "Bm", "Cm", "z"])
    oc = _out_code(out_dtype)
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = _cu_seqlens_device(cu_seqlens, L, x.device, check_cu_seqlens)
        nseq = cu.numel() - 1
    y = torch.empty((B, L, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    h_last = torch.empty((nseq, D, N), device=x.device, dtype=torch.float32) if return_last_state else None
    wp, wn = _workspace("selective_scan", _ws_bytes("selective_scan", B, L, D, N, nseq, int(cu is not None)),
                        x.device, workspace)
    st = lib().ssd_selective_scan(
        B, L, D, N, code, oc, _dev(x, "x"), _dev(dt, "dt", x.shape), _dev(A, "A", (D, N), torch.float32),
        _dev(Bm, "Bm", (B, L, N)), _dev(Cm, "Cm", (B, L, N)), _dev(Dskip, "Dskip", (D,), torch.float32),
        _dev(z, "z", x.shape), _dev(dt_bias, "dt_bias", (D,), torch.float32), int(bool(dt_softplus)),
        _dev(cu, "cu_seqlens"), nseq, _dev(h0, "h0", (nseq, D, N), torch.float32), _dev(y, "y"),
        _dev(h_last, "h_last"), wp, wn, _stream(x.device))
    _raise(st, "selective_scan")
    return (y, h_last) if return_last_state else y


def selective_update(x, dt, A, Bm, Cm, state, Dskip=None, z=None, dt_bias=None, dt_softplus: bool = True,
                     out_dtype=None):
    """One decode step; ``state`` [B, D, N] fp32 is updated in place.  Returns y [B, D]."""
    torch = _torch()
    B, D = x.shape
    N = A.shape[1]
    code = _act([x, dt, Bm, Cm, z], ["x", "dt", "Bm", "Cm", "z"])
    oc = _out_code(out_dtype)
    y = torch.empty((B, D), device=x.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    st = lib().ssd_selective_update(
        B, D, N, code, oc, _dev(x, "x"), _dev(dt, "dt", x.shape), _dev(A, "A", (D, N), torch.float32),
        _dev(Bm, "Bm", (B, N)), _dev(Cm, "Cm", (B, N)), _dev(Dskip, "Dskip", (D,), torch.float32),
        _dev(z, "z", x.shape), _dev(dt_bias, "dt_bias", (D,), torch.float32), int(bool(dt_softplus)),
        _dev(state, "state", (B, D, N), torch.float32), _dev(y, "y"), _stream(x.device))
    _raise(st, "selective_update")
    return y


def selective_scan_backward(x, dt, A, Bm, Cm, dy, Dskip=None, z=None, dt_bias=None, dt_softplus: bool = True, h0=None,
                            dh_last=None, out_dtype=None, cu_seqlens=None, check_cu_seqlens: bool = True,
                            workspace=None):
    """Gradients of ``selective_scan`` for the loss sum(dy * y) + sum(dh_last * h_last) (see
    ``ssd_selective_scan_backward``); ``cu_seqlens`` as for ``selective_scan``.  Returns a dict: dx,
    ddt [B, L, D], dBm, dCm [B, L, N] (out dtype), dA [D, N], dh0 [B or nseq, D, N] (fp32), and dDskip,
    ddt_bias [D] (fp32), dz [B, L, D] for the optional inputs that are given."""
    torch = _torch()
    B, L, D = x.shape
    N = int(A.shape[1])
    code = _act([x, dt, Bm, Cm, z, dy], ["x", "dt", "Bm", "Cm", "z", "dy"])
    oc = _out_code(out_dtype)
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = _cu_seqlens_device(cu_seqlens, L, x.device, check_cu_seqlens)
        nseq = cu.numel() - 1
    odt = torch.bfloat16 if oc == SSD_BF16 else torch.float32
    dev = x.device
    g = {"dx": torch.empty((B, L, D), device=dev, dtype=odt), "ddt": torch.empty((B, L, D), device=dev, dtype=odt),
         "dA": torch.empty((D, N), device=dev, dtype=torch.float32),
         "dBm": torch.empty((B, L, N), device=dev, dtype=odt), "dCm": torch.empty((B, L, N), device=dev, dtype=odt),
         "dh0": torch.empty((nseq, D, N), device=dev, dtype=torch.float32)}
    if Dskip is not None:
        g["dDskip"] = torch.empty((D,), device=dev, dtype=torch.float32)
    if z is not None:
        g["dz"] = torch.empty((B, L, D), device=dev, dtype=odt)
    if dt_bias is not None:
        g["ddt_bias"] = torch.empty((D,), device=dev, dtype=torch.float32)
    wp, wn = _workspace("selective_scan_backward",
                        _ws_bytes("selective_scan_backward", B, L, D, N, nseq, int(cu is not None)), dev, workspace)
    st = lib().ssd_selective_scan_backward(
        B, L, D, N, code, oc, _dev(x, "x"), _dev(dt, "dt", x.shape), _dev(A, "A", (D, N), torch.float32),
        _dev(Bm, "Bm", (B, L, N)), _dev(Cm, "Cm", (B, L, N)), _dev(Dskip, "Dskip", (D,), torch.float32),
        _dev(z, "z", x.shape), _dev(dt_bias, "dt_bias", (D,), torch.float32), int(bool(dt_softplus)),
        _dev(cu, "cu_seqlens"), nseq, _dev(h0, "h0", (nseq, D, N), torch.float32), _dev(dy, "dy", x.shape),
        _dev(dh_last, "dh_last", (nseq, D, N), torch.float32), _dev(g["dx"], "dx"), _dev(g["ddt"], "ddt"),
        _dev(g["dA"], "dA"), _dev(g["dBm"], "dBm"), _dev(g["dCm"], "dCm"), _dev(g.get("dDskip"), "dDskip"),
        _dev(g.get("dz"), "dz"), _dev(g.get("ddt_bias"), "ddt_bias"), _dev(g["dh0"], "dh0"), wp, wn, _stream(dev))
    _raise(st, "selective_scan_backward")
    return g


# ----------------------------------------------------------------------------- HGRN2
def hgrn2_scan(q, k, v, g_logit, lower_bound: float, S0=None, return_last_state: bool = False, out_dtype=None,
               gate_axis: str = "value"):
    """HGRN2 matrix-state scan over [B, L, H, d] (see ``ssd_hgrn2_scan``; ``gate_axis="key"`` takes
    ``ssd_hgrn2_key_scan``).  Returns o, or (o, S_last)."""
    torch = _torch()
    B, L, H, d = q.shape
    code = _act([q, k, v, g_logit], ["q", "k", "v", "g_logit"])
    oc = _out_code(out_dtype)
    o = torch.empty((B, L, H, d), device=q.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    S_last = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32) if return_last_state else None
    fn = _gate_axis_fn(gate_axis, lib().ssd_hgrn2_scan, lib().ssd_hgrn2_key_scan)
    st = fn(B, L, H, d, code, oc, _dev(q, "q"), _dev(k, "k", q.shape), _dev(v, "v", q.shape),
            _dev(g_logit, "g_logit", q.shape), float(lower_bound), _dev(S0, "S0", (B, H, d, d), torch.float32),
            _dev(o, "o"), _dev(S_last, "S_last"), _stream(q.device))
    _raise(st, "hgrn2_scan")
    return (o, S_last) if return_last_state else o


def hgrn2_scan_backward(q, k, v, g_logit, lower_bound: float, do, S0=None, dS_last=None, o=None, out_dtype=None,
                        workspace=None):
    """Gradients of ``hgrn2_scan`` for the loss sum(do * o) + sum(dS_last * S_last) (see
    ``ssd_hgrn2_scan_backward``).  ``o`` may pass the forward's fp32 output to save recomputing it.
    Returns a dict: dq, dk, dv, dg_logit [B, L, H, d] (out dtype) and dS0 [B, H, d, d] (fp32)."""
    torch = _torch()
    B, L, H, d = q.shape
    code = _act([q, k, v, g_logit, do], ["q", "k", "v", "g_logit", "do"])
    oc = _out_code(out_dtype)
    odt = torch.bfloat16 if oc == SSD_BF16 else torch.float32
    dev = q.device
    g = {n: torch.empty((B, L, H, d), device=dev, dtype=odt) for n in ("dq", "dk", "dv", "dg_logit")}
    g["dS0"] = torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    wp, wn = _workspace("hgrn2_scan_backward",
                        _ws_bytes("hgrn2_scan_backward", B, L, H, d, code, int(o is not None)), dev, workspace)
    st = lib().ssd_hgrn2_scan_backward(
        B, L, H, d, code, oc, _dev(q, "q"), _dev(k, "k", q.shape), _dev(v, "v", q.shape),
        _dev(g_logit, "g_logit", q.shape), float(lower_bound), _dev(S0, "S0", (B, H, d, d), torch.float32),
        _dev(o, "o", q.shape, torch.float32), _dev(do, "do", q.shape),
        _dev(dS_last, "dS_last", (B, H, d, d), torch.float32), _dev(g["dq"], "dq"), _dev(g["dk"], "dk"),
        _dev(g["dv"], "dv"), _dev(g["dg_logit"], "dg_logit"), _dev(g["dS0"], "dS0"), wp, wn, _stream(dev))
    _raise(st, "hgrn2_scan_backward")
    return g


def _gate_axis_fn(gate_axis, value_fn, key_fn):
    if gate_axis == "value":
        return value_fn
    if gate_axis == "key":
        return key_fn
    raise ValueError('gate_axis must be "value" or "key"')


def hgrn2_update(q, k, v, g_logit, lower_bound: float, S, out_dtype=None, gate_axis: str = "value"):
    """One decode step; ``S`` [B, H, d, d] fp32 is updated in place.  Returns o [B, H, d]."""
    torch = _torch()
    B, H, d = q.shape
    code = _act([q, k, v, g_logit], ["q", "k", "v", "g_logit"])
    oc = _out_code(out_dtype)
    o = torch.empty((B, H, d), device=q.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    fn = _gate_axis_fn(gate_axis, lib().ssd_hgrn2_update, lib().ssd_hgrn2_key_update)
    st = fn(B, H, d, code, oc, _dev(q, "q"), _dev(k, "k", q.shape), _dev(v, "v", q.shape),
            _dev(g_logit, "g_logit", q.shape), float(lower_bound), _dev(S, "S", (B, H, d, d), torch.float32),
            _dev(o, "o"), _stream(q.device))
    _raise(st, "hgrn2_update")
    return o


def readout_norm(o, gate=None, weight=None, bias=None, eps: float = 1e-5, out_dtype=None):
    """LayerNorm over the last axis of the fp32 ``o`` (biased variance), affine, times silu(gate) (see
    ``ssd_readout_norm``).  For the layer's norm over its hidden size pass o as [B, L, H * d]."""
    torch = _torch()
    width = int(o.shape[-1])
    rows = o.numel() // width if width else 0
    code = _act([gate], ["gate"]) if gate is not None else SSD_BF16 if out_dtype == torch.bfloat16 else SSD_F32
    oc = _out_code(out_dtype)
    y = torch.empty(o.shape, device=o.device, dtype=torch.bfloat16 if oc == SSD_BF16 else torch.float32)
    st = lib().ssd_readout_norm(rows, width, code, oc, _dev(o, "o", None, torch.float32), _dev(gate, "gate", o.shape),
                                _dev(weight, "weight", (width,), torch.float32),
                                _dev(bias, "bias", (width,), torch.float32), float(eps), _dev(y, "y"),
                                _stream(o.device))
    _raise(st, "readout_norm")
    return y


__all__ = ["chunk_states_shape", "SCAN_CHUNK", "rglru_scan", "rglru_scan_noalloc", "rglru_scan_backward", "rglru_update", "selective_scan",
           "selective_scan_backward", "selective_update", "hgrn2_scan", "hgrn2_scan_backward", "hgrn2_update",
           "readout_norm", "minmax_scan", "minmax_update", "minmax_scan_backward", "causal_conv1d",
           "causal_conv1d_update", "workspace_check", "testing_lookback", "lib", "LIB_PATH", "EXPORTS", "SSDError",
           "SSDValueError", "SSD_F32", "SSD_BF16", "SSD_ERR_HIP", "SSD_ERR_TIMEOUT"]
