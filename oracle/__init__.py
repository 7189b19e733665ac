"""ctypes loader for the fp64 CPU oracle (``oracle/ssd_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``selective_state_space_diag_amd``) never imports it, and this package never
imports the product path.

Every wrapper takes float64 numpy arrays (exact upcasts of the bf16 / fp32
input bits) and returns freshly allocated float64 outputs.  The recurrences
themselves live in the C file; this module only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_LIBRARY names another build of the same C file (a sanitizer build in the tests)
_LIB_PATH = os.environ.get("SSD_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_affine_scan.argtypes = [_i64, _dp, _dp, ctypes.c_double, _dp]
        L.oracle_gelu.argtypes = [ctypes.c_double]
        L.oracle_gelu.restype = ctypes.c_double
        L.oracle_rglru_scan.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp, _dp]
        L.oracle_rglru_update.argtypes = [_i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp]
        L.oracle_minmax_scan.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp]
        L.oracle_minmax_update.argtypes = [_i64, _i64, _dp, _dp, _dp, _dp, _dp]
        L.oracle_causal_conv1d.argtypes = [_i64, _i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp]
        L.oracle_causal_conv1d_update.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp]
        L.oracle_selective_scan.argtypes = [_i64, _i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                            ctypes.c_int, _ip, _i64, _dp, _dp, _dp]
        L.oracle_selective_update.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                              ctypes.c_int, _dp, _dp]
        L.oracle_hgrn2_scan.argtypes = [_i64, _i64, _i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp]
        L.oracle_hgrn2_update.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp]
        L.oracle_hgrn2_key_scan.argtypes = [_i64, _i64, _i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp,
                                            _dp]
        L.oracle_hgrn2_key_update.argtypes = [_i64, _i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp]
        L.oracle_readout_norm.argtypes = [_i64, _i64, _dp, _dp, _dp, _dp, ctypes.c_double, _dp]
        for fn in ("oracle_affine_scan", "oracle_rglru_scan", "oracle_rglru_update", "oracle_selective_scan",
                   "oracle_selective_update", "oracle_hgrn2_scan", "oracle_hgrn2_update", "oracle_minmax_scan",
                   "oracle_minmax_update", "oracle_causal_conv1d", "oracle_causal_conv1d_update",
                   "oracle_hgrn2_key_scan", "oracle_hgrn2_key_update", "oracle_readout_norm"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    """Pointer to a C-contiguous float64 array, or NULL for None."""
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous float64"
    return a.ctypes.data_as(_dp)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (status {rc})")


def affine_scan(a, b, h0=0.0):
    a, b = _f64(a), _f64(b)
    h = np.empty_like(a)
    _check(lib().oracle_affine_scan(a.size, _p(a), _p(b), float(h0), _p(h)), "affine_scan")
    return h


def gelu(v):
    return lib().oracle_gelu(float(v))


def rglru_scan(x, r_logit, i_logit, a_log, c, h0=None, gate=None):
    """Returns (y [B,L,D], h_last [B,D]); y = gelu(gate) * h when gate is given."""
    x, r_logit, i_logit, a_log, h0, gate = map(_f64, (x, r_logit, i_logit, a_log, h0, gate))
    B, L, D = x.shape
    y = np.empty((B, L, D))
    h_last = np.empty((B, D))
    _check(lib().oracle_rglru_scan(B, L, D, _p(x), _p(r_logit), _p(i_logit), _p(a_log), float(c), _p(h0),
                                   _p(gate), _p(y), _p(h_last)), "rglru_scan")
    return y, h_last


def rglru_update(x, r_logit, i_logit, a_log, c, state, gate=None):
    """Returns (y [B,D], new_state [B,D]); the input state is not modified."""
    x, r_logit, i_logit, a_log, gate = map(_f64, (x, r_logit, i_logit, a_log, gate))
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, D = x.shape
    y = np.empty((B, D))
    _check(lib().oracle_rglru_update(B, D, _p(x), _p(r_logit), _p(i_logit), _p(a_log), float(c), _p(gate),
                                     _p(st), _p(y)), "rglru_update")
    return y, st


def selective_scan(x, dt, A, Bm, Cm, Dskip=None, z=None, dt_bias=None, dt_softplus=True,
                   cu_seqlens=None, h0=None):
    """Returns (y [B,L,D], h_last [B or nseq, D, N])."""
    x, dt, A, Bm, Cm, Dskip, z, dt_bias, h0 = map(_f64, (x, dt, A, Bm, Cm, Dskip, z, dt_bias, h0))
    B, L, D = x.shape
    N = A.shape[1]
    cu = None
    nseq = B
    cu_ptr = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        nseq = cu.size - 1
        cu_ptr = cu.ctypes.data_as(_ip)
    y = np.empty((B, L, D))
    h_last = np.empty((nseq, D, N))
    _check(lib().oracle_selective_scan(B, L, D, N, _p(x), _p(dt), _p(A), _p(Bm), _p(Cm), _p(Dskip), _p(z),
                                       _p(dt_bias), int(bool(dt_softplus)), cu_ptr, nseq, _p(h0), _p(y),
                                       _p(h_last)), "selective_scan")
    return y, h_last


def selective_update(x, dt, A, Bm, Cm, state, Dskip=None, z=None, dt_bias=None, dt_softplus=True):
    """Returns (y [B,D], new_state [B,D,N]); the input state is not modified."""
    x, dt, A, Bm, Cm, Dskip, z, dt_bias = map(_f64, (x, dt, A, Bm, Cm, Dskip, z, dt_bias))
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, D = x.shape
    N = A.shape[1]
    y = np.empty((B, D))
    _check(lib().oracle_selective_update(B, D, N, _p(x), _p(dt), _p(A), _p(Bm), _p(Cm), _p(Dskip), _p(z),
                                         _p(dt_bias), int(bool(dt_softplus)), _p(st), _p(y)), "selective_update")
    return y, st


def hgrn2_scan(q, k, v, g_logit, lower_bound, S0=None):
    """Returns (o [B,L,H,d], S_last [B,H,d,d])."""
    q, k, v, g_logit, S0 = map(_f64, (q, k, v, g_logit, S0))
    B, L, H, d = q.shape
    o = np.empty((B, L, H, d))
    S_last = np.empty((B, H, d, d))
    _check(lib().oracle_hgrn2_scan(B, L, H, d, _p(q), _p(k), _p(v), _p(g_logit), float(lower_bound), _p(S0),
                                   _p(o), _p(S_last)), "hgrn2_scan")
    return o, S_last


def hgrn2_update(q, k, v, g_logit, lower_bound, S):
    """Returns (o [B,H,d], new_S [B,H,d,d]); the input state is not modified."""
    q, k, v, g_logit = map(_f64, (q, k, v, g_logit))
    St = np.array(S, dtype=np.float64, copy=True, order="C")
    B, H, d = q.shape
    o = np.empty((B, H, d))
    _check(lib().oracle_hgrn2_update(B, H, d, _p(q), _p(k), _p(v), _p(g_logit), float(lower_bound), _p(St), _p(o)),
           "hgrn2_update")
    return o, St


def hgrn2_key_scan(q, k, v, g_logit, lower_bound, S0=None):
    """Key-axis gating (S[i][j] = g_j S[i][j] + v_i k_j).  Returns (o [B,L,H,d], S_last [B,H,d,d])."""
    q, k, v, g_logit, S0 = map(_f64, (q, k, v, g_logit, S0))
    B, L, H, d = q.shape
    o = np.empty((B, L, H, d))
    S_last = np.empty((B, H, d, d))
    _check(lib().oracle_hgrn2_key_scan(B, L, H, d, _p(q), _p(k), _p(v), _p(g_logit), float(lower_bound), _p(S0),
                                       _p(o), _p(S_last)), "hgrn2_key_scan")
    return o, S_last


def hgrn2_key_update(q, k, v, g_logit, lower_bound, S):
    """Returns (o [B,H,d], new_S [B,H,d,d]); the input state is not modified."""
    q, k, v, g_logit = map(_f64, (q, k, v, g_logit))
    St = np.array(S, dtype=np.float64, copy=True, order="C")
    B, H, d = q.shape
    o = np.empty((B, H, d))
    _check(lib().oracle_hgrn2_key_update(B, H, d, _p(q), _p(k), _p(v), _p(g_logit), float(lower_bound), _p(St),
                                         _p(o)), "hgrn2_key_update")
    return o, St


def readout_norm(o, gate=None, weight=None, bias=None, eps=1e-5):
    """LayerNorm over the last axis of ``o`` (biased variance), affine, times silu(gate)."""
    o, gate, weight, bias = map(_f64, (o, gate, weight, bias))
    width = o.shape[-1]
    rows = o.size // width if width else 0
    y = np.empty(o.shape)
    _check(lib().oracle_readout_norm(rows, width, _p(o), _p(gate), _p(weight), _p(bias), float(eps), _p(y)),
           "readout_norm")
    return y


def minmax_scan(r, s, x0=None, gate=None):
    """Returns (y [B,L,D], x_last [B,D])."""
    r, s, x0, gate = map(_f64, (r, s, x0, gate))
    B, L, D = r.shape
    y = np.empty((B, L, D))
    x_last = np.empty((B, D))
    _check(lib().oracle_minmax_scan(B, L, D, _p(r), _p(s), _p(x0), _p(gate), _p(y), _p(x_last)), "minmax_scan")
    return y, x_last


def minmax_update(r, s, state, gate=None):
    """Returns (y [B,D], new_state [B,D]); the input state is not modified."""
    r, s, gate = map(_f64, (r, s, gate))
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, D = r.shape
    y = np.empty((B, D))
    _check(lib().oracle_minmax_update(B, D, _p(r), _p(s), _p(gate), _p(st), _p(y)), "minmax_update")
    return y, st


def causal_conv1d(x, weight, bias=None, state_in=None):
    """Returns (y [B,L,D], state_out [B,D,W])."""
    x, weight, bias, state_in = map(_f64, (x, weight, bias, state_in))
    B, L, D = x.shape
    W = weight.shape[1]
    y = np.empty((B, L, D))
    st = np.empty((B, D, W))
    _check(lib().oracle_causal_conv1d(B, L, D, W, _p(x), _p(weight), _p(bias), _p(state_in), _p(y), _p(st)),
           "causal_conv1d")
    return y, st


def causal_conv1d_update(x, weight, state, bias=None):
    """Returns (y [B,D], new_state [B,D,W]); the input state is not modified."""
    x, weight, bias = map(_f64, (x, weight, bias))
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, D = x.shape
    W = weight.shape[1]
    y = np.empty((B, D))
    _check(lib().oracle_causal_conv1d_update(B, D, W, _p(x), _p(weight), _p(bias), _p(st), _p(y)),
           "causal_conv1d_update")
    return y, st
