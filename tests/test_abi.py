"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol that
include/ssd.h declares, and rejects invalid arguments before anything touches the GPU.

Pointers passed here are fake addresses: validation never dereferences them, and every call
below fails validation (or is an empty problem), so no kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_diag_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULL, SHAPE, DTYPE, ALIGN, VALUE, ALIAS, HIP, TIMEOUT = 0, 1, 2, 3, 4, 5, 6, 7, 8
F32, BF16 = 0, 1
P = 0x10000000  # fake, 16-byte aligned device addresses, far apart
MB = 1 << 20


def ptr(i):
    return ctypes.c_void_p(P + i * 64 * MB)


WS, WSB = ptr(30), 64 * MB  # a fake workspace, large enough for every call below


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ssd.LIB_PATH):
        import selective_state_space_diag_amd.build as b
        b.build()
    return ssd.lib()


def test_library_exports_every_declared_symbol(L):
    decl = declared_symbols()
    assert set(decl) == set(ssd.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ssd_[a-z0-9_]+)$", out, re.M))
    for name in decl:
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings_and_version(L):
    assert L.ssd_version() >= 100
    for code in range(9):
        assert L.ssd_status_str(code) != b"unknown status"
    assert L.ssd_status_str(99) == b"unknown status"


def rglru(L, B=2, Lq=8, D=4, ind=F32, outd=F32, x=0, r=1, i=2, a=3, c=8.0, h0=None, g=None, y=4, hl=None, cs=None,
          ws=WS, wsb=WSB):
    p = lambda k: None if k is None else ptr(k)
    return L.ssd_rglru_scan(B, Lq, D, ind, outd, p(x), p(r), p(i), p(a), c, p(h0), p(g), p(y), p(hl), p(cs), ws, wsb,
                            None)


def test_rglru_scan_validation(L):
    assert rglru(L, B=-1) == SHAPE
    assert rglru(L, ind=2) == DTYPE
    assert rglru(L, ind=F32, outd=BF16) == DTYPE
    assert rglru(L, x=None) == NULL
    assert rglru(L, a=None) == NULL
    assert rglru(L, c=float("inf")) == VALUE
    assert rglru(L, c=float("nan")) == VALUE
    assert rglru(L, y=0) == ALIAS                  # y on top of x
    assert rglru(L, h0=5, hl=5) == ALIAS           # h_last on top of h0
    assert rglru(L, g=6, y=6) == ALIAS             # y on top of the gate
    assert rglru(L, cs=2) == ALIAS                 # chunk states on top of i_logit
    assert L.ssd_rglru_scan(2, 8, 4, F32, F32, ctypes.c_void_p(P + 8), ptr(1), ptr(2), ptr(3), 8.0, None, None,
                            ptr(4), None, None, WS, WSB, None) == ALIGN
    assert L.ssd_rglru_scan(2, 8, 4, F32, F32, ptr(0), ptr(1), ptr(2), ptr(3), 8.0, None, None,
                            ptr(4), None, ctypes.c_void_p(P + 5 * 64 * MB + 4), WS, WSB, None) == ALIGN
    assert b"aligned" in L.ssd_last_error()
    # empty problem: nothing to do, no launch
    assert rglru(L, B=0) == OK
    assert L.ssd_last_error() == b""


def test_rglru_update_validation(L):
    f = lambda **kw: L.ssd_rglru_update(kw.get("B", 4), kw.get("D", 8), kw.get("ind", BF16), kw.get("outd", F32),
                                        ptr(0), ptr(1), ptr(2), ptr(3), kw.get("c", 8.0), kw.get("gate", None),
                                        kw.get("state", ptr(4)), kw.get("y", ptr(5)), None)
    assert f(D=-3) == SHAPE
    assert f(state=None) == NULL
    assert f(y=ptr(4)) == ALIAS
    assert f(y=ptr(0)) == ALIAS
    assert f(gate=ptr(6), y=ptr(6)) == ALIAS
    assert f(B=0) == OK


def test_minmax_validation(L):
    p = lambda k: None if k is None else ptr(k)
    f = lambda B=2, Lq=8, D=4, ind=BF16, outd=F32, r=0, s=1, x0=None, g=None, y=4, xl=None, cs=None: \
        L.ssd_minmax_scan(B, Lq, D, ind, outd, p(r), p(s), p(x0), p(g), p(y), p(xl), p(cs), WS, WSB, None)
    assert f(B=-1) == SHAPE
    assert f(ind=F32, outd=BF16) == DTYPE
    assert f(s=None) == NULL
    assert f(y=1) == ALIAS
    assert f(x0=5, xl=5) == ALIAS
    assert f(g=6, y=6) == ALIAS
    assert f(cs=0) == ALIAS
    assert L.ssd_minmax_scan(2, 8, 4, BF16, F32, ptr(0), ctypes.c_void_p(P + 1), None, None, ptr(4), None,
                             None, WS, WSB, None) == ALIGN
    assert f(D=0) == OK
    u = lambda B=4, D=8, st=4, y=5, g=None: L.ssd_minmax_update(B, D, BF16, F32, ptr(0), ptr(1), p(g), p(st), p(y),
                                                                None)
    assert u(D=-1) == SHAPE
    assert u(st=None) == NULL
    assert u(y=4) == ALIAS
    assert u(B=0) == OK


def test_causal_conv1d_validation(L):
    p = lambda k: None if k is None else ptr(k)
    f = lambda B=2, Lq=8, D=4, W=4, x=0, w=1, b=None, si=None, y=4, so=None: L.ssd_causal_conv1d(
        B, Lq, D, W, BF16, F32, p(x), p(w), p(b), p(si), p(y), p(so), None)
    assert f(W=0) == SHAPE
    assert f(W=5) == SHAPE
    assert f(Lq=-2) == SHAPE
    assert f(w=None) == NULL
    assert f(x=None) == NULL
    assert f(y=0) == ALIAS
    assert f(si=6, so=6) == ALIAS
    assert f(B=0) == OK
    u = lambda W=4, st=4, y=5: L.ssd_causal_conv1d_update(4, 8, W, BF16, F32, ptr(0), ptr(1), None, p(st), p(y), None)
    assert u(W=7) == SHAPE
    assert u(st=None) == NULL
    assert u(y=4) == ALIAS


def sel(L, B=1, Lq=16, D=8, N=16, ind=BF16, outd=F32, cu=None, nseq=0, y=9, A=2, Bm=3, Cm=4, h0=None, hl=None,
        ws=WS, wsb=WSB):
    p = lambda k: None if k is None else ptr(k)
    return L.ssd_selective_scan(B, Lq, D, N, ind, outd, ptr(0), ptr(1), p(A), p(Bm), p(Cm), None, None, None, 1,
                                p(cu), nseq, p(h0), p(y), p(hl), ws, wsb, None)


def test_selective_scan_validation(L):
    assert sel(L, N=3) == SHAPE
    assert sel(L, N=32) == SHAPE
    assert sel(L, B=2, cu=6, nseq=2) == SHAPE       # varlen needs B == 1
    assert sel(L, cu=6, nseq=-1) == SHAPE
    assert sel(L, cu=6, nseq=0) == SHAPE            # no sequences but L > 0
    assert sel(L, A=None) == NULL
    assert sel(L, Bm=None) == NULL
    assert sel(L, y=1) == ALIAS
    assert sel(L, h0=7, hl=7) == ALIAS
    assert sel(L, ind=F32, outd=BF16) == DTYPE
    assert sel(L, D=0) == OK


def test_selective_update_validation(L):
    f = lambda **kw: L.ssd_selective_update(kw.get("B", 2), kw.get("D", 8), kw.get("N", 16), BF16, F32, ptr(0),
                                            ptr(1), ptr(2), ptr(3), ptr(4), None, None, None, 1,
                                            kw.get("state", ptr(5)), kw.get("y", ptr(6)), None)
    assert f(N=5) == SHAPE
    assert f(state=None) == NULL
    assert f(y=ptr(5)) == ALIAS
    assert f(B=0) == OK


def h2(L, d=128, lb=0.5, o=5, S0=None, SL=None, B=2):
    p = lambda k: None if k is None else ptr(k)
    return L.ssd_hgrn2_scan(B, 16, 4, d, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), lb, p(S0), p(o), p(SL), None)


def test_hgrn2_validation(L):
    assert h2(L, d=48) == SHAPE
    assert h2(L, d=256) == SHAPE
    assert h2(L, lb=-0.1) == VALUE
    assert h2(L, lb=1.5) == VALUE
    assert h2(L, lb=float("nan")) == VALUE
    assert h2(L, o=None) == NULL
    assert h2(L, o=2) == ALIAS
    assert h2(L, S0=6, SL=6) == ALIAS
    assert h2(L, B=0) == OK
    f = lambda **kw: L.ssd_hgrn2_update(2, 4, kw.get("d", 64), BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3),
                                        kw.get("lb", 0.5), kw.get("S", ptr(4)), kw.get("o", ptr(5)), None)
    assert f(d=100) == SHAPE
    assert f(S=None) == NULL
    assert f(o=ptr(4)) == ALIAS
    assert f(lb=2.0) == VALUE


def test_hgrn2_backward_validation(L):
    p = lambda k: None if k is None else ptr(k)
    f = lambda B=2, d=64, lb=0.5, do=5, o=None, dq=6, dS0=None, S0=None, ws=WS, wsb=WSB: L.ssd_hgrn2_scan_backward(
        B, 16, 4, d, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), lb, p(S0), p(o), p(do), None, p(dq), ptr(7), ptr(8),
        ptr(9), p(dS0), ws, wsb, None)
    assert f(d=48) == SHAPE
    assert f(lb=1.5) == VALUE
    assert f(do=None) == NULL
    assert f(dq=None) == NULL
    assert f(dq=0) == ALIAS           # dq on top of q
    assert f(o=10, dq=10) == ALIAS    # dq on top of the given forward output
    assert f(S0=11, dS0=11) == ALIAS
    assert L.ssd_hgrn2_scan_backward(2, 16, 4, 64, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), 0.5, None,
                                     ctypes.c_void_p(P + 10 * 64 * MB + 8), ptr(5), None, ptr(6), ptr(7), ptr(8),
                                     ptr(9), None, WS, WSB, None) == ALIGN
    assert f(B=0) == OK


def test_hgrn2_key_and_readout_norm_validation(L):
    p = lambda k: None if k is None else ptr(k)
    f = lambda B=2, Lq=16, d=64, lb=0.5, o=5, S0=None, SL=None: L.ssd_hgrn2_key_scan(
        B, Lq, 4, d, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), lb, p(S0), p(o), p(SL), None)
    assert f(d=48) == SHAPE
    assert f(lb=-1.0) == VALUE
    assert f(o=None) == NULL
    assert f(o=1) == ALIAS
    assert f(S0=6, SL=6) == ALIAS
    assert f(B=0) == OK
    u = lambda d=64, S=4, o=5: L.ssd_hgrn2_key_update(2, 4, d, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), 0.5, p(S),
                                                      p(o), None)
    assert u(d=100) == SHAPE
    assert u(S=None) == NULL
    assert u(o=4) == ALIAS
    n = lambda rows=8, width=64, ind=BF16, outd=F32, o=0, g=1, w=None, b=None, eps=1e-5, y=4: L.ssd_readout_norm(
        rows, width, ind, outd, p(o), p(g), p(w), p(b), eps, p(y), None)
    assert n(width=8193) == SHAPE
    assert n(rows=-1) == SHAPE
    assert n(ind=F32, outd=BF16) == DTYPE
    assert n(eps=-1.0) == VALUE
    assert n(eps=float("nan")) == VALUE
    assert n(o=None) == NULL
    assert n(y=0) == ALIAS
    assert n(y=1) == ALIAS
    assert n(w=4, y=4) == ALIAS
    assert L.ssd_readout_norm(8, 64, BF16, F32, ctypes.c_void_p(P + 4), None, None, None, 1e-5, ptr(4), None) == ALIGN
    assert n(rows=0) == OK


def test_workspace_validation(L):
    """A call that passes every other check still needs its workspace: present, 256-byte aligned, as large as
    the query says, and apart from every other argument.  (These calls stop at the workspace check.)"""
    need = ctypes.c_size_t(0)
    assert L.ssd_rglru_scan_workspace_bytes(2, 8, 4, ctypes.byref(need)) == OK and need.value > 0
    assert rglru(L, ws=None) == NULL
    assert b"workspace" in L.ssd_last_error()
    assert rglru(L, ws=ctypes.c_void_p(P + 30 * 64 * MB + 128)) == ALIGN
    assert rglru(L, wsb=need.value - 1) == SHAPE
    assert rglru(L, ws=ptr(0)) == ALIAS                         # on top of x
    assert rglru(L, ws=ptr(4), wsb=need.value) == ALIAS        # on top of y
    assert sel(L, ws=None) == NULL
    assert sel(L, wsb=16) == SHAPE
    assert sel(L, ws=ptr(9)) == ALIAS
    # empty problems need none
    assert rglru(L, B=0, ws=None, wsb=0) == OK
    assert sel(L, D=0, ws=None, wsb=0) == OK
    # the backward calls too
    p = lambda k: None if k is None else ptr(k)
    assert L.ssd_rglru_scan_backward(2, 8, 4, F32, F32, ptr(0), ptr(1), ptr(2), ptr(3), 8.0, None, None, None, ptr(5),
                                     None, ptr(6), ptr(7), ptr(8), ptr(9), None, None, None, 0, None) == NULL
    assert L.ssd_minmax_scan_backward(2, 8, 4, BF16, F32, ptr(0), ptr(1), None, None, None, ptr(5), None, ptr(6),
                                      ptr(7), None, None, ptr(6), WSB, None) == ALIAS
    assert L.ssd_selective_scan_backward(1, 16, 8, 16, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), ptr(4), None, None,
                                         None, 1, None, 0, None, ptr(5), None, ptr(6), ptr(7), ptr(8), ptr(10),
                                         ptr(11), None, None, None, None, WS, 8, None) == SHAPE
    assert L.ssd_hgrn2_scan_backward(2, 16, 4, 64, BF16, F32, ptr(0), ptr(1), ptr(2), ptr(3), 0.5, None, None, ptr(5),
                                     None, ptr(6), ptr(7), ptr(8), ptr(9), None, None, 0, None) == NULL


def test_workspace_queries(L):
    n = ctypes.c_size_t(123)
    q = lambda fn, *a: (fn(*a, ctypes.byref(n)), n.value)
    # scan1 family: control block + lookback words, growing with the number of (batch, tile, chunk) units
    st, small = q(L.ssd_rglru_scan_workspace_bytes, 2, 64, 128)
    assert st == OK and small > 0
    st, big = q(L.ssd_rglru_scan_workspace_bytes, 2, 6400, 128)
    assert st == OK and big > small
    assert q(L.ssd_minmax_scan_workspace_bytes, 2, 6400, 128) == (OK, big)
    assert q(L.ssd_rglru_scan_workspace_bytes, 0, 64, 128) == (OK, 0)
    assert L.ssd_rglru_scan_workspace_bytes(-1, 64, 128, ctypes.byref(n)) == SHAPE
    assert L.ssd_rglru_scan_workspace_bytes(2, 64, 128, None) == NULL
    for fn in (L.ssd_rglru_scan_backward_workspace_bytes, L.ssd_minmax_scan_backward_workspace_bytes):
        st, v = q(fn, 4, 1000, 96)
        assert st == OK and v > 0
    st, v = q(L.ssd_selective_scan_workspace_bytes, 4, 2048, 1536, 16, 0, 0)
    assert st == OK and v > 0
    st, v = q(L.ssd_selective_scan_workspace_bytes, 1, 5000, 256, 16, 3, 1)
    assert st == OK and v > 0
    assert q(L.ssd_selective_scan_workspace_bytes, 1, 0, 256, 16, 0, 1) == (OK, 0)
    assert L.ssd_selective_scan_workspace_bytes(2, 100, 256, 16, 3, 1, ctypes.byref(n)) == SHAPE  # packed needs B = 1
    assert L.ssd_selective_scan_workspace_bytes(1, 100, 256, 5, 0, 0, ctypes.byref(n)) == SHAPE   # N
    st, v = q(L.ssd_selective_scan_backward_workspace_bytes, 2, 100, 64, 16, 0, 0)
    assert st == OK and v > 0
    st, with_o = q(L.ssd_hgrn2_scan_backward_workspace_bytes, 2, 100, 4, 64, BF16, 1)
    st2, without_o = q(L.ssd_hgrn2_scan_backward_workspace_bytes, 2, 100, 4, 64, BF16, 0)
    assert st == st2 == OK and without_o == with_o + 2 * 100 * 4 * 64 * 4
    st, f32 = q(L.ssd_hgrn2_scan_backward_workspace_bytes, 2, 100, 4, 64, F32, 1)
    assert st == OK and f32 > with_o   # fp32 inputs keep state checkpoints
    assert L.ssd_hgrn2_scan_backward_workspace_bytes(2, 100, 4, 48, BF16, 1, ctypes.byref(n)) == SHAPE
    assert L.ssd_hgrn2_scan_backward_workspace_bytes(2, 100, 4, 64, 5, 1, ctypes.byref(n)) == DTYPE


def test_workspace_check_validation(L):
    assert L.ssd_workspace_check(None, None) == NULL
    L.ssd_testing_lookback(0, 0)   # the hook itself touches no device


def test_python_layer_requires_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        ssd.rglru_scan(x, x, x, torch.zeros(8), 8.0)
