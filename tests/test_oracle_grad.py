"""Pins of the gradient oracle (oracle/grad.py, autograd over a sequential float64 forward) against
central finite differences of the C forward oracle, which shares no code with it, and closed forms."""
import math

import numpy as np
import pytest

import oracle
from oracle import grad as og


def _loss(y, hl, dy, dhl):
    return float(np.sum(y * dy) + (0.0 if dhl is None else np.sum(hl * dhl)))


def _rglru_case(seed, B=2, L=7, D=3, gated=True, with_h0=True):
    rng = np.random.default_rng(seed)
    x, r, i, g, dy = (rng.standard_normal((B, L, D)) for _ in range(5))
    a_log = np.log(rng.uniform(0.9, 0.999, size=D))
    h0 = rng.standard_normal((B, D)) if with_h0 else None
    dhl = rng.standard_normal((B, D))
    return dict(x=x, r_logit=r, i_logit=i, a_log=a_log, h0=h0, gate=g if gated else None, dy=dy, dh_last=dhl)


@pytest.mark.parametrize("gated", [False, True])
def test_rglru_grads_match_central_differences(gated):
    k = _rglru_case(3 + gated, gated=gated)
    c = 8.0
    G = og.rglru_scan_grads(k["x"], k["r_logit"], k["i_logit"], k["a_log"], c, k["dy"], h0=k["h0"], gate=k["gate"],
                            dh_last=k["dh_last"])

    def F(**over):
        a = dict(k, **over)
        y, hl = oracle.rglru_scan(a["x"], a["r_logit"], a["i_logit"], a["a_log"], c, h0=a["h0"], gate=a["gate"])
        return _loss(y, hl, k["dy"], k["dh_last"])

    names = [("x", "dx"), ("r_logit", "dr_logit"), ("i_logit", "di_logit"), ("a_log", "da_log"), ("h0", "dh0")]
    if gated:
        names.append(("gate", "dgate"))
    eps = 1e-6
    for arg, gname in names:
        base = k[arg]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += eps
            m[idx] -= eps
            num[idx] = (F(**{arg: p}) - F(**{arg: m})) / (2 * eps)
        err = np.max(np.abs(num - G[gname])) / max(np.max(np.abs(num)), 1e-12)
        assert err < 1e-6, (gname, err)


def test_rglru_state_gradient_closed_form():
    """dL/dh0 for L = sum(h_last) is prod_t a_t with a_t = exp(c sigmoid(r_t) a_log)."""
    rng = np.random.default_rng(9)
    B, L, D, c = 1, 12, 2, 8.0
    r = rng.standard_normal((B, L, D))
    a_log = np.log(np.array([0.95, 0.99]))
    z = np.zeros((B, L, D))
    G = og.rglru_scan_grads(z + 0.3, r, z, a_log, c, z, h0=np.zeros((B, D)), dh_last=np.ones((B, D)))
    want = np.exp(np.sum(c * (1.0 / (1.0 + np.exp(-r))) * a_log, axis=1))
    assert np.allclose(G["dh0"], want, rtol=1e-13, atol=0)
    assert np.all(G["dx"][:, :, :] != 0.0)  # every input reaches h_last


def test_minmax_grads_match_central_differences():
    """Away from ties the MinMax scan is piecewise linear in its inputs: differences are exact."""
    rng = np.random.default_rng(21)
    B, L, D = 2, 9, 3
    r, s, g, dy = (rng.standard_normal((B, L, D)) for _ in range(4))
    x0, dxl = rng.standard_normal((B, D)), rng.standard_normal((B, D))
    G = og.minmax_scan_grads(r, s, dy, x0=x0, gate=g, dx_last=dxl)

    def F(r=r, s=s, x0=x0, g=g):
        y, xl = oracle.minmax_scan(r, s, x0=x0, gate=g)
        return _loss(y, xl, dy, dxl)

    eps = 1e-7
    for arg, gname, base in (("r", "dr", r), ("s", "ds", s), ("x0", "dx0", x0), ("g", "dgate", g)):
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += eps
            m[idx] -= eps
            num[idx] = (F(**{arg: p}) - F(**{arg: m})) / (2 * eps)
        assert np.max(np.abs(num - G[gname])) < 1e-6, gname


def test_minmax_grads_route_and_split_at_ties():
    one = lambda v: np.array(v, dtype=np.float64).reshape(1, -1, 1)
    # the upper clamp wins: the gradient goes to r, none to the state
    G = og.minmax_scan_grads(one([0.5]), one([-5.0]), one([1.0]), x0=np.array([[2.0]]))
    assert G["dr"][0, 0, 0] == 1.0 and G["dx0"][0, 0] == 0.0 and G["ds"][0, 0, 0] == 0.0
    # the lower clamp wins
    G = og.minmax_scan_grads(one([0.5]), one([0.7]), one([1.0]), x0=np.array([[2.0]]))
    assert G["ds"][0, 0, 0] == 1.0 and G["dr"][0, 0, 0] == 0.0
    # r equal to the state: half each; then s equal to that minimum: half of it again
    G = og.minmax_scan_grads(one([1.0]), one([-5.0]), one([1.0]), x0=np.array([[1.0]]))
    assert G["dr"][0, 0, 0] == 0.5 and G["dx0"][0, 0] == 0.5
    G = og.minmax_scan_grads(one([1.0]), one([1.0]), one([1.0]), x0=np.array([[1.0]]))
    assert G["ds"][0, 0, 0] == 0.5 and G["dr"][0, 0, 0] == 0.25 and G["dx0"][0, 0] == 0.25
