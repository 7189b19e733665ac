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


def _selective_case(seed, softplus=True, clamp=False, threshold=False):
    rng = np.random.default_rng(seed)
    B, L, D, N = 2, 6, 3, 4
    x, z, dy = (rng.standard_normal((B, L, D)) for _ in range(3))
    dt = rng.standard_normal((B, L, D)) * 0.5 - (1.0 if softplus else -0.6)
    A = -rng.uniform(0.5, 3.0, size=(D, N))
    Bm, Cm = (rng.standard_normal((B, L, N)) * 0.5 for _ in range(2))
    Dskip, dt_bias = rng.standard_normal(D), rng.standard_normal(D) * 0.3
    h0, dhl = rng.standard_normal((B, D, N)), rng.standard_normal((B, D, N))
    if clamp:  # channel 0: positive A, steps delta = 0.01 except delta = 1 at t = 2, where the clamp at 20 acts
        A[0, :] = [30.0, 45.0, 0.3, 60.0]  # on states 0, 1, 3 (10 to 40 beyond its edge) and they grow by e^20
        delta = np.full(L, 0.01)           # once; a tiny h0 and no input before that step keep the loss and
        delta[2] = 1.0                     # the gradients of order one, so differences stay precise
        v = np.log(np.expm1(delta)) if softplus else delta  # dt + dt_bias giving these steps
        dt[:, :, 0] = v - dt_bias[0]
        h0[:, 0, :] *= 1e-8
        x[:, :2, 0] = 0.0
    if threshold:  # channel 1: dt + dt_bias on both sides of softplus's threshold at 20, at least 0.3 away
        dt[:, :, 1] = np.array([18.5, 19.7, 20.3, 21.0, 24.0, 19.0]) - dt_bias[1]
    return dict(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, Dskip=Dskip, z=z, dt_bias=dt_bias, h0=h0), dy, dhl


# clamp: channel 0 has positive A and steps that put delta*A above the clamp at 20 (no gradient through
# the clamped exponent); threshold: channel 1 has dt + dt_bias around softplus's threshold at 20, where
# delta = dt + dt_bias exactly and its derivative is 1 (only with softplus on)
@pytest.mark.parametrize("softplus,clamp,threshold", [(True, False, False), (False, False, False),
                                                      (True, True, False), (False, True, False),
                                                      (True, False, True)])
def test_selective_grads_match_central_differences(softplus, clamp, threshold):
    k, dy, dhl = _selective_case(31 + softplus + 2 * clamp + 4 * threshold, softplus, clamp, threshold)
    G = og.selective_scan_grads(k["x"], k["dt"], k["A"], k["Bm"], k["Cm"], dy, Dskip=k["Dskip"], z=k["z"],
                                dt_bias=k["dt_bias"], dt_softplus=softplus, h0=k["h0"], dh_last=dhl)

    def F(**over):
        a = dict(k, **over)
        y, hl = oracle.selective_scan(a["x"], a["dt"], a["A"], a["Bm"], a["Cm"], Dskip=a["Dskip"], z=a["z"],
                                      dt_bias=a["dt_bias"], dt_softplus=softplus, h0=a["h0"])
        return _loss(y, hl, dy, dhl)

    names = [("x", "dx"), ("dt", "ddt"), ("A", "dA"), ("Bm", "dBm"), ("Cm", "dCm"), ("h0", "dh0"),
             ("Dskip", "dDskip"), ("z", "dz"), ("dt_bias", "ddt_bias")]
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
        assert err < 2e-6, (gname, err)


def test_selective_state_gradient_closed_form():
    """One state, no input: h_L = prod_t abar_t h0, so dL/dh0 = prod_t exp(delta_t A) for L = sum h_L."""
    B, L, D, N = 1, 5, 1, 1
    dt = np.array([0.1, 0.2, 0.05, 0.3, 0.15]).reshape(B, L, D)
    A = np.array([[-1.5]])
    zero = np.zeros((B, L, D))
    G = og.selective_scan_grads(zero, dt, A, np.zeros((B, L, N)), np.zeros((B, L, N)), zero, dt_softplus=False,
                                h0=np.ones((B, D, N)), dh_last=np.ones((B, D, N)))
    assert np.isclose(G["dh0"][0, 0, 0], np.exp(-1.5 * dt.sum()), rtol=1e-14, atol=0)
    # and dL/dA = sum(dt) * that (the state is h0 times the product)
    assert np.isclose(G["dA"][0, 0], dt.sum() * np.exp(-1.5 * dt.sum()), rtol=1e-13, atol=0)


def test_selective_clamp_passes_no_gradient_closed_form():
    """Two steps, one state, A > 0: the first exponent 0.1 A is below the clamp, the second 0.9 A = 27
    is clamped to 20.  With y_t = C_t h_t and L = w1 y1 + w2 y2 + dhl h2 (written out by hand):
    G2 = w2 C1 + dhl, G1 = w1 C0 + e^20 G2; dA = G1 d0 e^(d0 a) c (step 2 contributes nothing);
    d delta1 = G2 B1 x1 (no term through the clamped exponent); d delta0 = G1 (a e^(d0 a) c + B0 x0)."""
    a, c, d0, d1 = 30.0, 0.7, 0.1, 0.9
    x0, x1, B0, B1, C0, C1, w1, w2, dhl = 0.3, -1.1, 0.8, 0.5, -0.4, 1.3, 0.6, -0.2, 0.9
    G = og.selective_scan_grads(np.array([x0, x1]).reshape(1, 2, 1), np.array([d0, d1]).reshape(1, 2, 1),
                                np.array([[a]]), np.array([B0, B1]).reshape(1, 2, 1),
                                np.array([C0, C1]).reshape(1, 2, 1), np.array([w1, w2]).reshape(1, 2, 1),
                                dt_softplus=False, h0=np.array([[[c]]]), dh_last=np.array([[[dhl]]]))
    e0 = math.exp(d0 * a)
    G2 = w2 * C1 + dhl
    G1 = w1 * C0 + math.exp(20.0) * G2
    assert np.isclose(G["dA"][0, 0], G1 * d0 * e0 * c, rtol=1e-12, atol=0)
    assert np.isclose(G["ddt"][0, 1, 0], G2 * B1 * x1, rtol=1e-12, atol=0)
    assert np.isclose(G["ddt"][0, 0, 0], G1 * (a * e0 * c + B0 * x0), rtol=1e-12, atol=0)
    assert np.isclose(G["dh0"][0, 0, 0], G1 * e0, rtol=1e-12, atol=0)


def _hgrn2_case(seed, B=1, L=5, H=2, d=3, lb=0.3):
    rng = np.random.default_rng(seed)
    q, k, v, gl, do = (rng.standard_normal((B, L, H, d)) for _ in range(5))
    S0, dSl = rng.standard_normal((B, H, d, d)), rng.standard_normal((B, H, d, d))
    return dict(q=q, k=k, v=v, g_logit=gl, S0=S0), do, dSl, lb


def test_hgrn2_grads_match_central_differences():
    k, do, dSl, lb = _hgrn2_case(41)
    G = og.hgrn2_scan_grads(k["q"], k["k"], k["v"], k["g_logit"], lb, do, S0=k["S0"], dS_last=dSl)

    def F(**over):
        a = dict(k, **over)
        o, Sl = oracle.hgrn2_scan(a["q"], a["k"], a["v"], a["g_logit"], lb, S0=a["S0"])
        return float(np.sum(o * do) + np.sum(Sl * dSl))

    eps = 1e-6
    for arg, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g_logit", "dg_logit"), ("S0", "dS0")):
        base = k[arg]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += eps
            m[idx] -= eps
            num[idx] = (F(**{arg: p}) - F(**{arg: m})) / (2 * eps)
        err = np.max(np.abs(num - G[gname])) / max(np.max(np.abs(num)), 1e-12)
        assert err < 1e-6, (gname, err)


def test_hgrn2_grads_without_decay_are_linear_attention_closed_form():
    """lb = 1 makes g = 1: o_t = S0 q_t + sum_{s<=t} v_s (k_s . q_t) (causal linear attention), so, by hand,
    dq_t = S0^T do_t + sum_{s<=t} k_s (v_s . do_t), dk_s = sum_{t>=s} q_t (v_s . do_t) + dS_last^T v_s,
    dv_s = sum_{t>=s} do_t (k_s . q_t) + dS_last k_s, dS0 = sum_t do_t q_t^T + dS_last, dg_logit = 0."""
    k, do, dSl, _ = _hgrn2_case(43, B=1, L=6, H=1, d=4)
    q, kk, v, S0 = k["q"][0, :, 0], k["k"][0, :, 0], k["v"][0, :, 0], k["S0"][0, 0]
    dO, dS = do[0, :, 0], dSl[0, 0]
    G = og.hgrn2_scan_grads(k["q"], k["k"], k["v"], k["g_logit"], 1.0, do, S0=k["S0"], dS_last=dSl)
    L = q.shape[0]
    dq = np.array([S0.T @ dO[t] + sum(kk[s] * (v[s] @ dO[t]) for s in range(t + 1)) for t in range(L)])
    dk = np.array([sum(q[t] * (v[s] @ dO[t]) for t in range(s, L)) + dS.T @ v[s] for s in range(L)])
    dv = np.array([sum(dO[t] * (kk[s] @ q[t]) for t in range(s, L)) + dS @ kk[s] for s in range(L)])
    dS0 = sum(np.outer(dO[t], q[t]) for t in range(L)) + dS
    assert np.allclose(G["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    assert np.allclose(G["dk"][0, :, 0], dk, rtol=1e-12, atol=1e-12)
    assert np.allclose(G["dv"][0, :, 0], dv, rtol=1e-12, atol=1e-12)
    assert np.allclose(G["dS0"][0, 0], dS0, rtol=1e-12, atol=1e-12)
    assert np.all(G["dg_logit"] == 0.0)


def test_hgrn2_decay_only_closed_form():
    """v = 0 and do = 0: S_L = diag(prod_t g_t) S0, so with L = sum(dS_last * S_L):
    dS0 = diag(prod g) dS_last and dg_logit_t[i] = c_i (1 - lb) sigmoid'(x_t[i]) / g_t[i] with
    c_i = sum_j dS_last[i][j] S_L[i][j]; q and k get no gradient."""
    k, _, dSl, lb = _hgrn2_case(47, B=1, L=4, H=1, d=3, lb=0.25)
    z = np.zeros_like(k["v"])
    G = og.hgrn2_scan_grads(k["q"], k["k"], z, k["g_logit"], lb, z, S0=k["S0"], dS_last=dSl)
    x = k["g_logit"][0, :, 0]
    sig = 1.0 / (1.0 + np.exp(-x))
    g = lb + (1 - lb) * sig
    P = np.prod(g, axis=0)
    SL = P[:, None] * k["S0"][0, 0]
    c = np.sum(dSl[0, 0] * SL, axis=1)
    assert np.allclose(G["dS0"][0, 0], P[:, None] * dSl[0, 0], rtol=1e-13, atol=0)
    assert np.allclose(G["dg_logit"][0, :, 0], c[None, :] * (1 - lb) * sig * (1 - sig) / g, rtol=1e-12, atol=0)
    assert np.all(G["dq"] == 0.0) and np.all(G["dk"] == 0.0)
