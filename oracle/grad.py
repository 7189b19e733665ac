"""Gradients of the scans, for checking the backward kernels.  TEST INFRASTRUCTURE ONLY (same rule
as the rest of ``oracle/``: only the tests, the smoke check and the benchmark's CPU-baseline leg use
it; it shares no code with the HIP library).

The pages train their models with torch autograd over the forward pass and print no backward pass,
so the reference gradient is autograd itself, run in float64 on the CPU over a plain sequential
forward loop written from the recurrence:

  RG-LRU (lrnnx documentation, "lrnnx.models.ltv.rglru": RGLRU.forward gates and the RGLRU.step
  update, with the block's gelu(gate) output multiply):
      r = sigmoid(r_logit), i = sigmoid(i_logit), a = exp(c r a_log),
      h_t = a h_{t-1} + sqrt(1 - a^2) (i x),   y_t = h_t, or gelu(gate_t) h_t.

  MinMax (minmaxrnc package, MinMaxNeuron / minmax_operator): x_t = max(min(r_t, x_{t-1}), s_t),
      y_t = x_t or x_t g_t; torch's min / max split the gradient equally between equal operands.

  Selective scan (cortexnet 3.2.1, cortexnet/ssm.py, MultiScaleSSM.forward / _selective_scan):
      delta = softplus(dt + dt_bias) (or dt + dt_bias), abar = exp(clamp(delta A, max=20)),
      h_t = abar h_{t-1} + (delta B_t) x_t,  y_t = (sum_n C_t,n h_t,n + Dskip x_t) silu(z_t);
      the clamp passes the gradient where delta A <= 20 (torch.clamp).

  HGRN2 (frankenstein-transformer documentation, "HGRN2 Attention", state update and gate):
      g = lb + (1 - lb) sigmoid(g_logit),  S[i][j] = g_i S[i][j] + v_i k_j,  o_i = sum_j S[i][j] q_j.

The loss whose gradient is returned is  sum(dy * y) + sum(dh_last * h_last) (x_last for MinMax;
do and dS_last for HGRN2).
"""
from __future__ import annotations

import numpy as np


def _t(a):
    import torch
    return None if a is None else torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64, requires_grad=True)


def rglru_scan_grads(x, r_logit, i_logit, a_log, c, dy, h0=None, gate=None, dh_last=None):
    """Returns a dict of float64 numpy gradients: dx, dr_logit, di_logit [B,L,D], da_log [D],
    dh0 [B,D] (of a zero state when h0 is None), dgate [B,L,D] (when gate is given)."""
    import torch
    xs, rs, is_, al, gt = _t(x), _t(r_logit), _t(i_logit), _t(a_log), _t(gate)
    B, L, D = xs.shape
    h = _t(h0) if h0 is not None else torch.zeros((B, D), dtype=torch.float64, requires_grad=True)
    h_init = h
    ys = []
    for t in range(L):
        r = torch.sigmoid(rs[:, t])
        i = torch.sigmoid(is_[:, t])
        lam = c * r * al
        a = torch.exp(lam)
        beta = torch.sqrt(1.0 - a * a)
        h = a * h + beta * (i * xs[:, t])
        ys.append(h if gt is None else torch.nn.functional.gelu(gt[:, t]) * h)
    y = torch.stack(ys, dim=1) if L > 0 else torch.zeros((B, 0, D), dtype=torch.float64)
    loss = (y * torch.as_tensor(np.asarray(dy, dtype=np.float64))).sum()
    if dh_last is not None:
        loss = loss + (h * torch.as_tensor(np.asarray(dh_last, dtype=np.float64))).sum()
    inputs = [xs, rs, is_, al, h_init] + ([gt] if gt is not None else [])
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    z = lambda g, ref: np.zeros(ref.shape) if g is None else g.detach().numpy()
    out = dict(dx=z(grads[0], xs), dr_logit=z(grads[1], rs), di_logit=z(grads[2], is_), da_log=z(grads[3], al),
               dh0=z(grads[4], h_init))
    if gt is not None:
        out["dgate"] = z(grads[5], gt)
    return out


def minmax_scan_grads(r, s, dy, x0=None, gate=None, dx_last=None):
    """Gradients of the MinMax scan (minmaxrnc MinMaxNeuron: x_t = max(min(r_t, x_{t-1}), s_t), y_t = x_t
    or x_t * gate_t) for the loss sum(dy * y) + sum(dx_last * x_last), by autograd through
    torch.minimum / torch.maximum: where the two operands are equal, torch gives each half of the
    gradient.  Returns dr, ds [B,L,D], dx0 [B,D] and dgate [B,L,D] (when gate is given)."""
    import torch
    rs, ss, gt = _t(r), _t(s), _t(gate)
    B, L, D = rs.shape
    xv = _t(x0) if x0 is not None else torch.zeros((B, D), dtype=torch.float64, requires_grad=True)
    x_init = xv
    ys = []
    for t in range(L):
        xv = torch.maximum(torch.minimum(rs[:, t], xv), ss[:, t])
        ys.append(xv if gt is None else xv * gt[:, t])
    y = torch.stack(ys, dim=1) if L > 0 else torch.zeros((B, 0, D), dtype=torch.float64)
    loss = (y * torch.as_tensor(np.asarray(dy, dtype=np.float64))).sum()
    if dx_last is not None:
        loss = loss + (xv * torch.as_tensor(np.asarray(dx_last, dtype=np.float64))).sum()
    inputs = [rs, ss, x_init] + ([gt] if gt is not None else [])
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    z = lambda g, ref: np.zeros(ref.shape) if g is None else g.detach().numpy()
    out = dict(dr=z(grads[0], rs), ds=z(grads[1], ss), dx0=z(grads[2], x_init))
    if gt is not None:
        out["dgate"] = z(grads[3], gt)
    return out


def selective_scan_grads(x, dt, A, Bm, Cm, dy, Dskip=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
                         dh_last=None):
    """Gradients of the batched selective scan for the loss sum(dy * y) + sum(dh_last * h_last).
    Shapes: x, dt, z, dy [B,L,D]; A [D,N]; Bm, Cm [B,L,N]; Dskip, dt_bias [D]; h0, dh_last [B,D,N].
    Returns a dict of float64 arrays: dx, ddt [B,L,D], dA [D,N], dBm, dCm [B,L,N], dh0 [B,D,N], and
    dDskip, dz, ddt_bias for the optional inputs that are given."""
    import torch
    F = torch.nn.functional
    xs, dts, As, Bs, Cs = _t(x), _t(dt), _t(A), _t(Bm), _t(Cm)
    Ds, zs, dbs = _t(Dskip), _t(z), _t(dt_bias)
    B, L, D = xs.shape
    N = As.shape[1]
    h = _t(h0) if h0 is not None else torch.zeros((B, D, N), dtype=torch.float64, requires_grad=True)
    h_init = h
    v = dts + dbs if dbs is not None else dts
    delta = F.softplus(v) if dt_softplus else v
    ys = []
    for t in range(L):
        abar = torch.exp((delta[:, t, :, None] * As[None]).clamp(max=20))
        h = abar * h + (delta[:, t, :, None] * Bs[:, t, None, :]) * xs[:, t, :, None]
        y_t = (h * Cs[:, t, None, :]).sum(-1)
        if Ds is not None:
            y_t = y_t + xs[:, t] * Ds
        if zs is not None:
            y_t = y_t * F.silu(zs[:, t])
        ys.append(y_t)
    y = torch.stack(ys, dim=1) if L > 0 else torch.zeros((B, 0, D), dtype=torch.float64)
    loss = (y * torch.as_tensor(np.asarray(dy, dtype=np.float64))).sum()
    if dh_last is not None:
        loss = loss + (h * torch.as_tensor(np.asarray(dh_last, dtype=np.float64))).sum()
    names = ["dx", "ddt", "dA", "dBm", "dCm", "dh0"]
    inputs = [xs, dts, As, Bs, Cs, h_init]
    for nm, tsr in (("dDskip", Ds), ("dz", zs), ("ddt_bias", dbs)):
        if tsr is not None:
            names.append(nm)
            inputs.append(tsr)
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    return {nm: (np.zeros(tsr.shape) if g is None else g.detach().numpy()) for nm, g, tsr in zip(names, grads, inputs)}


def hgrn2_scan_grads(q, k, v, g_logit, lower_bound, do, S0=None, dS_last=None):
    """Gradients of the HGRN2 scan (frankenstein-transformer documentation, "HGRN2 Attention": the gate
    g = lb + (1 - lb) sigmoid(g_logit) scales row i of the state, S[i][j] = g_i S[i][j] + v_i k_j, and
    the readout is o_i = sum_j S[i][j] q_j including the current token) for the loss
    sum(do * o) + sum(dS_last * S_last).  Shapes: q, k, v, g_logit, do [B,L,H,d]; S0, dS_last [B,H,d,d].
    Returns float64 dq, dk, dv, dg_logit [B,L,H,d] and dS0 [B,H,d,d] (of a zero state when S0 is None)."""
    import torch
    qs, ks, vs, gs = _t(q), _t(k), _t(v), _t(g_logit)
    B, L, H, d = qs.shape
    S = _t(S0) if S0 is not None else torch.zeros((B, H, d, d), dtype=torch.float64, requires_grad=True)
    S_init = S
    lb = float(lower_bound)
    os_ = []
    for t in range(L):
        g = lb + (1.0 - lb) * torch.sigmoid(gs[:, t])                          # [B,H,d] over rows i
        S = g[..., :, None] * S + vs[:, t, :, :, None] * ks[:, t, :, None, :]  # row i scaled, v_i k_j added
        os_.append((S * qs[:, t, :, None, :]).sum(-1))                        # o_i = sum_j S[i][j] q_j
    o = torch.stack(os_, dim=1) if L > 0 else torch.zeros((B, 0, H, d), dtype=torch.float64)
    loss = (o * torch.as_tensor(np.asarray(do, dtype=np.float64))).sum()
    if dS_last is not None:
        loss = loss + (S * torch.as_tensor(np.asarray(dS_last, dtype=np.float64))).sum()
    inputs = [qs, ks, vs, gs, S_init]
    grads = torch.autograd.grad(loss, inputs, allow_unused=True)
    names = ["dq", "dk", "dv", "dg_logit", "dS0"]
    return {nm: (np.zeros(tsr.shape) if g is None else g.detach().numpy()) for nm, g, tsr in zip(names, grads, inputs)}
