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

The loss whose gradient is returned is  sum(dy * y) + sum(dh_last * h_last) (x_last for MinMax).
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
