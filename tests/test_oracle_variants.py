"""Pins of the oracle's HGRN2 variants (key-axis gating, readout LayerNorm with silu gate) against
what fixes them independently: the row-gated oracle on transposed roles, a brute-force sum over
per-(t, j) gate products, the lb = 1 reduction to linear attention, decode steps, and torch's
layer_norm."""
import numpy as np
import pytest

import oracle


def _case(seed, B=2, L=7, H=2, d=5, lb=0.3):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, L, H, d)) for _ in range(3))
    g = rng.standard_normal((B, L, H, d)) + 1.0
    S0 = rng.standard_normal((B, H, d, d))
    return q, k, v, g, S0, lb


def test_key_gating_state_is_transposed_row_gating():
    """S[i][j] = g_j S[i][j] + v_i k_j is the transpose of the row-gated recurrence with v and k
    exchanged: (S^T)[j][i] = g_j (S^T)[j][i] + k_j v_i."""
    q, k, v, g, S0, lb = _case(61)
    _, S_key = oracle.hgrn2_key_scan(q, k, v, g, lb, S0=S0)
    _, S_row = oracle.hgrn2_scan(q, v, k, g, lb, S0=np.swapaxes(S0, -1, -2).copy())
    assert np.allclose(S_key, np.swapaxes(S_row, -1, -2), rtol=1e-13, atol=1e-13)


def test_key_gating_readout_brute_force():
    q, k, v, g, S0, lb = _case(62, B=1, L=6, H=1, d=4)
    o, _ = oracle.hgrn2_key_scan(q, k, v, g, lb, S0=S0)
    gate = lb + (1 - lb) / (1 + np.exp(-g[0, :, 0]))  # [L, d] over the key index j
    L = q.shape[1]
    want = np.zeros((L, 4))
    for t in range(L):
        for i in range(4):
            acc = 0.0
            for s in range(t + 1):
                for j in range(4):
                    acc += v[0, s, 0, i] * np.prod(gate[s + 1:t + 1, j]) * k[0, s, 0, j] * q[0, t, 0, j]
            for j in range(4):
                acc += np.prod(gate[:t + 1, j]) * S0[0, 0, i, j] * q[0, t, 0, j]
            want[t, i] = acc
    assert np.allclose(o[0, :, 0], want, rtol=1e-12, atol=1e-12)


def test_key_gating_without_decay_equals_row_gating():
    q, k, v, g, S0, _ = _case(63)
    ok, Sk = oracle.hgrn2_key_scan(q, k, v, g, 1.0, S0=S0)
    orr, Sr = oracle.hgrn2_scan(q, k, v, g, 1.0, S0=S0)
    assert np.allclose(ok, orr, rtol=1e-13, atol=1e-13) and np.allclose(Sk, Sr, rtol=1e-13, atol=1e-13)
    # and the two readings differ once the gate acts
    ok2, _ = oracle.hgrn2_key_scan(q, k, v, g, 0.3, S0=S0)
    orr2, _ = oracle.hgrn2_scan(q, k, v, g, 0.3, S0=S0)
    assert np.max(np.abs(ok2 - orr2)) > 1e-3


def test_key_gating_decode_steps_equal_scan():
    q, k, v, g, S0, lb = _case(64)
    o, S_last = oracle.hgrn2_key_scan(q, k, v, g, lb, S0=S0)
    S = S0.copy()
    for t in range(q.shape[1]):
        ot, S = oracle.hgrn2_key_update(q[:, t], k[:, t], v[:, t], g[:, t], lb, S)
        assert np.allclose(ot, o[:, t], rtol=1e-13, atol=1e-13)
    assert np.allclose(S, S_last, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("affine,gated", [(False, False), (True, False), (True, True)])
def test_readout_norm_is_torch_layer_norm_times_silu(affine, gated):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(65)
    rows, width = 6, 48
    o = rng.standard_normal((rows, width)) * 3.0 + 1.5
    w = rng.standard_normal(width) if affine else None
    b = rng.standard_normal(width) if affine else None
    gate = rng.standard_normal((rows, width)) if gated else None
    y = oracle.readout_norm(o, gate=gate, weight=w, bias=b, eps=1e-5)
    tt = lambda a: None if a is None else torch.from_numpy(a)
    ref = torch.nn.functional.layer_norm(tt(o), (width,), tt(w), tt(b), eps=1e-5)
    if gated:
        ref = ref * torch.nn.functional.silu(tt(gate))
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_readout_norm_constant_row_gives_bias():
    o = np.full((2, 8), 3.25)
    b = np.arange(8.0)
    y = oracle.readout_norm(o, weight=np.full(8, 7.0), bias=b)
    assert np.array_equal(y, np.broadcast_to(b, (2, 8)))
