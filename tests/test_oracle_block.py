"""Pins of the oracle's RG-LRU block pieces (causal depthwise convolution, gelu output gate) and of
its MinMax recurrence, against what the pages and the mathematics fix.

Each check compares the oracle with something it does not share code with: textbook values of the
normal distribution function, numpy's own convolution, running maxima and minima, an O(L^2)
unrolled lattice formula, or invariants (split and decode equal the full scan; every MinMax state
is one of the inputs).
"""
import math

import numpy as np
import pytest

import oracle

# Standard normal distribution function at 1 and 2 (printed normal tables)
PHI_1 = 0.8413447460685429
PHI_2 = 0.9772498680518208


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


# ============================================================================ gelu output gate
def test_gelu_is_x_times_normal_cdf():
    assert abs(oracle.gelu(1.0) - PHI_1) < 1e-15
    assert abs(oracle.gelu(2.0) - 2.0 * PHI_2) < 2e-15
    assert abs(oracle.gelu(-1.0) - (-(1.0 - PHI_1))) < 1e-15
    assert oracle.gelu(0.0) == 0.0
    for v in (0.3, 1.7, 4.0):  # gelu(v) - gelu(-v) = v (Phi(v) + Phi(-v) = 1)
        assert abs(oracle.gelu(v) - oracle.gelu(-v) - v) < 1e-14


def _rglru_inputs(rng, B, L, D):
    x, r, i, g = (rng.standard_normal((B, L, D)) for _ in range(4))
    a_log = np.log(rng.uniform(0.9, 0.999, size=D))
    return x, r, i, a_log, g


def test_rglru_gate_scales_output_only():
    rng = np.random.default_rng(11)
    x, r, i, a_log, g = _rglru_inputs(rng, 2, 37, 5)
    h0 = rng.standard_normal((2, 5))
    y, hl = oracle.rglru_scan(x, r, i, a_log, 8.0, h0=h0)
    yg, hlg = oracle.rglru_scan(x, r, i, a_log, 8.0, h0=h0, gate=g)
    gel = np.vectorize(oracle.gelu)(g)
    assert rel(yg, gel * y) < 1e-15
    assert np.array_equal(hl, hlg)  # the carried state is the ungated h
    # gate = 0 silences the output; a large gate passes it through (gelu(v) -> v)
    y0, _ = oracle.rglru_scan(x, r, i, a_log, 8.0, h0=h0, gate=np.zeros_like(g))
    assert np.all(y0 == 0.0)
    y8, _ = oracle.rglru_scan(x, r, i, a_log, 8.0, h0=h0, gate=np.full_like(g, 10.0))
    assert rel(y8, 10.0 * y) < 1e-15


def test_rglru_gated_decode_equals_gated_scan():
    rng = np.random.default_rng(12)
    x, r, i, a_log, g = _rglru_inputs(rng, 3, 9, 4)
    y, hl = oracle.rglru_scan(x, r, i, a_log, 8.0, gate=g)
    st = np.zeros((3, 4))
    for t in range(9):
        yt, st = oracle.rglru_update(x[:, t], r[:, t], i[:, t], a_log, 8.0, st, gate=g[:, t])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(st, hl)


# ============================================================================ MinMax recurrence
def _ints(rng, shape, lo=-6, hi=6):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def test_minmax_open_upper_bound_is_running_max():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((2, 50, 3))
    x0 = rng.standard_normal((2, 3))
    y, xl = oracle.minmax_scan(np.full_like(s, np.inf), s, x0=x0)
    want = np.maximum.accumulate(np.concatenate([x0[:, None, :], s], axis=1), axis=1)[:, 1:]
    assert np.array_equal(y, want)
    assert np.array_equal(xl, want[:, -1])


def test_minmax_open_lower_bound_is_running_min():
    rng = np.random.default_rng(2)
    r = rng.standard_normal((2, 50, 3))
    x0 = rng.standard_normal((2, 3))
    y, _ = oracle.minmax_scan(r, np.full_like(r, -np.inf), x0=x0)
    want = np.minimum.accumulate(np.concatenate([x0[:, None, :], r], axis=1), axis=1)[:, 1:]
    assert np.array_equal(y, want)


def test_minmax_unrolled_lattice_formula():
    """x_t = max over k in {-1..t} of min(v_k, r_{k+1}, ..., r_t), with v_{-1} = x0, v_k = s_k."""
    rng = np.random.default_rng(3)
    for trial in range(20):
        L = int(rng.integers(1, 25))
        r, s = _ints(rng, (1, L, 1)), _ints(rng, (1, L, 1))
        x0 = _ints(rng, (1, 1))
        y, _ = oracle.minmax_scan(r, s, x0=x0)
        for t in range(L):
            terms = []
            for k in range(-1, t + 1):
                v = x0[0, 0] if k < 0 else s[0, k, 0]
                terms.append(min([v] + [r[0, j, 0] for j in range(k + 1, t + 1)]))
            assert y[0, t, 0] == max(terms), (trial, t)


def test_minmax_states_are_inputs_and_zero_default_state():
    rng = np.random.default_rng(4)
    r, s = rng.standard_normal((2, 40, 6)), rng.standard_normal((2, 40, 6))
    y, _ = oracle.minmax_scan(r, s)
    for b in range(2):
        for d in range(6):
            allowed = set(r[b, :, d]) | set(s[b, :, d]) | {0.0}
            assert set(y[b, :, d]) <= allowed
    y2, _ = oracle.minmax_scan(r, s, x0=np.zeros((2, 6)))
    assert np.array_equal(y, y2)


def test_minmax_split_decode_and_gate():
    rng = np.random.default_rng(5)
    r, s, g = _ints(rng, (2, 30, 4)), _ints(rng, (2, 30, 4)), rng.standard_normal((2, 30, 4))
    x0 = _ints(rng, (2, 4))
    y, xl = oracle.minmax_scan(r, s, x0=x0)
    y1, x1 = oracle.minmax_scan(r[:, :11], s[:, :11], x0=x0)
    y2, x2 = oracle.minmax_scan(r[:, 11:], s[:, 11:], x0=x1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y) and np.array_equal(x2, xl)
    st = x0.copy()
    for t in range(30):
        yt, st = oracle.minmax_update(r[:, t], s[:, t], st)
        assert np.array_equal(yt, y[:, t])
    yg, xg = oracle.minmax_scan(r, s, x0=x0, gate=g)
    assert np.array_equal(yg, y * g) and np.array_equal(xg, xl)
    ygt, _ = oracle.minmax_update(r[:, 0], s[:, 0], x0, gate=g[:, 0])
    assert np.array_equal(ygt, y[:, 0] * g[:, 0])


def test_minmax_signed_zero_and_nan_readings():
    one = lambda v: np.array(v, dtype=np.float64).reshape(1, -1, 1)
    # -0 orders below +0: min(-0, +0) = -0, max(-0, +0) = +0
    y, _ = oracle.minmax_scan(one([-0.0]), one([-np.inf]), x0=np.array([[0.0]]))
    assert y[0, 0, 0] == 0.0 and math.copysign(1.0, y[0, 0, 0]) < 0
    y, _ = oracle.minmax_scan(one([np.inf]), one([0.0]), x0=np.array([[-0.0]]))
    assert y[0, 0, 0] == 0.0 and math.copysign(1.0, y[0, 0, 0]) > 0
    # a NaN operand makes the state NaN from that step on
    y, xl = oracle.minmax_scan(one([1.0, np.nan, 3.0, 4.0]), one([0.0, 0.0, 0.0, 0.0]))
    assert y[0, 0, 0] == 0.0 and np.all(np.isnan(y[0, 1:, 0])) and np.isnan(xl[0, 0])


# ============================================================================ causal convolution
def _conv_inputs(rng, B, L, D, W):
    return rng.standard_normal((B, L, D)), rng.standard_normal((D, W)), rng.standard_normal(D)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_conv_matches_numpy_convolve(W):
    rng = np.random.default_rng(20 + W)
    B, L, D = 2, 23, 5
    x, w, bias = _conv_inputs(rng, B, L, D, W)
    y, st = oracle.causal_conv1d(x, w, bias)
    for b in range(B):
        for d in range(D):
            want = np.convolve(x[b, :, d], w[d][::-1])[:L] + bias[d]
            assert rel(y[b, :, d], want) < 1e-14
            hist = np.concatenate([np.zeros(W), x[b, :, d]])
            assert np.array_equal(st[b, d], hist[-W:])


def test_conv_history_is_the_preceding_inputs():
    rng = np.random.default_rng(30)
    B, L, D, W = 2, 9, 3, 4
    x, w, bias = _conv_inputs(rng, B, L, D, W)
    hist = rng.standard_normal((B, D, W))
    y, st = oracle.causal_conv1d(x, w, bias, state_in=hist)
    for b in range(B):
        for d in range(D):
            seq = np.concatenate([hist[b, d], x[b, :, d]])
            want = np.convolve(seq, w[d][::-1])[W:W + L] + bias[d]
            assert rel(y[b, :, d], want) < 1e-14
            assert np.array_equal(st[b, d], seq[-W:])
    # a sequence shorter than the window keeps part of the history in the new window
    ys, sts = oracle.causal_conv1d(x[:, :2], w, bias, state_in=hist)
    assert np.array_equal(sts[:, :, :2], hist[:, :, 2:]) and np.array_equal(sts[:, :, 2:], np.moveaxis(x[:, :2], 1, 2))


def test_conv_identity_and_shift_weights():
    rng = np.random.default_rng(31)
    B, L, D, W = 2, 12, 3, 4
    x, _, bias = _conv_inputs(rng, B, L, D, W)
    last = np.zeros((D, W)); last[:, W - 1] = 1.0
    y, _ = oracle.causal_conv1d(x, last, bias)
    assert np.array_equal(y, x + bias)
    first = np.zeros((D, W)); first[:, 0] = 1.0
    y, _ = oracle.causal_conv1d(x, first)
    assert np.array_equal(y[:, W - 1:], x[:, :L - W + 1]) and np.all(y[:, :W - 1] == 0.0)


def test_conv_split_and_decode_equal_full_scan():
    rng = np.random.default_rng(32)
    B, L, D, W = 2, 17, 3, 4
    x, w, bias = _conv_inputs(rng, B, L, D, W)
    hist = rng.standard_normal((B, D, W))
    y, st = oracle.causal_conv1d(x, w, bias, state_in=hist)
    y1, s1 = oracle.causal_conv1d(x[:, :6], w, bias, state_in=hist)
    y2, s2 = oracle.causal_conv1d(x[:, 6:], w, bias, state_in=s1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y) and np.array_equal(s2, st)
    win = hist.copy()
    for t in range(L):
        yt, win = oracle.causal_conv1d_update(x[:, t], w, win, bias=bias)
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(win, st)
