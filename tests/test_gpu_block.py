"""GPU parity of the RG-LRU block pieces and the MinMax scan against the fp64 oracle (through the
C ABI): the gelu-gated RG-LRU output, the causal depthwise convolution and its decode window, and
the MinMax recurrence.

Tolerances: the gated RG-LRU output and the convolution use max|err| <= tau * RMS(oracle) with
tau = 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs).  The MinMax states select input values, so the
ungated MinMax output and final state must equal the oracle bit for bit (NaN where it is NaN);
a gated MinMax output is one fp32 product per element, checked to 2^-23 relative."""
import math

import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


def same_bits(gpu32, ref64, what):
    """fp32 GPU values equal the oracle's values exactly (signed zeros included; NaN where NaN)."""
    g = np.asarray(gpu32, dtype=np.float32)
    r = np.asarray(ref64, dtype=np.float64).astype(np.float32)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    ok = ~nan_r
    assert np.array_equal(g[ok].view(np.uint32), r[ok].view(np.uint32)), \
        f"{what}: {int(np.sum(g[ok].view(np.uint32) != r[ok].view(np.uint32)))} values differ"


def f32_host(t):
    return t.float().cpu().numpy()


# ============================================================================ gated RG-LRU
def run_gated(B, L, D, dtype, seed, with_h0=True):
    import torch
    inp = synth.rglru_inputs(B, L, D, dtype, seed, with_h0=with_h0, with_gate=True)
    x, r, i, g = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit", "gate"))
    a_log = to_dev(inp.p["a_log"])
    h0 = to_dev(inp.p["h0"]) if with_h0 else None
    y, hl = ssd.rglru_scan(x, r, i, a_log, 8.0, h0=h0, return_last_state=True, gate=g)
    torch.cuda.synchronize()
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                               8.0, f64(inp.p.get("h0")), gate=f64(inp.t["gate"]))
    assert_close(host(y), yr, TOL[dtype], "gated y")
    assert_close(host(hl), hr, TOL[dtype], "h_last")
    return inp, y, hl


def test_gated_rglru_fp32():
    run_gated(2, 128, 64, synth.F32, 1100, with_h0=False)


@pytest.mark.parametrize("L,D", [(1, 130), (65, 129), (300, 256), (64 * 9 + 3, 384)])
def test_gated_rglru_bf16_ragged(L, D):
    run_gated(2, L, D, synth.BF16, 1200 + L + D)


def test_gated_rglru_fp32_long():
    run_gated(1, 64 * 30 + 17, 130, synth.F32, 1300)


def test_gated_rglru_state_equals_ungated():
    import torch
    inp, yg, hg = run_gated(2, 200, 256, synth.BF16, 1400)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    y, h = ssd.rglru_scan(x, r, i, to_dev(inp.p["a_log"]), 8.0, h0=to_dev(inp.p["h0"]), return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(h, hg)


def test_gated_rglru_decode_steps():
    import torch
    B, L, D = 4, 12, 320
    inp = synth.rglru_inputs(B, L, D, synth.BF16, 1500, with_h0=True, with_gate=True)
    x, r, i, g = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit", "gate"))
    a_log = to_dev(inp.p["a_log"])
    state = to_dev(inp.p["h0"]).clone()
    ys = [ssd.rglru_update(x[:, t].contiguous(), r[:, t].contiguous(), i[:, t].contiguous(), a_log, 8.0, state,
                           gate=g[:, t].contiguous()) for t in range(L)]
    torch.cuda.synchronize()
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                               8.0, f64(inp.p["h0"]), gate=f64(inp.t["gate"]))
    assert_close(np.stack([host(v) for v in ys], axis=1), yr, TOL[synth.BF16], "decode y")
    assert_close(host(state), hr, TOL[synth.BF16], "decode state")


# ============================================================================ MinMax
def run_minmax(B, L, D, dtype, seed, with_x0=True, with_gate=False, ties=False, nan_at=None):
    import torch
    inp = synth.minmax_inputs(B, L, D, dtype, seed, with_x0=with_x0, with_gate=with_gate, ties=ties)
    r64, s64 = f64(inp.t["r"]), f64(inp.t["s"])
    rd, sd = to_dev(inp.t["r"]), to_dev(inp.t["s"])
    if nan_at is not None:  # plant NaNs in r at the given (b, t, d)
        for (b, t, d) in nan_at:
            r64[b, t, d] = np.nan
            rd[b, t, d] = float("nan")
    x0 = to_dev(inp.p["x0"]) if with_x0 else None
    g = to_dev(inp.t["gate"]) if with_gate else None
    y, xl = ssd.minmax_scan(rd, sd, x0=x0, gate=g, return_last_state=True)
    torch.cuda.synchronize()
    yr, xr = oracle.minmax_scan(r64, s64, x0=f64(inp.p.get("x0")), gate=f64(inp.t.get("gate")))
    return inp, y, xl, yr, xr


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("L,D", [(1, 64), (63, 130), (64, 129), (200, 256), (64 * 11 + 5, 1)])
def test_minmax_bitwise(dtype, L, D):
    _, y, xl, yr, xr = run_minmax(2, L, D, dtype, 2000 + L + D)
    same_bits(f32_host(y), yr, "y")
    same_bits(f32_host(xl), xr, "x_last")


def test_minmax_ties_and_signed_zeros_bitwise():
    _, y, xl, yr, xr = run_minmax(3, 64 * 7 + 9, 258, synth.BF16, 2100, ties=True)
    same_bits(f32_host(y), yr, "y")
    same_bits(f32_host(xl), xr, "x_last")
    assert np.any(np.signbit(yr) & (yr == 0.0)) and np.any(~np.signbit(yr) & (yr == 0.0))


def test_minmax_nan_propagates_from_its_step():
    _, y, xl, yr, xr = run_minmax(2, 300, 128, synth.F32, 2200, nan_at=[(0, 5, 3), (1, 250, 77), (1, 64, 0)])
    same_bits(f32_host(y), yr, "y")
    same_bits(f32_host(xl), xr, "x_last")
    yh = f32_host(y)
    assert np.all(np.isnan(yh[0, 5:, 3])) and not np.any(np.isnan(yh[0, :5, 3]))


def test_minmax_long_lookback_and_default_state():
    _, y, xl, yr, xr = run_minmax(1, 64 * 41 + 1, 512, synth.F32, 2300, with_x0=False)
    same_bits(f32_host(y), yr, "y")
    same_bits(f32_host(xl), xr, "x_last")


def test_minmax_gated():
    _, y, xl, yr, xr = run_minmax(2, 150, 192, synth.BF16, 2400, with_gate=True)
    g, r = f32_host(y).astype(np.float64), yr
    assert np.all(np.abs(g - r) <= np.abs(r) * 2.0 ** -23)
    same_bits(f32_host(xl), xr, "x_last")


def test_minmax_bf16_output_is_exact_for_bf16_states():
    import torch
    inp = synth.minmax_inputs(2, 100, 128, synth.BF16, 2500)
    y = ssd.minmax_scan(to_dev(inp.t["r"]), to_dev(inp.t["s"]), out_dtype=torch.bfloat16)
    yr, _ = oracle.minmax_scan(f64(inp.t["r"]), f64(inp.t["s"]))
    same_bits(f32_host(y), yr, "bf16 y")  # every state is a bf16 input value or the zero start


@pytest.mark.parametrize("D", [130, 131, 200])
def test_minmax_decode_steps_bitwise(D):
    import torch
    B, L = 4, 20
    inp = synth.minmax_inputs(B, L, D, synth.BF16, 2600, with_x0=True, ties=True)
    r, s = to_dev(inp.t["r"]), to_dev(inp.t["s"])
    state = to_dev(inp.p["x0"]).clone()
    ys = [ssd.minmax_update(r[:, t].contiguous(), s[:, t].contiguous(), state) for t in range(L)]
    torch.cuda.synchronize()
    yr, xr = oracle.minmax_scan(f64(inp.t["r"]), f64(inp.t["s"]), x0=f64(inp.p["x0"]))
    same_bits(np.stack([f32_host(v) for v in ys], axis=1), yr, "decode y")
    same_bits(f32_host(state), xr, "decode state")


def test_minmax_empty_sequence_copies_state():
    import torch
    r = torch.empty((2, 0, 8), device="cuda", dtype=torch.bfloat16)
    x0 = torch.randn((2, 8), device="cuda")
    y, xl = ssd.minmax_scan(r, r, x0=x0, return_last_state=True)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 8) and torch.equal(xl, x0)


# ============================================================================ causal conv1d
def run_conv(B, L, D, W, dtype, seed, with_state=True, with_bias=True):
    import torch
    inp = synth.conv_inputs(B, L, D, W, dtype, seed, with_bias=with_bias, with_state=with_state)
    x = to_dev(inp.t["x"])
    w = to_dev(inp.p["weight"])
    b = to_dev(inp.p["bias"]) if with_bias else None
    st = to_dev(inp.p["state"]) if with_state else None
    y, so = ssd.causal_conv1d(x, w, bias=b, state_in=st, return_state=True)
    torch.cuda.synchronize()
    yr, sr = oracle.causal_conv1d(f64(inp.t["x"]), f64(inp.p["weight"]), f64(inp.p.get("bias")),
                                  f64(inp.p.get("state")))
    assert_close(host(y), yr, TOL[dtype], "conv y")
    same_bits(f32_host(so), sr, "state_out")
    return inp, y, so


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_conv_widths_fp32(W):
    run_conv(2, 100, 64, W, synth.F32, 3000 + W)


@pytest.mark.parametrize("L", [1, 2, 3, 15, 16, 17, 64, 65, 333])
def test_conv_ragged_lengths_bf16(L):
    run_conv(2, L, 130, 4, synth.BF16, 3100 + L)


@pytest.mark.parametrize("D", [1, 3, 127, 257])
def test_conv_ragged_channels(D):
    run_conv(2, 90, D, 4, synth.BF16, 3200 + D, with_bias=False)
    run_conv(1, 40, D, 3, synth.F32, 3300 + D, with_state=False)


def test_conv_split_and_decode_equal_scan():
    import torch
    B, L, D, W = 2, 37, 192, 4
    inp = synth.conv_inputs(B, L, D, W, synth.BF16, 3400, with_state=True)
    x, w, b, st = to_dev(inp.t["x"]), to_dev(inp.p["weight"]), to_dev(inp.p["bias"]), to_dev(inp.p["state"])
    y, so = ssd.causal_conv1d(x, w, bias=b, state_in=st, return_state=True)
    y1, s1 = ssd.causal_conv1d(x[:, :20].contiguous(), w, bias=b, state_in=st, return_state=True)
    y2, s2 = ssd.causal_conv1d(x[:, 20:].contiguous(), w, bias=b, state_in=s1, return_state=True)
    win = st.clone()
    ys = [ssd.causal_conv1d_update(x[:, t].contiguous(), w, win, bias=b) for t in range(L)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], dim=1), y) and torch.equal(s2, so)
    assert torch.equal(torch.stack(ys, dim=1), y) and torch.equal(win, so)


def test_conv_bf16_output_rounds_fp32_result():
    import torch
    inp = synth.conv_inputs(2, 70, 128, 4, synth.BF16, 3500)
    x, w, b = to_dev(inp.t["x"]), to_dev(inp.p["weight"]), to_dev(inp.p["bias"])
    y32 = ssd.causal_conv1d(x, w, bias=b)
    y16 = ssd.causal_conv1d(x, w, bias=b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_conv_empty_sequence_copies_window():
    import torch
    x = torch.empty((2, 0, 8), device="cuda", dtype=torch.bfloat16)
    w = torch.randn((8, 4), device="cuda")
    st = torch.randn((2, 8, 4), device="cuda")
    y, so = ssd.causal_conv1d(x, w, state_in=st, return_state=True)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 8) and torch.equal(so, st)
