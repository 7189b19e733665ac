"""GPU parity on the edges of the kernels' paths that ordinary draws do not reach, through the C ABI,
against the fp64 oracle:
  * softplus's threshold: delta = dt + dt_bias exactly above 20 (torch's softplus), forward and gradients,
    up to arguments where e^v overflows fp32;
  * the chunked MFMA form of HGRN2 where its decay check binds: gates saturated at the lower bound over
    whole chunks, at bounds where the in-chunk decay stays above 2^-96 (just above 2^-1.5) and where it
    does not (0.2, 0), so chunks go token by token; every chunk token by token; a NaN gate;
  * the decode steps at the benchmark shapes (HGRN2 B = 8, H = 16, d = 128 with either gate axis) and
    the selective decode step at B = 1 and with fp32 inputs.
Tolerances as everywhere: max|err| <= tau * RMS(oracle), tau = 1e-5 (fp32 inputs) or 2e-2 (bf16)."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from oracle import grad as og
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu

# dt + dt_bias of the threshold channels: below and above 20 (at least 1.5 away, so fp32 and fp64 sums
# fall on the same side), and far above, where e^v is not finite in fp32
THRESHOLD_V = np.array([17.0, 18.5, 21.5, 23.0, 50.0, 100.0, 300.0, 1000.0], dtype=np.float32)


def _set_dt(inp, dtype, ch, values_by_row):
    """dt[:, :, ch] = values (one value per row, cycled), stored in the input dtype."""
    B, L, D = inp.t["dt"].shape
    vals = np.resize(values_by_row, L).astype(np.float32)
    if dtype == synth.BF16:
        inp.t["dt"].data[:, :, ch] = synth.f32_to_bf16_bits(np.broadcast_to(vals, (B, L)).copy())
    else:
        inp.t["dt"].data[:, :, ch] = vals


def threshold_inputs(dtype, seed, B=2, L=150, D=64, N=16):
    inp = synth.selective_inputs(B, L, D, N, dtype, seed, with_h0=True)
    bias = np.linspace(-0.4, 0.4, D).astype(np.float32)
    inp.p["dt_bias"] = bias
    # channel c < 8: every row at THRESHOLD_V[c]; channels 8..15: rows cycle through all of them
    for c in range(8):
        _set_dt(inp, dtype, c, np.array([THRESHOLD_V[c] - bias[c]]))
    for c in range(8, 16):
        _set_dt(inp, dtype, c, np.roll(THRESHOLD_V, c) - bias[c])
    return inp


def run_selective(inp, dtype):
    t = {n: to_dev(v) for n, v in inp.t.items()}
    return ssd.selective_scan(t["x"], t["dt"], to_dev(inp.p["A"]), t["Bm"], t["Cm"], Dskip=to_dev(inp.p["Dskip"]),
                              z=t["z"], dt_bias=to_dev(inp.p["dt_bias"]), h0=to_dev(inp.p["h0"]),
                              return_last_state=True)


def oracle_selective(inp):
    t = inp.t
    return oracle.selective_scan(f64(t["x"]), f64(t["dt"]), f64(inp.p["A"]), f64(t["Bm"]), f64(t["Cm"]),
                                 Dskip=f64(inp.p["Dskip"]), z=f64(t["z"]), dt_bias=f64(inp.p["dt_bias"]),
                                 h0=f64(inp.p["h0"]))


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_selective_softplus_threshold_forward(dtype):
    import torch
    inp = threshold_inputs(dtype, 9100)
    y, hl = run_selective(inp, dtype)
    torch.cuda.synchronize()
    yr, hr = oracle_selective(inp)
    assert_close(host(y), yr, TOL[dtype], "y")
    assert_close(host(hl), hr, TOL[dtype], "h_last")
    # the threshold channels alone, on their own scale, and the ordinary channels on theirs
    assert_close(host(y)[:, :, :16], yr[:, :, :16], TOL[dtype], "y threshold channels")
    assert_close(host(y)[:, :, 16:], yr[:, :, 16:], TOL[dtype], "y other channels")


def test_selective_softplus_threshold_backward_fp32():
    import torch
    inp = threshold_inputs(synth.F32, 9200, B=2, L=70, D=40, N=8)
    B, L, D = inp.t["x"].shape
    rng = np.random.default_rng(9201)
    dy = rng.standard_normal((B, L, D)).astype(np.float32)
    dhl = rng.standard_normal((B, D, 8)).astype(np.float32)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    G = ssd.selective_scan_backward(t["x"], t["dt"], to_dev(inp.p["A"]), t["Bm"], t["Cm"], to_dev(dy),
                                    Dskip=to_dev(inp.p["Dskip"]), z=t["z"], dt_bias=to_dev(inp.p["dt_bias"]),
                                    h0=to_dev(inp.p["h0"]), dh_last=to_dev(dhl))
    torch.cuda.synchronize()
    R = og.selective_scan_grads(f64(inp.t["x"]), f64(inp.t["dt"]), f64(inp.p["A"]), f64(inp.t["Bm"]),
                                f64(inp.t["Cm"]), dy.astype(np.float64), Dskip=f64(inp.p["Dskip"]), z=f64(inp.t["z"]),
                                dt_bias=f64(inp.p["dt_bias"]), h0=f64(inp.p["h0"]), dh_last=dhl.astype(np.float64))
    for name in R:
        assert_close(host(G[name]), R[name], TOL[synth.F32], name)
    # per-channel gradients of the threshold channels on their own scale
    assert_close(host(G["ddt"])[:, :, :16], R["ddt"][:, :, :16], TOL[synth.F32], "ddt threshold channels")
    assert_close(host(G["ddt_bias"])[:16], R["ddt_bias"][:16], TOL[synth.F32], "ddt_bias threshold channels")


def test_selective_update_softplus_threshold():
    import torch
    inp = threshold_inputs(synth.F32, 9300, B=3, L=12, D=64)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    state = to_dev(inp.p["h0"]).clone()
    ys = [ssd.selective_update(t["x"][:, s].contiguous(), t["dt"][:, s].contiguous(), to_dev(inp.p["A"]),
                               t["Bm"][:, s].contiguous(), t["Cm"][:, s].contiguous(), state,
                               Dskip=to_dev(inp.p["Dskip"]), z=t["z"][:, s].contiguous(),
                               dt_bias=to_dev(inp.p["dt_bias"])) for s in range(12)]
    torch.cuda.synchronize()
    yr, hr = oracle_selective(inp)
    assert_close(host(torch.stack(ys, 1)), yr, TOL[synth.F32], "decode y")
    assert_close(host(state), hr, TOL[synth.F32], "decode state")


# ----------------------------------------------------------------------------- HGRN2 numeric guard
def saturated_hgrn2(seed, lb=0.36, B=2, L=200, H=3):
    inp = synth.hgrn2_inputs(B, L, H, 128, synth.BF16, seed, lower_bound=lb, with_S0=True)
    g = synth.bf16_to_f32(inp.t["g_logit"].data).copy()
    g[:, 64:128] = -30.0                     # chunk 1: every gate at the bound, all heads
    g[:, 128:192, :, ::2] = -30.0            # chunk 2: half the channels saturated
    g[0, :, 1] = -30.0                       # one whole head saturated over the whole sequence
    inp.t["g_logit"] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g))
    return inp


@pytest.mark.parametrize("lb", [0.36, 0.354, 0.2, 0.0])
def test_hgrn2_chunked_form_with_saturated_gates(lb):
    """bf16 inputs with d = 128 take the chunked MFMA form at any lower bound.  Gates saturated at the
    bound over a chunk give in-chunk decays down to lb^64: 2^-94.3 at 0.36 and 2^-95.9 at 0.354 (the
    products' range still holds), 2^-148.6 at 0.2 and about 10^-830 at 0 (the chunk goes token by token).
    Chunk 0 has ordinary gates, so every sequence mixes the two ways through a chunk."""
    import torch
    inp = saturated_hgrn2(9400 + int(lb * 1000), lb=lb)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    o, S = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], lb, S0=to_dev(inp.p["S0"]), return_last_state=True)
    torch.cuda.synchronize()
    orf, Sr = oracle.hgrn2_scan(f64(inp.t["q"]), f64(inp.t["k"]), f64(inp.t["v"]), f64(inp.t["g_logit"]), lb,
                                f64(inp.p["S0"]))
    assert_close(host(o), orf, TOL[synth.BF16], "o")
    assert_close(host(S), Sr, TOL[synth.BF16], "S_last")
    # each head on its own scale (the saturated head's outputs are small)
    for b in range(o.shape[0]):
        for h in range(o.shape[2]):
            assert_close(host(o[b, :, h]), orf[b, :, h], TOL[synth.BF16], f"o head {b},{h}")


def test_hgrn2_chunked_form_all_chunks_token_by_token():
    """Every gate at the bound 0 (logit -30 everywhere): every chunk of every head fails the decay check;
    with an S0 and a ragged last chunk."""
    import torch
    inp = synth.hgrn2_inputs(2, 64 * 3 + 9, 2, 128, synth.BF16, 9450, lower_bound=0.0, with_S0=True)
    g = np.full(inp.t["g_logit"].shape, -30.0, dtype=np.float32)
    g[:, :, :, 5] = 3.0  # one channel with gates near 1 keeps a long memory
    inp.t["g_logit"] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g))
    t = {n: to_dev(v) for n, v in inp.t.items()}
    o, S = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.0, S0=to_dev(inp.p["S0"]), return_last_state=True)
    torch.cuda.synchronize()
    orf, Sr = oracle.hgrn2_scan(f64(inp.t["q"]), f64(inp.t["k"]), f64(inp.t["v"]), f64(inp.t["g_logit"]), 0.0,
                                f64(inp.p["S0"]))
    assert_close(host(o), orf, TOL[synth.BF16], "o")
    assert_close(host(S), Sr, TOL[synth.BF16], "S_last")


def test_hgrn2_chunked_form_nan_gate_propagates():
    """A NaN gate logit makes its value row NaN from that token on, as in the recurrence; other rows and
    heads keep the oracle's values."""
    import torch
    inp = synth.hgrn2_inputs(1, 150, 2, 128, synth.BF16, 9460, lower_bound=0.5)
    g = synth.bf16_to_f32(inp.t["g_logit"].data).copy()
    g[0, 70, 1, 9] = np.nan
    inp.t["g_logit"] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g))
    t = {n: to_dev(v) for n, v in inp.t.items()}
    o = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5)
    torch.cuda.synchronize()
    oh = host(o)
    orf, _ = oracle.hgrn2_scan(f64(inp.t["q"]), f64(inp.t["k"]), f64(inp.t["v"]), f64(inp.t["g_logit"]), 0.5)
    assert np.all(np.isnan(oh[0, 70:, 1, 9])) and np.all(np.isnan(orf[0, 70:, 1, 9]))
    mask = np.ones(oh.shape, dtype=bool)
    mask[0, 70:, 1, 9] = False
    assert_close(oh[mask], orf[mask], TOL[synth.BF16], "o outside the NaN row")


# ----------------------------------------------------------------------------- decode at the benchmark shapes
@pytest.mark.parametrize("gate_axis", ["value", "key"])
def test_hgrn2_update_benchmark_shape(gate_axis):
    """B = 8, H = 16, d = 128: the decode kernel's lanes each walk two value rows (d = 128)."""
    import torch
    B, H, d, steps = 8, 16, 128, 6
    inp = synth.hgrn2_inputs(B, steps, H, d, synth.BF16, 9500 + len(gate_axis), with_S0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    S = to_dev(inp.p["S0"]).clone()
    outs = [ssd.hgrn2_update(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(), t["v"][:, s].contiguous(),
                             t["g_logit"][:, s].contiguous(), 0.5, S, gate_axis=gate_axis) for s in range(steps)]
    o_scan, S_scan = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5, S0=to_dev(inp.p["S0"]),
                                    return_last_state=True, gate_axis=gate_axis)
    torch.cuda.synchronize()
    fn = oracle.hgrn2_scan if gate_axis == "value" else oracle.hgrn2_key_scan
    orf, Sr = fn(*(f64(inp.t[n]) for n in ("q", "k", "v", "g_logit")), 0.5, f64(inp.p["S0"]))
    assert_close(host(torch.stack(outs, 1)), orf, TOL[synth.BF16], "decode o")
    assert_close(host(S), Sr, TOL[synth.BF16], "decode S")
    # the scans at d = 128 with bf16 inputs (either gate axis, lower bound 0.5) run the chunked MFMA form,
    # whose derived operands are bf16 hi/lo pairs (about 16 significant bits, 2^-16 = 1.5e-5 relative per
    # product); the decode steps are fp32 register arithmetic
    assert_close(host(torch.stack(outs, 1)), host(o_scan), 1e-4, "decode o vs scan")
    assert_close(host(S), host(S_scan), 1e-4, "decode S vs scan")


@pytest.mark.parametrize("B,dtype", [(1, synth.BF16), (1, synth.F32), (4, synth.F32)])
def test_selective_update_batch_one_and_fp32(B, dtype):
    import torch
    L, D, N = 20, 200, 16
    inp = synth.selective_inputs(B, L, D, N, dtype, 9600 + B, with_h0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    A, Dskip, h0 = to_dev(inp.p["A"]), to_dev(inp.p["Dskip"]), to_dev(inp.p["h0"])
    state = h0.clone()
    ys = [ssd.selective_update(t["x"][:, s].contiguous(), t["dt"][:, s].contiguous(), A, t["Bm"][:, s].contiguous(),
                               t["Cm"][:, s].contiguous(), state, Dskip=Dskip, z=t["z"][:, s].contiguous())
          for s in range(L)]
    torch.cuda.synchronize()
    yr, hr = oracle.selective_scan(f64(inp.t["x"]), f64(inp.t["dt"]), f64(inp.p["A"]), f64(inp.t["Bm"]),
                                   f64(inp.t["Cm"]), Dskip=f64(inp.p["Dskip"]), z=f64(inp.t["z"]), h0=f64(inp.p["h0"]))
    assert_close(host(torch.stack(ys, 1)), yr, TOL[dtype], "decode y")
    assert_close(host(state), hr, TOL[dtype], "decode state")
