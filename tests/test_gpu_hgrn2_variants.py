"""GPU parity of the HGRN2 variants against the fp64 oracle (pinned in tests/test_oracle_variants.py),
through the C ABI: the key-axis-gated scan and decode step, and the readout LayerNorm with silu gate.
Tolerance: max|err| <= tau * RMS(oracle), tau = 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


def key_check(B, L, H, d, dtype, seed, lb=0.5, with_S0=True):
    import torch
    inp = synth.hgrn2_inputs(B, L, H, d, dtype, seed, lower_bound=lb, with_S0=with_S0)
    t = inp.t
    o, S = ssd.hgrn2_scan(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), to_dev(t["g_logit"]), lb,
                          S0=to_dev(inp.p.get("S0")), return_last_state=True, gate_axis="key")
    torch.cuda.synchronize()
    orf, Sr = oracle.hgrn2_key_scan(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["g_logit"]), lb, f64(inp.p.get("S0")))
    assert_close(host(o), orf, TOL[dtype], "o")
    assert_close(host(S), Sr, TOL[dtype], "S_last")
    return o, S


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_key_gated_head_dims_fp32(d):
    key_check(2, 45, 2, d, synth.F32, 8000 + d)


@pytest.mark.parametrize("lb", [0.0, 0.5, 1.0])
def test_key_gated_lower_bounds_bf16(lb):
    key_check(2, 200, 2, 128, synth.BF16, 8100 + int(10 * lb), lb=lb)


@pytest.mark.parametrize("L", [1, 7, 8, 9, 130])
def test_key_gated_ragged_without_state(L):
    key_check(1, L, 3, 64, synth.BF16, 8200 + L, with_S0=False)


def test_key_gated_bf16_output():
    """bf16 output = the fp32 result rounded (both outputs come from the same fp32 arithmetic), within 1 ulp."""
    import torch
    inp = synth.hgrn2_inputs(2, 100, 2, 128, synth.BF16, 8300, with_S0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    args = (t["q"], t["k"], t["v"], t["g_logit"], 0.5)
    o32 = ssd.hgrn2_scan(*args, S0=to_dev(inp.p["S0"]), gate_axis="key")
    o16 = ssd.hgrn2_scan(*args, S0=to_dev(inp.p["S0"]), gate_axis="key", out_dtype=torch.bfloat16)
    diff = (o16.float() - o32.to(torch.bfloat16).float()).abs()
    assert bool((diff <= o32.abs().clamp_min(1e-30) * 2.0 ** -7).all())


def test_key_gated_decode_steps_equal_scan():
    import torch
    B, L, H, d = 2, 12, 3, 64
    inp = synth.hgrn2_inputs(B, L, H, d, synth.BF16, 8400, with_S0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    o, S_last = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5, S0=to_dev(inp.p["S0"]),
                               return_last_state=True, gate_axis="key")
    S = to_dev(inp.p["S0"]).clone()
    Sr = f64(inp.p["S0"])
    for s in range(L):
        os_ = ssd.hgrn2_update(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(), t["v"][:, s].contiguous(),
                               t["g_logit"][:, s].contiguous(), 0.5, S, gate_axis="key")
        orf, Sr = oracle.hgrn2_key_update(*(f64(inp.t[n])[:, s] for n in ("q", "k", "v", "g_logit")), 0.5, Sr)
        torch.cuda.synchronize()
        assert_close(host(os_), orf, 2e-2, f"o step {s}")
        assert_close(host(os_), host(o[:, s]), 1e-5, f"o step {s} vs scan")
    assert_close(host(S), Sr, 2e-2, "S")
    assert_close(host(S), host(S_last), 1e-5, "S vs scan")


def test_key_gated_full_workload_sampled_heads():
    """B=8, L=4096, H=16, d=128 bf16: every head on the GPU, 64 heads checked against the oracle alone."""
    import torch
    from tests.test_gpu_hgrn2 import _full_size_heads
    inp = synth.workload_inputs("hgrn2")
    t = inp.t
    o = ssd.hgrn2_scan(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), to_dev(t["g_logit"]), 0.5, gate_axis="key")
    torch.cuda.synchronize()
    assert _full_size_heads(inp, o, None, fn=oracle.hgrn2_key_scan) == 64


@pytest.mark.parametrize("width", [1, 37, 128, 256, 2048, 3000])
@pytest.mark.parametrize("gated", [False, True])
def test_readout_norm(width, gated):
    import torch
    rng = np.random.default_rng(8500 + width + gated)
    rows = 33
    o = (rng.standard_normal((rows, width)) * 2.0 + 0.7).astype(np.float32)
    w = rng.standard_normal(width).astype(np.float32)
    b = rng.standard_normal(width).astype(np.float32)
    g32 = rng.standard_normal((rows, width)).astype(np.float32)
    gate = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g32)) if gated else None
    y = ssd.readout_norm(to_dev(o), gate=to_dev(gate) if gated else None, weight=to_dev(w), bias=to_dev(b))
    torch.cuda.synchronize()
    ref = oracle.readout_norm(o.astype(np.float64), gate=f64(gate) if gated else None, weight=w.astype(np.float64),
                              bias=b.astype(np.float64))
    assert_close(host(y), ref, 1e-5, "y")


def test_readout_norm_over_hidden_of_scan_output():
    """The layer's use: the scan's fp32 output [B, L, H, d] normalised over its H * d hidden features."""
    import torch
    B, L, H, d = 2, 50, 4, 64
    inp = synth.hgrn2_inputs(B, L, H, d, synth.BF16, 8600, with_S0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    o = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5, S0=to_dev(inp.p["S0"]))
    gate = torch.randn((B, L, H * d), device="cuda").to(torch.bfloat16)
    w = torch.randn(H * d, device="cuda")
    bvec = torch.randn(H * d, device="cuda")
    y = ssd.readout_norm(o.view(B, L, H * d), gate=gate, weight=w, bias=bvec)
    y16 = ssd.readout_norm(o.view(B, L, H * d), gate=gate, weight=w, bias=bvec, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # the norm's own error, on the scan output it is given (fp32 throughout)
    ref = oracle.readout_norm(host(o).reshape(B, L, H * d), gate=host(gate), weight=host(w), bias=host(bvec))
    assert_close(host(y), ref, 1e-5, "y")
    # bf16 output: the fp32 result rounded, within 1 ulp
    diff = (y16.float() - y.to(torch.bfloat16).float()).abs()
    assert bool((diff <= y.abs().clamp_min(1e-30) * 2.0 ** -7).all())


@pytest.mark.parametrize("width", [64, 100, 2048])
def test_readout_norm_fp32_gate_without_affine(width):
    import torch
    rng = np.random.default_rng(8700 + width)
    rows = 20
    o = (rng.standard_normal((rows, width)) * 0.5 - 3.0).astype(np.float32)
    g = rng.standard_normal((rows, width)).astype(np.float32)
    y = ssd.readout_norm(to_dev(o), gate=to_dev(g), eps=1e-3)
    y0 = ssd.readout_norm(to_dev(o), eps=1e-3)
    torch.cuda.synchronize()
    assert_close(host(y), oracle.readout_norm(o.astype(np.float64), gate=g.astype(np.float64), eps=1e-3), 1e-5, "y")
    assert_close(host(y0), oracle.readout_norm(o.astype(np.float64), eps=1e-3), 1e-5, "y0")


def test_variants_deterministic_and_nan_propagating():
    """Runs repeat bit for bit; a NaN in one head's input stays in that head (key gate) or row (norm)."""
    import torch
    inp = synth.hgrn2_inputs(2, 40, 3, 64, synth.BF16, 8800, with_S0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    S0 = to_dev(inp.p["S0"])
    o1 = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5, S0=S0, gate_axis="key")
    o2 = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5, S0=S0, gate_axis="key")
    assert torch.equal(o1, o2)
    v = t["v"].clone()
    v[1, 5, 2, 7] = float("nan")
    o3 = ssd.hgrn2_scan(t["q"], t["k"], v, t["g_logit"], 0.5, S0=S0, gate_axis="key")
    torch.cuda.synchronize()
    bad = torch.isnan(o3)
    assert bool(bad[1, 5:, 2, 7].all())          # row 7 of head (1, 2) from token 5 on
    assert not bool(bad[0].any()) and not bool(bad[1, :, :2].any())  # other heads untouched
    assert torch.equal(o3[0], o1[0])
    x = torch.randn((6, 256), device="cuda")
    n1, n2 = ssd.readout_norm(x), ssd.readout_norm(x)
    assert torch.equal(n1, n2)
    x[3, 10] = float("nan")
    n3 = ssd.readout_norm(x)
    assert bool(torch.isnan(n3[3]).all()) and not bool(torch.isnan(n3[[0, 1, 2, 4, 5]]).any())
