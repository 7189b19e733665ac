"""GPU parity of the HGRN2 backward sweeps against the gradient oracle (float64 autograd over the
sequential row-gated forward, pinned in tests/test_oracle_grad.py), called through the C ABI.
Tolerance per gradient tensor: max|err| <= tau * RMS(oracle gradient), tau = 1e-5 for fp32 inputs
and 2e-2 for bf16 inputs (fp32 state and accumulation)."""
import numpy as np
import pytest

import selective_state_space_diag_amd as ssd
from oracle import grad as og
from selective_state_space_diag_amd import synth
from tests.helpers import assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu
TOLB = {synth.F32: 1e-5, synth.BF16: 2e-2}
NAMES = ("dq", "dk", "dv", "dg_logit", "dS0")


def make(B, L, H, d, dtype, seed, lb=0.5, with_S0=True, with_dSl=True):
    inp = synth.hgrn2_inputs(B, L, H, d, dtype, seed, lower_bound=lb, with_S0=with_S0)
    rng = np.random.default_rng(seed + 11)
    do32 = (rng.standard_normal((B, L, H, d)) / np.sqrt(d)).astype(np.float32)
    do = synth.Tensor(dtype, synth.f32_to_bf16_bits(do32)) if dtype == synth.BF16 else synth.Tensor(dtype, do32)
    dSl = (rng.standard_normal((B, H, d, d)) * 0.1).astype(np.float32) if with_dSl else None
    return inp, do, dSl


def gpu_grads(inp, do, dSl, o=None, out_dtype=None):
    import torch
    t = inp.t
    G = ssd.hgrn2_scan_backward(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), to_dev(t["g_logit"]),
                                inp.s["lower_bound"], to_dev(do), S0=to_dev(inp.p.get("S0")), dS_last=to_dev(dSl),
                                o=o, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return G


def oracle_grads(inp, do, dSl):
    t = inp.t
    return og.hgrn2_scan_grads(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["g_logit"]), inp.s["lower_bound"],
                               f64(do), S0=f64(inp.p.get("S0")), dS_last=None if dSl is None else f64(dSl))


def check(B, L, H, d, dtype, seed, **kw):
    inp, do, dSl = make(B, L, H, d, dtype, seed, **kw)
    G = gpu_grads(inp, do, dSl)
    R = oracle_grads(inp, do, dSl)
    for n in NAMES:
        assert_close(host(G[n]), R[n], TOLB[dtype], n)
    return G


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_head_dims_fp32(d):
    check(2, 37, 2, d, synth.F32, 7000 + d)


@pytest.mark.parametrize("lb", [0.0, 0.5, 1.0])
def test_lower_bounds_bf16(lb):
    # d = 128, bf16 and lb = 0.5 recompute the forward output with the chunked MFMA kernel
    check(2, 200, 2, 128, synth.BF16, 7100 + int(10 * lb), lb=lb)


def test_fp32_long_chain():
    check(1, 300, 2, 64, synth.F32, 7200, lb=0.2)


@pytest.mark.parametrize("L", [1, 7, 8, 9, 65])
def test_ragged_lengths_without_state_inputs(L):
    check(2, L, 3, 32, synth.BF16, 7300 + L, with_S0=False, with_dSl=False)


def test_given_forward_output_matches_recomputed():
    import torch
    inp, do, dSl = make(2, 150, 2, 128, synth.BF16, 7400)
    t = inp.t
    o = ssd.hgrn2_scan(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), to_dev(t["g_logit"]), inp.s["lower_bound"],
                       S0=to_dev(inp.p["S0"]))
    G1 = gpu_grads(inp, do, dSl, o=o)
    G2 = gpu_grads(inp, do, dSl)
    for n in NAMES:
        assert torch.equal(G1[n], G2[n]), n


def test_deterministic_and_bf16_output():
    import torch
    inp, do, dSl = make(2, 120, 2, 64, synth.BF16, 7500)
    G1 = gpu_grads(inp, do, dSl)
    G2 = gpu_grads(inp, do, dSl)
    Gb = gpu_grads(inp, do, dSl, out_dtype=torch.bfloat16)
    for n in NAMES:
        assert torch.equal(G1[n], G2[n]), n
    for n in ("dq", "dk", "dv", "dg_logit"):
        assert torch.equal(Gb[n], G1[n].to(torch.bfloat16)), n
    assert torch.equal(Gb["dS0"], G1["dS0"])


def test_empty_sequence_passes_state_gradient():
    import torch
    inp, do, dSl = make(2, 0, 2, 32, synth.BF16, 7600)
    G = gpu_grads(inp, do, dSl)
    assert G["dq"].numel() == 0
    assert torch.equal(G["dS0"].cpu(), torch.from_numpy(dSl))


def test_full_workload_sampled_heads():
    """B=8, L=4096, H=16, d=128 (bf16, lb = 0.5), the benchmark shape: every head is computed on the
    GPU; four heads (independent of the others) are checked against the oracle run on them alone."""
    B, L, H, d = 8, 4096, 16, 128
    inp = synth.workload_inputs("hgrn2")
    rng = np.random.default_rng(7700)
    do32 = (rng.standard_normal((B, L, H, d)) / np.sqrt(d)).astype(np.float32)
    do = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(do32))
    G = gpu_grads(inp, do, None)
    # four heads of both (b, h) parities and four positions modulo the 8 XCDs (the gradient oracle, a
    # float64 autograd loop over 4096 tokens, takes about ten seconds per head)
    for b, h in ((0, 0), (3, 7), (5, 10), (7, 13)):
        sub = {n: f64(inp.t[n])[b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "g_logit")}
        R = og.hgrn2_scan_grads(sub["q"], sub["k"], sub["v"], sub["g_logit"], 0.5, f64(do)[b:b + 1, :, h:h + 1])
        for n in ("dq", "dk", "dv", "dg_logit"):
            assert_close(host(G[n][b:b + 1, :, h:h + 1]), R[n], TOLB[synth.BF16], f"{n} b={b} h={h}")
        assert_close(host(G["dS0"][b:b + 1, h:h + 1]), R["dS0"], TOLB[synth.BF16], f"dS0 b={b} h={h}")
