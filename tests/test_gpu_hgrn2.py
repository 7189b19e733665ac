"""GPU parity of the HGRN2 kernels against the fp64 oracle (through the C ABI).

Tolerance: max|err| <= tau * RMS(oracle), tau = 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs, fp32
state), on every output element and on S_last."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, parallel_map, spread_heads, to_dev

pytestmark = pytest.mark.gpu


def gpu_run(inp, out_dtype=None):
    t = inp.t
    return ssd.hgrn2_scan(to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"]), to_dev(t["g_logit"]),
                          inp.s["lower_bound"], S0=to_dev(inp.p.get("S0")), return_last_state=True,
                          out_dtype=out_dtype)


def oracle_run(inp):
    t = inp.t
    return oracle.hgrn2_scan(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["g_logit"]), inp.s["lower_bound"],
                             f64(inp.p.get("S0")))


def check(inp, tol):
    import torch
    o, S = gpu_run(inp)
    torch.cuda.synchronize()
    orf, Sr = oracle_run(inp)
    assert_close(host(o), orf, tol, "o")
    assert_close(host(S), Sr, tol, "S_last")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_head_dims_fp32(d):
    check(synth.hgrn2_inputs(2, 70, 3, d, synth.F32, d, with_S0=True), TOL[synth.F32])


@pytest.mark.parametrize("lb", [0.0, 0.5, 0.9, 1.0])
def test_lower_bounds_bf16(lb):
    check(synth.hgrn2_inputs(2, 200, 2, 128, synth.BF16, 5, lower_bound=lb, with_S0=True), TOL[synth.BF16])


@pytest.mark.parametrize("L", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths(L, d):
    # d = 128 with bf16 inputs and lower bound 0.5 runs the chunked MFMA form; d = 64 the recurrent one
    check(synth.hgrn2_inputs(1, L, 4, d, synth.BF16, 100 + L, with_S0=True), TOL[synth.BF16])


@pytest.mark.parametrize("B,H", [(1, 3), (3, 8)])
def test_chunked_form_head_mappings(B, H):
    # B*H not a multiple of 8 and a multiple of 8 take the two workgroup-to-head mappings
    check(synth.hgrn2_inputs(B, 150, H, 128, synth.BF16, 7 * B + H, with_S0=True), TOL[synth.BF16])


def test_decode_steps_equal_scan():
    import torch
    B, L, H, d = 2, 20, 3, 64
    inp = synth.hgrn2_inputs(B, L, H, d, synth.BF16, 7, with_S0=True)
    t = {k: to_dev(v) for k, v in inp.t.items()}
    S = to_dev(inp.p["S0"]).clone()
    outs = [ssd.hgrn2_update(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(), t["v"][:, s].contiguous(),
                             t["g_logit"][:, s].contiguous(), 0.5, S) for s in range(L)]
    torch.cuda.synchronize()
    orf, Sr = oracle_run(inp)
    assert_close(host(torch.stack(outs, 1)), orf, TOL[synth.BF16], "decode o")
    assert_close(host(S), Sr, TOL[synth.BF16], "decode S")


def test_bf16_output():
    import torch
    inp = synth.hgrn2_inputs(1, 100, 2, 128, synth.BF16, 8)
    o32, _ = gpu_run(inp)
    o16, _ = gpu_run(inp, out_dtype=torch.bfloat16)
    diff = (o16.float() - o32.to(torch.bfloat16).float()).abs()
    assert bool((diff <= o32.abs().clamp_min(1e-30) * 2.0 ** -7).all())


def _full_size_heads(inp, o, S, fn=None):
    """Every output and the final state of 64 heads (spread_heads) vs the oracle run on each head alone."""
    B, L, H, d = inp.t["q"].shape
    fn = fn or oracle.hgrn2_scan
    oh, Sh = o.cpu().double().numpy(), S.cpu().double().numpy() if S is not None else None
    pairs = spread_heads(B, H)

    def run(bh):
        b, h = bh
        g = lambda n: synth.bf16_to_f64(inp.t[n].data[b:b + 1, :, h:h + 1])
        return fn(g("q"), g("k"), g("v"), g("g_logit"), inp.s["lower_bound"])

    for (b, h), (orf, Sr) in zip(pairs, parallel_map(run, pairs)):
        assert_close(oh[b:b + 1, :, h:h + 1], orf, TOL[synth.BF16], f"o head {b},{h}")
        if Sh is not None:
            assert_close(Sh[b:b + 1, h:h + 1], Sr, TOL[synth.BF16], f"S head {b},{h}")
    return len(pairs)


def test_hgrn2_workload_full_size_sampled_heads():
    """B=8, H=16, d=128, L=4096 bf16 at full size (the chunked MFMA form): every output and the final
    state of 64 heads (four batch rows of both parities, every head index) vs the oracle."""
    import torch
    inp = synth.workload_inputs("hgrn2")
    o, S = gpu_run(inp)
    torch.cuda.synchronize()
    assert _full_size_heads(inp, o, S) == 64
    assert torch.isfinite(o).all()


def test_full_size_default_lower_bound_sampled_heads():
    """The same workload with the page's default lower bound 0: 64 heads and their final states."""
    import torch
    inp = synth.workload_inputs("hgrn2")
    inp.s["lower_bound"] = 0.0
    o, S = gpu_run(inp)
    torch.cuda.synchronize()
    assert _full_size_heads(inp, o, S) == 64
    assert torch.isfinite(o).all()
