"""Seeded random shapes against the fp64 oracle, through the C ABI: the selective scan (state sizes
1..16, optional h0 / z / skip), the HGRN2 scan with both gate axes at several lower bounds, and the
HGRN2 backward on the smaller draws.  Each case draws batch, length (1..299, so ragged against every
tile), width and dtype; the bound is the one of the fixed-shape tests (1e-5 of RMS for fp32 inputs,
2e-2 for bf16)."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from oracle import grad as og
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


def _draw(case):
    rng = np.random.default_rng(4242 + 97 * case)
    dt_ = synth.BF16 if rng.random() < 0.6 else synth.F32
    return rng, dt_, int(rng.integers(1, 4)), int(rng.integers(1, 300)), int(rng.integers(1 << 30))


@pytest.mark.parametrize("case", range(12))
def test_selective_random_shape(case):
    import torch
    rng, dt_, B, L, seed = _draw(case)
    D, N = int(rng.integers(1, 300)), int(rng.choice([1, 2, 4, 8, 16]))
    s = synth.selective_inputs(B, L, D, N, dt_, seed, with_h0=bool(rng.random() < 0.5),
                               with_z=bool(rng.random() < 0.7), with_skip=bool(rng.random() < 0.7))
    t, p = s.t, s.p
    print(f"selective case {case}: B={B} L={L} D={D} N={N} {dt_}", flush=True)
    y, hl = ssd.selective_scan(to_dev(t["x"]), to_dev(t["dt"]), to_dev(p["A"]), to_dev(t["Bm"]), to_dev(t["Cm"]),
                               Dskip=to_dev(p.get("Dskip")), z=to_dev(t.get("z")), h0=to_dev(p.get("h0")),
                               return_last_state=True)
    torch.cuda.synchronize()
    yr, hr = oracle.selective_scan(f64(t["x"]), f64(t["dt"]), f64(p["A"]), f64(t["Bm"]), f64(t["Cm"]),
                                   Dskip=f64(p.get("Dskip")), z=f64(t.get("z")), h0=f64(p.get("h0")))
    assert_close(host(y), yr, TOL[dt_], "y")
    assert_close(host(hl), hr, TOL[dt_], "h_last")


@pytest.mark.parametrize("case", range(12))
def test_hgrn2_random_shape(case):
    import torch
    rng, dt_, B, L, seed = _draw(case + 1000)
    H, d = int(rng.integers(1, 4)), int(rng.choice([16, 32, 64, 128]))
    lb = float(rng.choice([0.0, 0.3, 0.5, 0.9, 1.0]))
    h = synth.hgrn2_inputs(B, L, H, d, dt_, seed, lower_bound=lb, with_S0=bool(rng.random() < 0.5))
    ht = {k: to_dev(v) for k, v in h.t.items()}
    print(f"hgrn2 case {case}: B={B} L={L} H={H} d={d} lb={lb} {dt_}", flush=True)
    for axis, orf in (("value", oracle.hgrn2_scan), ("key", oracle.hgrn2_key_scan)):
        o, S = ssd.hgrn2_scan(ht["q"], ht["k"], ht["v"], ht["g_logit"], lb, S0=to_dev(h.p.get("S0")),
                              return_last_state=True, gate_axis=axis)
        torch.cuda.synchronize()
        orr, Sr = orf(f64(h.t["q"]), f64(h.t["k"]), f64(h.t["v"]), f64(h.t["g_logit"]), lb, f64(h.p.get("S0")))
        assert_close(host(o), orr, TOL[dt_], f"o ({axis} gate)")
        assert_close(host(S), Sr, TOL[dt_], f"S_last ({axis} gate)")
    if L <= 80 and d <= 64:
        do = (rng.standard_normal((B, L, H, d)) / np.sqrt(d)).astype(np.float32)
        dod = to_dev(do).to(torch.bfloat16 if dt_ == synth.BF16 else torch.float32)
        G = ssd.hgrn2_scan_backward(ht["q"], ht["k"], ht["v"], ht["g_logit"], lb, dod, S0=to_dev(h.p.get("S0")))
        torch.cuda.synchronize()
        R = og.hgrn2_scan_grads(f64(h.t["q"]), f64(h.t["k"]), f64(h.t["v"]), f64(h.t["g_logit"]), lb, host(dod),
                                S0=f64(h.p.get("S0")))
        for n in ("dq", "dk", "dv", "dg_logit", "dS0"):
            assert_close(host(G[n]), R[n], TOL[dt_], n)
