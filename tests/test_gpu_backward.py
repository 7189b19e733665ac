"""GPU parity of the RG-LRU backward kernels against the gradient oracle (float64 autograd over the
sequential forward, pinned to finite differences in tests/test_oracle_grad.py), called through the
C ABI.  Tolerance per gradient tensor, as for the forward: max|err| <= tau * RMS(oracle gradient),
tau = 1e-5 for fp32 inputs and 2e-2 for bf16 inputs; d a_log, a sum over batch and time, is checked
to the same relative bound.  Where boundary states put some elements tens of times above the RMS, fp32
gradients are checked element by element: |err| <= tau * max(|oracle|, RMS)."""
import numpy as np
import pytest

import selective_state_space_diag_amd as ssd
from oracle import grad as og
from selective_state_space_diag_amd import synth
from tests.helpers import assert_close, assert_close_elem, f64, host, to_dev

pytestmark = pytest.mark.gpu
TOLB = {synth.F32: 1e-5, synth.BF16: 2e-2}


def run_bwd(B, L, D, dtype, seed, gated=False, with_h0=True, with_dhl=True):
    import torch
    inp = synth.rglru_inputs(B, L, D, dtype, seed, with_h0=with_h0, with_gate=gated)
    rng = np.random.default_rng(seed + 7)
    dy32 = rng.standard_normal((B, L, D)).astype(np.float32)
    dy = synth.Tensor(dtype, synth.f32_to_bf16_bits(dy32)) if dtype == synth.BF16 else synth.Tensor(dtype, dy32)
    dhl = rng.standard_normal((B, D)).astype(np.float32) if with_dhl else None
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    G = ssd.rglru_scan_backward(x, r, i, to_dev(inp.p["a_log"]), 8.0, to_dev(dy), h0=to_dev(inp.p.get("h0")),
                                gate=to_dev(inp.t["gate"]) if gated else None, dh_last=to_dev(dhl))
    torch.cuda.synchronize()
    R = og.rglru_scan_grads(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]), 8.0,
                            f64(dy), h0=f64(inp.p.get("h0")), gate=f64(inp.t["gate"]) if gated else None,
                            dh_last=None if dhl is None else dhl.astype(np.float64))
    for name in ("dx", "dr_logit", "di_logit", "da_log", "dh0") + (("dgate",) if gated else ()):
        assert_close(host(G[name]), R[name], TOLB[dtype], name)
    return G


def test_backward_fp32_small():
    run_bwd(2, 128, 64, synth.F32, 4000)


@pytest.mark.parametrize("L,D", [(1, 64), (63, 65), (64, 130), (65, 128), (200, 257)])
def test_backward_bf16_ragged(L, D):
    run_bwd(2, L, D, synth.BF16, 4100 + L + D)


def test_backward_gated_fp32_long_chain():
    run_bwd(1, 64 * 9 + 11, 96, synth.F32, 4200, gated=True)


def test_backward_gated_bf16_no_state_inputs():
    run_bwd(3, 150, 192, synth.BF16, 4300, gated=True, with_h0=False, with_dhl=False)


def test_backward_deterministic_and_bf16_output():
    import torch
    inp = synth.rglru_inputs(2, 300, 256, synth.BF16, 4400, with_h0=True)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    dy = torch.randn((2, 300, 256), device="cuda").to(torch.bfloat16)
    args = (x, r, i, to_dev(inp.p["a_log"]), 8.0, dy)
    g1 = ssd.rglru_scan_backward(*args, h0=to_dev(inp.p["h0"]))
    g2 = ssd.rglru_scan_backward(*args, h0=to_dev(inp.p["h0"]))
    g16 = ssd.rglru_scan_backward(*args, h0=to_dev(inp.p["h0"]), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    for k in ("dx", "dr_logit", "di_logit"):
        assert torch.equal(g16[k], g1[k].to(torch.bfloat16)), k


def test_backward_empty_sequence():
    import torch
    x = torch.empty((2, 0, 8), device="cuda")
    dhl = torch.randn((2, 8), device="cuda")
    a_log = torch.full((8,), -0.05, device="cuda")
    g = ssd.rglru_scan_backward(x, x, x, a_log, 8.0, x, dh_last=dhl)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dhl) and torch.all(g["da_log"] == 0)


# ----------------------------------------------------------------------------- MinMax
def run_mm_bwd(B, L, D, dtype, seed, gated=False, with_x0=True, with_dxl=True, ties=False, nan_at=()):
    inp = synth.minmax_inputs(B, L, D, dtype, seed, with_x0=with_x0, with_gate=gated, ties=ties)
    for name, idx in nan_at:  # plant NaN inputs (the forward carries them; torch's rule routes gradients)
        inp.t[name].data[idx] = 0x7FC0 if dtype == synth.BF16 else np.nan
    rng = np.random.default_rng(seed + 7)
    dy32 = rng.standard_normal((B, L, D)).astype(np.float32)
    dy = synth.Tensor(dtype, synth.f32_to_bf16_bits(dy32)) if dtype == synth.BF16 else synth.Tensor(dtype, dy32)
    dxl = rng.standard_normal((B, D)).astype(np.float32) if with_dxl else None
    import torch
    G = ssd.minmax_scan_backward(to_dev(inp.t["r"]), to_dev(inp.t["s"]), to_dev(dy), x0=to_dev(inp.p.get("x0")),
                                 gate=to_dev(inp.t["gate"]) if gated else None, dx_last=to_dev(dxl))
    torch.cuda.synchronize()
    R = og.minmax_scan_grads(f64(inp.t["r"]), f64(inp.t["s"]), f64(dy), x0=f64(inp.p.get("x0")),
                             gate=f64(inp.t["gate"]) if gated else None,
                             dx_last=None if dxl is None else dxl.astype(np.float64))
    names = ("dr", "ds", "dx0") + (("dgate",) if gated else ())
    for name in names:
        got, want = host(G[name]), R[name]
        if nan_at:
            assert np.array_equal(np.isnan(got), np.isnan(want)), name
            keep = ~np.isnan(want)
            got, want = got[keep], want[keep]
        assert_close(got, want, TOLB[dtype], name)
    return G


def test_minmax_backward_fp32_gated():
    run_mm_bwd(2, 64 * 5 + 9, 130, synth.F32, 5000, gated=True)


@pytest.mark.parametrize("L,D", [(1, 64), (63, 65), (64, 130), (65, 128), (300, 257)])
def test_minmax_backward_bf16_ragged(L, D):
    run_mm_bwd(2, L, D, synth.BF16, 5100 + L + D)


def test_minmax_backward_ties_split_the_gradient():
    """Inputs drawn from {-2, -1, -0, +0, 1, 2}: equal operands at every other step."""
    run_mm_bwd(2, 64 * 6 + 5, 96, synth.F32, 5200, gated=True, ties=True)
    run_mm_bwd(1, 200, 64, synth.BF16, 5201, ties=True, with_x0=False, with_dxl=False)


def test_minmax_backward_nan_inputs():
    run_mm_bwd(2, 64 * 3 + 1, 64, synth.F32, 5300, gated=True, nan_at=[("r", (0, 70, 3)), ("s", (1, 150, 9))])


def test_minmax_backward_deterministic_and_bf16_output():
    import torch
    inp = synth.minmax_inputs(2, 300, 256, synth.BF16, 5400, with_x0=True, with_gate=True)
    r, s, gt = (to_dev(inp.t[n]) for n in ("r", "s", "gate"))
    dy = torch.randn((2, 300, 256), device="cuda").to(torch.bfloat16)
    g1 = ssd.minmax_scan_backward(r, s, dy, x0=to_dev(inp.p["x0"]), gate=gt)
    g2 = ssd.minmax_scan_backward(r, s, dy, x0=to_dev(inp.p["x0"]), gate=gt)
    g16 = ssd.minmax_scan_backward(r, s, dy, x0=to_dev(inp.p["x0"]), gate=gt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    for k in ("dr", "ds", "dgate"):
        assert torch.equal(g16[k], g1[k].to(torch.bfloat16)), k


def test_minmax_backward_empty_sequence():
    import torch
    r = torch.empty((2, 0, 8), device="cuda")
    dxl = torch.randn((2, 8), device="cuda")
    g = ssd.minmax_scan_backward(r, r, r, dx_last=dxl)
    torch.cuda.synchronize()
    assert torch.equal(g["dx0"], dxl)


# ----------------------------------------------------------------------------- saved chunk states
@pytest.mark.parametrize("dtype,L,D", [(synth.F32, 64 * 3 + 7, 130), (synth.BF16, 64 * 5, 257)])
def test_rglru_chunk_states_match_oracle_and_feed_backward(dtype, L, D):
    import torch
    import oracle
    B = 2
    inp = synth.rglru_inputs(B, L, D, dtype, 6000 + L, with_h0=True, with_gate=True)
    x, r, i, g = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit", "gate"))
    a_log, h0 = to_dev(inp.p["a_log"]), to_dev(inp.p["h0"])
    cs = torch.full(ssd.chunk_states_shape(B, L, D), float("nan"), device="cuda")
    ssd.rglru_scan(x, r, i, a_log, 8.0, h0=h0, gate=g, chunk_states=cs)
    torch.cuda.synchronize()
    # the state entering chunk k is h_{64k - 1} (h0 for k = 0): the ungated oracle's output there
    y_ref, _ = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                                 8.0, h0=f64(inp.p["h0"]))
    want = np.concatenate([f64(inp.p["h0"])[:, None, :], y_ref[:, 63:L - 1:64, :]], axis=1)
    assert want.shape == tuple(cs.shape)
    assert_close(host(cs), want, TOLB[dtype], "chunk_states")
    dy = torch.randn((B, L, D), device="cuda").to(x.dtype)
    args = (x, r, i, a_log, 8.0, dy)
    g1 = ssd.rglru_scan_backward(*args, h0=h0, gate=g, chunk_states=cs)
    g2 = ssd.rglru_scan_backward(*args, h0=h0, gate=g)
    torch.cuda.synchronize()
    for k in g2:
        assert torch.equal(g1[k], g2[k]), k


def test_minmax_chunk_states_exact_and_feed_backward():
    import torch
    import oracle
    B, L, D = 2, 64 * 4 + 3, 96
    inp = synth.minmax_inputs(B, L, D, synth.BF16, 6100, with_x0=True, with_gate=True, ties=True)
    r, s, g = (to_dev(inp.t[n]) for n in ("r", "s", "gate"))
    x0 = to_dev(inp.p["x0"])
    cs = torch.full(ssd.chunk_states_shape(B, L, D), float("nan"), device="cuda")
    ssd.minmax_scan(r, s, x0=x0, gate=g, chunk_states=cs)
    torch.cuda.synchronize()
    y_ref, _ = oracle.minmax_scan(f64(inp.t["r"]), f64(inp.t["s"]), x0=f64(inp.p["x0"]))
    want = np.concatenate([f64(inp.p["x0"])[:, None, :], y_ref[:, 63:L - 1:64, :]], axis=1)
    assert np.array_equal(host(cs), want)  # every MinMax state is one of the inputs
    dy = torch.randn((B, L, D), device="cuda").to(torch.bfloat16)
    g1 = ssd.minmax_scan_backward(r, s, dy, x0=x0, gate=g, chunk_states=cs)
    g2 = ssd.minmax_scan_backward(r, s, dy, x0=x0, gate=g)
    torch.cuda.synchronize()
    for k in g2:
        assert torch.equal(g1[k], g2[k]), k


# ----------------------------------------------------------------------------- selective scan
def run_sel_bwd(B, L, D, N, dtype, seed, softplus=True, with_z=True, with_skip=True, with_bias=True, with_h0=True,
                with_dhl=True, A=None, edit=None, tol=None, elem=False):
    import torch
    inp = synth.selective_inputs(B, L, D, N, dtype, seed, dt_softplus=softplus, with_z=with_z, with_skip=with_skip,
                                 with_h0=with_h0)
    rng = np.random.default_rng(seed + 7)
    if A is not None:
        inp.p["A"] = A.astype(np.float32)
    if edit is not None:
        edit(inp)
    bias = (rng.standard_normal(D) * 0.1).astype(np.float32) if with_bias else None
    dy32 = rng.standard_normal((B, L, D)).astype(np.float32)
    dy = synth.Tensor(dtype, synth.f32_to_bf16_bits(dy32)) if dtype == synth.BF16 else synth.Tensor(dtype, dy32)
    dhl = rng.standard_normal((B, D, N)).astype(np.float32) if with_dhl else None
    t = {n: to_dev(inp.t[n]) for n in inp.t}
    G = ssd.selective_scan_backward(t["x"], t["dt"], to_dev(inp.p["A"]), t["Bm"], t["Cm"], to_dev(dy),
                                    Dskip=to_dev(inp.p.get("Dskip")), z=t.get("z"), dt_bias=to_dev(bias),
                                    dt_softplus=softplus, h0=to_dev(inp.p.get("h0")), dh_last=to_dev(dhl))
    torch.cuda.synchronize()
    R = og.selective_scan_grads(f64(inp.t["x"]), f64(inp.t["dt"]), f64(inp.p["A"]), f64(inp.t["Bm"]),
                                f64(inp.t["Cm"]), f64(dy), Dskip=f64(inp.p.get("Dskip")),
                                z=f64(inp.t["z"]) if with_z else None, dt_bias=f64(bias), dt_softplus=softplus,
                                h0=f64(inp.p.get("h0")), dh_last=None if dhl is None else dhl.astype(np.float64))
    check = assert_close_elem if elem else assert_close
    for name in R:
        check(host(G[name]), R[name], TOLB[dtype] if tol is None else tol, name)
    return G


def test_selective_backward_fp32_ragged():
    # 100 rows = a unit of 64 and a ragged one of 36; 300 channels = two channel blocks, the second ragged
    run_sel_bwd(2, 100, 300, 16, synth.F32, 7000)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("L", [64, 65, 127, 168, 200, 304])
def test_selective_backward_unit_shapes(dtype, L):
    """Units of 64 rows worked in 16-row sub-blocks: whole units, a one-row unit, and last units of 63, 40
    (three sub-blocks, the last of 8 rows), 8 and 48 rows, over up to five units.  fp32 gradients are held
    to 1e-5 of each element's own magnitude (the RMS for elements below it): the first row takes the full
    weight of h0 ~ N(0, 1) and the last that of dh_last ~ N(0, 1), which puts some of their d dt at 30-160
    times the RMS, and fp32 computes those to a few 1e-7 of their value (as every other element) -- an
    RMS-relative bound would ask them for ~1e-7."""
    run_sel_bwd(2, L, 320, 16, dtype, 7050 + L, elem=dtype == synth.F32)


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_selective_backward_small_n(N):
    run_sel_bwd(2, 37, 96, N, synth.F32, 7100 + N, with_bias=N % 2 == 0, with_h0=N > 2)


@pytest.mark.parametrize("L", [1, 16, 17])
def test_selective_backward_short_sequences(L):
    run_sel_bwd(3, L, 64, 16, synth.F32, 7200 + L)


def test_selective_backward_bf16_raw_dt_no_gate():
    run_sel_bwd(2, 64 * 3, 256, 8, synth.BF16, 7300, softplus=False, with_z=False, with_skip=False, with_bias=False,
                with_h0=False, with_dhl=False)


def test_selective_backward_clamp_active():
    """Channels with positive A and one large step, where delta A exceeds 20 on some states (clamped,
    no gradient through the exponent) and not on another; elsewhere delta = 1e-3 keeps the growth small
    (the state is multiplied by e^20 once).  Tolerance 1e-4 RMS: before the clamped step the gradient
    terms of the states are e^20 larger than the sums they cancel into (each element is within a few
    1e-6 of its own magnitude); a wrong clamp mask errs by O(1)."""
    D, N, L = 64, 4, 40
    A = -np.tile(np.arange(1, N + 1, dtype=np.float64), (D, 1))
    hot = np.arange(0, D, 7)
    A[hot, :] = [60.0, 30.0, 100.0, 2.0]

    def edit(inp):
        dt = inp.t["dt"].data  # raw delta (softplus off), fp32
        dt[:, :, hot] = 1e-3
        dt[:, 20, hot] = 0.8   # delta A = 48, 24, 80, 1.6: states 0, 1, 2 clamped, state 3 not

    run_sel_bwd(1, L, D, N, synth.F32, 7400, softplus=False, with_bias=False, A=A, with_dhl=False, edit=edit,
                tol=1e-4)


def test_selective_backward_deterministic_and_bf16_output():
    import torch
    inp = synth.selective_inputs(2, 96, 320, 16, synth.BF16, 7500, with_h0=True)
    t = {n: to_dev(inp.t[n]) for n in inp.t}
    dy = torch.randn((2, 96, 320), device="cuda").to(torch.bfloat16)
    args = (t["x"], t["dt"], to_dev(inp.p["A"]), t["Bm"], t["Cm"], dy)
    kw = dict(Dskip=to_dev(inp.p["Dskip"]), z=t["z"], h0=to_dev(inp.p["h0"]))
    g1 = ssd.selective_scan_backward(*args, **kw)
    g2 = ssd.selective_scan_backward(*args, **kw)
    g16 = ssd.selective_scan_backward(*args, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    for k in ("dx", "ddt", "dz", "dBm", "dCm"):
        assert torch.equal(g16[k], g1[k].to(torch.bfloat16)), k


def test_selective_backward_empty_sequence():
    import torch
    x = torch.empty((2, 0, 8), device="cuda")
    bm = torch.empty((2, 0, 4), device="cuda")
    A = -torch.ones((8, 4), device="cuda")
    dhl = torch.randn((2, 8, 4), device="cuda")
    g = ssd.selective_scan_backward(x, x, A, bm, bm, x, Dskip=torch.ones(8, device="cuda"), dh_last=dhl)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dhl) and torch.all(g["dA"] == 0) and torch.all(g["dDskip"] == 0)


def test_selective_backward_full_width_bf16():
    """All 1536 channels of the headline workload (6 channel blocks summed for dB / dC), its multi-scale
    A, softplus steps, gate and skip, over 256 steps."""
    run_sel_bwd(2, 256, 1536, 16, synth.BF16, 7600)



def test_selective_backward_varlen_matches_per_sequence_oracle():
    """Packed sequences (incl. empty and single-row ones) are independent (reading R7): the reference is
    the gradient oracle run on each sequence alone, compared per sequence (against that sequence's RMS:
    a one-row sequence's gradients are ~100x the others'); dA, dDskip and ddt_bias add over the
    sequences."""
    import torch
    lengths = [37, 0, 1, 64, 100, 16, 17]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    L, D, N = int(cu[-1]), 96, 16
    inp = synth.selective_inputs(1, L, D, N, synth.F32, 7700, cu_seqlens=cu, with_h0=True)
    rng = np.random.default_rng(7707)
    bias = (rng.standard_normal(D) * 0.1).astype(np.float32)
    dy = rng.standard_normal((1, L, D)).astype(np.float32)
    nseq = len(lengths)
    dhl = rng.standard_normal((nseq, D, N)).astype(np.float32)
    t = {n: to_dev(inp.t[n]) for n in inp.t}
    G = ssd.selective_scan_backward(t["x"], t["dt"], to_dev(inp.p["A"]), t["Bm"], t["Cm"], to_dev(dy),
                                    Dskip=to_dev(inp.p["Dskip"]), z=t["z"], dt_bias=to_dev(bias),
                                    h0=to_dev(inp.p["h0"]), dh_last=to_dev(dhl), cu_seqlens=cu)
    torch.cuda.synchronize()
    pooled = {k: 0.0 for k in ("dA", "dDskip", "ddt_bias")}
    for sq in range(nseq):
        a, b = int(cu[sq]), int(cu[sq + 1])
        if b == a:
            assert np.array_equal(host(G["dh0"])[sq], dhl[sq].astype(np.float64)), "empty sequence: dh0 = dh_last"
            continue
        sl = lambda arr: f64(arr)[:, a:b]
        R = og.selective_scan_grads(sl(inp.t["x"]), sl(inp.t["dt"]), f64(inp.p["A"]), sl(inp.t["Bm"]),
                                    sl(inp.t["Cm"]), dy[:, a:b].astype(np.float64), Dskip=f64(inp.p["Dskip"]),
                                    z=sl(inp.t["z"]), dt_bias=bias.astype(np.float64), h0=f64(inp.p["h0"])[sq:sq + 1],
                                    dh_last=dhl[sq:sq + 1].astype(np.float64))
        for k in ("dx", "ddt", "dBm", "dCm", "dz"):
            assert_close(host(G[k])[:, a:b], R[k], TOLB[synth.F32], f"{k} of sequence {sq}")
        assert_close(host(G["dh0"])[sq], R["dh0"][0], TOLB[synth.F32], f"dh0 of sequence {sq}")
        for k in pooled:
            pooled[k] = pooled[k] + R[k]
    for k, v in pooled.items():
        assert_close(host(G[k]), v, TOLB[synth.F32], k)
