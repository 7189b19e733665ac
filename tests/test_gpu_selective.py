"""GPU parity of the selective-scan kernels against the fp64 oracle (through the C ABI).

Tolerance: max|err| <= tau * RMS(oracle), tau = 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs, fp32
state), on every output element and on h_last.  Full-size workloads are checked on every output
of sampled channels (exact for those channels, since channels are independent)."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, parallel_map, spread_channels, to_dev

pytestmark = pytest.mark.gpu


def gpu_run(inp, out_dtype=None, return_last_state=True):
    t = inp.t
    return ssd.selective_scan(to_dev(t["x"]), to_dev(t["dt"]), to_dev(inp.p["A"]), to_dev(t["Bm"]), to_dev(t["Cm"]),
                              Dskip=to_dev(inp.p.get("Dskip")), z=to_dev(t["z"]) if "z" in t else None,
                              dt_bias=to_dev(inp.p.get("dt_bias")), dt_softplus=inp.s["dt_softplus"],
                              cu_seqlens=inp.s.get("cu_seqlens"), h0=to_dev(inp.p.get("h0")),
                              return_last_state=return_last_state, out_dtype=out_dtype)


def oracle_run(inp):
    t = inp.t
    return oracle.selective_scan(f64(t["x"]), f64(t["dt"]), f64(inp.p["A"]), f64(t["Bm"]), f64(t["Cm"]),
                                 Dskip=f64(inp.p.get("Dskip")), z=f64(t.get("z")), dt_bias=f64(inp.p.get("dt_bias")),
                                 dt_softplus=inp.s["dt_softplus"], cu_seqlens=inp.s.get("cu_seqlens"),
                                 h0=f64(inp.p.get("h0")))


def check(inp, tol):
    import torch
    y, hl = gpu_run(inp)
    torch.cuda.synchronize()
    yr, hr = oracle_run(inp)
    e1 = assert_close(host(y), yr, tol, "y")
    e2 = assert_close(host(hl), hr, tol, "h_last")
    return e1, e2


@pytest.mark.parametrize("L", [1, 17, 100, 333])
def test_batched_bf16_ragged(L):
    check(synth.selective_inputs(2, L, 200, 16, synth.BF16, 100 + L, with_h0=True), TOL[synth.BF16])


def test_batched_fp32_tight_tolerance():
    check(synth.selective_inputs(2, 300, 96, 16, synth.F32, 7, with_h0=True), TOL[synth.F32])


def test_scan_term_alone_without_skip_and_gate():
    # with Dskip and z absent the output is the scan readout only, so scan errors are not masked
    check(synth.selective_inputs(3, 257, 130, 16, synth.BF16, 8, with_z=False, with_skip=False, with_h0=True),
          TOL[synth.BF16])
    check(synth.selective_inputs(2, 129, 64, 16, synth.F32, 9, with_z=False, with_skip=False), TOL[synth.F32])


def _general_A(D, N, seed):
    # negative rates with no common structure across n: every state takes its own exponential
    rng = np.random.default_rng(seed)
    return (-np.exp(rng.uniform(np.log(0.5), np.log(64.0), size=(D, N)))).astype(np.float32)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_unstructured_A_mixed_with_multiscale_A(dtype):
    # channels 0..63 keep A_n = -(n+1) 2^s, the others get unstructured rates: the kernels make no
    # use of the structure of A, and both kinds of row meet the tolerance in one call
    inp = synth.selective_inputs(2, 300, 200, 16, dtype, 30, with_h0=True)
    A = _general_A(200, 16, 31)
    A[:64] = inp.p["A"][:64]
    inp.p["A"] = A
    check(inp, TOL[dtype])


def test_heavy_tailed_gated_output_fp32():
    # a gated output whose largest element is about 45 times its RMS: the bound then asks for a few
    # ulp on that element, so the error of delta (softplus of dt in about -7..-2) must stay near 1 ulp
    inp = synth.selective_inputs(3, 203, 79, 4, synth.F32, 939316136, with_z=True, with_skip=False)
    check(inp, TOL[synth.F32])


def test_softplus_at_minus_infinity_gives_zero_step():
    # dt = -inf: delta = softplus(-inf) = 0, so the row leaves the states unchanged
    inp = synth.selective_inputs(2, 40, 64, 16, synth.F32, 36, with_h0=True)
    inp.t["dt"].data[:, 5:9, :7] = -np.inf
    check(inp, TOL[synth.F32])


def test_long_memory_fp32():
    # one scale (A_n = -(n+1)) over 2048 steps: the longest-lived states accumulate the most rounding
    inp = synth.selective_inputs(1, 2048, 64, 16, synth.F32, 32, num_scales=1, with_h0=True)
    check(inp, TOL[synth.F32])


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_smaller_state_sizes(N):
    check(synth.selective_inputs(2, 90, 70, N, synth.F32, 10 + N, num_scales=2, with_h0=True), TOL[synth.F32])


def test_raw_delta_without_softplus_and_bias():
    inp = synth.selective_inputs(2, 150, 64, 16, synth.F32, 20, dt_softplus=False, with_h0=True)
    inp.p["dt_bias"] = np.full(64, 0.01, dtype=np.float32)
    check(inp, TOL[synth.F32])


def test_softplus_with_bias():
    inp = synth.selective_inputs(2, 150, 64, 16, synth.BF16, 21)
    inp.p["dt_bias"] = np.linspace(-1, 1, 64).astype(np.float32)
    check(inp, TOL[synth.BF16])


def test_clamp_acts_for_positive_A():
    # delta*A > 20 for some states: abar is capped at e^20 (short sequence so values stay finite)
    inp = synth.selective_inputs(1, 3, 64, 16, synth.F32, 22, dt_softplus=False)
    inp.p["A"] = np.abs(inp.p["A"]) * 300.0
    check(inp, TOL[synth.F32])


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_positive_A_beside_negative_A_with_softplus_steps(dtype, packed):
    """A few states with A > 0 put their channels' waves on the clamped path, where the other channels
    of those waves still have A <= 0: the carries rebuild the segment decay of those channels from the
    segment's delta sum and read the stored products of the others.  Several segments per sequence
    (packed bf16: first, middle and last pieces), so every kind of carry is used."""
    if packed:
        cu = synth.cu_seqlens_from_lengths([700, 130, 1300, 3])
        inp = synth.selective_inputs(1, int(cu[-1]), 130, 16, dtype, 37, cu_seqlens=cu, with_h0=True)
    else:
        inp = synth.selective_inputs(2, 300, 130, 16, dtype, 38, with_h0=True)
    A = inp.p["A"].copy()
    A[5, 3] = A[70, 0] = A[129, 15] = 0.004  # slow growth: finite over the longest sequence
    inp.p["A"] = A
    check(inp, TOL[dtype])


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_varlen_more_sequences_than_one_planner_pass(dtype):
    """1500 packed sequences (the planners take sequences 1024 at a time): short and empty ones on both
    sides of the 1024 boundary, and three long ones cut into first, middle and last pieces."""
    rng = np.random.default_rng(39)
    lengths = rng.integers(0, 24, size=1500)
    lengths[rng.choice(1500, 200, replace=False)] = 0
    lengths[[10, 1023, 1024]] = [700, 0, 1300]
    lengths[1499] = 611
    cu = synth.cu_seqlens_from_lengths([int(v) for v in lengths])
    inp = synth.selective_inputs(1, int(cu[-1]), 64, 16, dtype, 40, cu_seqlens=cu, with_h0=True)
    check(inp, TOL[dtype])


def test_varlen_with_empty_and_unit_sequences():
    lengths = [5, 0, 1, 300, 0, 77, 2, 0]
    cu = synth.cu_seqlens_from_lengths(lengths)
    inp = synth.selective_inputs(1, int(cu[-1]), 130, 16, synth.BF16, 30, cu_seqlens=cu, with_h0=True)
    check(inp, TOL[synth.BF16])
    inp = synth.selective_inputs(1, int(cu[-1]), 64, 16, synth.F32, 31, cu_seqlens=cu, with_h0=True)
    check(inp, TOL[synth.F32])


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_varlen_single_sequence_equals_batched(dtype):
    """One packed sequence is the batched scan of that sequence.  With bf16 inputs the two calls cut
    it into different pieces (the packed plan keeps pieces long, the batched one cuts 16-row
    segments), so the results agree up to the reassociation of a 500-step fp32 recurrence; each
    meets the oracle."""
    import torch
    inp = synth.selective_inputs(1, 500, 96, 16, dtype, 32, with_h0=True)
    yb, hb = gpu_run(inp)
    inp.s["cu_seqlens"] = np.array([0, 500], dtype=np.int32)
    yv, hv = gpu_run(inp)
    torch.cuda.synchronize()
    yr, hr = oracle_run(inp)
    for y, h, what in ((yb, hb, "batched"), (yv, hv, "packed")):
        assert_close(host(y), yr, TOL[dtype], f"{what} y")
        assert_close(host(h), hr, TOL[dtype], f"{what} h_last")
    assert_close(host(yv), host(yb), 1e-4, "packed vs batched y")
    assert_close(host(hv), host(hb), 1e-4, "packed vs batched h_last")


@pytest.mark.parametrize("with_h0", [True, False])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_varlen_long_sequences_cut_into_pieces(dtype, with_h0):
    """Packed sequences longer than the plan's piece length are cut into pieces.  bf16 inputs (the
    two-phase plan, pieces of 256 rows here): 700 -> 256 + 256 + 188 rows (one middle piece), 1300
    -> 256 + 4 x 256 + 20 (four), 257 -> 256 + 1 (none: the last piece starts from the first piece's
    end state), 256 and 3 unsplit.  fp32 inputs take 16-row segments with the carry kernel."""
    lengths = [700, 3, 1300, 0, 257, 256]
    cu = synth.cu_seqlens_from_lengths(lengths)
    inp = synth.selective_inputs(1, int(cu[-1]), 130, 16, dtype, 35, cu_seqlens=cu, with_h0=with_h0)
    check(inp, TOL[dtype])


def test_bf16_output():
    import torch
    inp = synth.selective_inputs(2, 200, 128, 16, synth.BF16, 33)
    y32 = gpu_run(inp, return_last_state=False)
    y16 = gpu_run(inp, out_dtype=torch.bfloat16, return_last_state=False)
    diff = (y16.float() - y32.to(torch.bfloat16).float()).abs()
    assert bool((diff <= y32.abs().clamp_min(1e-30) * 2.0 ** -7).all())


def test_deterministic_and_fully_written():
    import torch
    inp = synth.selective_inputs(2, 777, 200, 16, synth.BF16, 34)
    a = gpu_run(inp)
    b = gpu_run(inp)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.isfinite(a[0]).all()


def test_decode_steps_equal_scan():
    import torch
    B, L, D, N = 4, 30, 130, 16
    inp = synth.selective_inputs(B, L, D, N, synth.BF16, 40, with_h0=True)
    t = {k: to_dev(v) for k, v in inp.t.items()}
    A, Dskip, h0 = to_dev(inp.p["A"]), to_dev(inp.p["Dskip"]), to_dev(inp.p["h0"])
    state = h0.clone()
    ys = [ssd.selective_update(t["x"][:, s].contiguous(), t["dt"][:, s].contiguous(), A, t["Bm"][:, s].contiguous(),
                               t["Cm"][:, s].contiguous(), state, Dskip=Dskip, z=t["z"][:, s].contiguous())
          for s in range(L)]
    torch.cuda.synchronize()
    yr, hr = oracle_run(inp)
    assert_close(host(torch.stack(ys, 1)), yr, TOL[synth.BF16], "decode y")
    assert_close(host(state), hr, TOL[synth.BF16], "decode state")


def _sampled_check(inp, nrandom, seed, tol):
    """Every output of sampled channels vs the oracle (channels are independent): the first and last
    channel of every 256-channel workgroup and of every scale block, plus nrandom seeded ones, per batch
    row; the oracle runs on groups of them in parallel."""
    import torch
    y, hl = gpu_run(inp)
    torch.cuda.synchronize()
    B, L, D = inp.t["x"].shape
    yh = y.cpu()
    hlh = hl.cpu()
    cu = inp.s.get("cu_seqlens")
    worst = 0.0
    for b in range(B):
        ds = spread_channels(D, nrandom, seed + b)
        groups = np.array_split(ds, 8)

        def run(g):
            sel = lambda n: synth.bf16_to_f64(inp.t[n].data[b:b + 1][:, :, g])
            full = lambda n: synth.bf16_to_f64(inp.t[n].data[b:b + 1])
            return oracle.selective_scan(sel("x"), sel("dt"), inp.p["A"][g].astype(np.float64), full("Bm"),
                                         full("Cm"), Dskip=f64(inp.p["Dskip"][g]) if "Dskip" in inp.p else None,
                                         z=sel("z") if "z" in inp.t else None, dt_softplus=inp.s["dt_softplus"],
                                         cu_seqlens=cu)

        refs = parallel_map(run, groups)
        yr = np.concatenate([r[0] for r in refs], axis=2)
        hr = np.concatenate([r[1] for r in refs], axis=1)
        dsel = torch.as_tensor(ds)
        worst = max(worst, assert_close(yh[b:b + 1][:, :, dsel].double().numpy(), yr, tol, f"y batch {b}"))
        hsel = hlh[b:b + 1] if cu is None else hlh
        assert_close(hsel[:, dsel].double().numpy(), hr, tol, f"h_last batch {b}")
    assert torch.isfinite(y).all()
    return worst


def test_selective_workload_full_size_sampled_channels():
    """B=4 L=2048 D=1536: per batch row the 12 edge channels of the 6 workgroups (which include the
    scale-block edges) plus 52 random ones = 64 channels, 256 in all."""
    inp = synth.workload_inputs("selective")
    _sampled_check(inp, 52, 1, TOL[synth.BF16])
    inp.t.pop("z")
    inp.p.pop("Dskip")
    _sampled_check(inp, 52, 2, TOL[synth.BF16])


def test_varlen_workload_full_size_sampled_channels():
    """Packed L=131072 D=4096, 32 sequences: the 32 edge channels of the 16 workgroups (and of the 4
    scale blocks) plus 32 random ones = 64 channels, every output and every sequence's final state."""
    inp = synth.workload_inputs("selective_varlen")
    _sampled_check(inp, 32, 3, TOL[synth.BF16])
    # and the scan term alone (the skip term dominates the output otherwise)
    inp.t.pop("z")
    inp.p.pop("Dskip")
    _sampled_check(inp, 32, 4, TOL[synth.BF16])
