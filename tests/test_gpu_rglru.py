"""GPU parity of the RG-LRU kernels against the fp64 oracle (called through the C ABI).

Tolerance: max|err| <= tau * RMS(oracle) on every output element and on h_last, tau = 1e-5 for
fp32 inputs and 2e-2 for bf16 inputs (fp32 state)."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


def run_case(B, L, D, dtype, seed, with_h0=True, c=8.0):
    import torch
    inp = synth.rglru_inputs(B, L, D, dtype, seed, c=c, with_h0=with_h0)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    a_log = to_dev(inp.p["a_log"])
    h0 = to_dev(inp.p["h0"]) if with_h0 else None
    y, hl = ssd.rglru_scan(x, r, i, a_log, c, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]),
                               f64(inp.p["a_log"]), c, f64(inp.p.get("h0")))
    assert_close(host(y), yr, TOL[dtype], "y")
    assert_close(host(hl), hr, TOL[dtype], "h_last")
    return inp, y


def test_rglru_small_workload_fp32():
    run_case(2, 128, 64, synth.F32, 1000, with_h0=False)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 127, 200])
def test_ragged_lengths_bf16(L):
    run_case(3, L, 300, synth.BF16, 7 + L)


@pytest.mark.parametrize("D", [1, 129, 130, 257])
def test_ragged_channels(D):
    # odd D takes the one-channel-per-lane path, even D the two-channel one
    run_case(2, 150, D, synth.BF16, 11 + D)
    run_case(1, 70, D, synth.F32, 12 + D)


def test_many_chunks_lookback_fp32():
    # 40 chunks per (b, tile): long lookback chains, fp32 tolerance
    run_case(2, 64 * 40 + 5, 256, synth.F32, 21)


def test_bf16_output_rounds_fp32_result():
    import torch
    inp = synth.rglru_inputs(2, 300, 256, synth.BF16, 31, with_h0=True)
    args = [to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit")] + [to_dev(inp.p["a_log"]), 8.0]
    y32 = ssd.rglru_scan(*args, h0=to_dev(inp.p["h0"]))
    y16 = ssd.rglru_scan(*args, h0=to_dev(inp.p["h0"]), out_dtype=torch.bfloat16)
    assert y16.dtype == torch.bfloat16
    diff = (y16.float() - y32.to(torch.bfloat16).float()).abs()
    ulp = y32.abs().clamp_min(1e-30) * 2.0 ** -7
    assert bool((diff <= ulp).all())


def test_every_output_written_and_deterministic():
    import torch
    inp = synth.rglru_inputs(2, 333, 384, synth.BF16, 41)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    a_log = to_dev(inp.p["a_log"])
    outs = []
    need = ssd._ws_bytes("rglru_scan", 2, 333, 384)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")  # the caller's own workspace, reused
    for _ in range(2):
        y = torch.full((2, 333, 384), float("nan"), device="cuda")
        hl = torch.full((2, 384), float("nan"), device="cuda")
        st = ssd.lib().ssd_rglru_scan(2, 333, 384, ssd.SSD_BF16, ssd.SSD_F32, x.data_ptr(), r.data_ptr(),
                                      i.data_ptr(), a_log.data_ptr(), 8.0, None, None, y.data_ptr(), hl.data_ptr(),
                                      None, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        assert not torch.isnan(y).any() and not torch.isnan(hl).any()
        outs.append((y.clone(), hl.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert ssd.lib().ssd_workspace_check(ws.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0


def test_decode_steps_equal_scan_and_oracle():
    import torch
    B, L, D = 4, 40, 320
    inp = synth.rglru_inputs(B, L, D, synth.BF16, 51, with_h0=True)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    a_log = to_dev(inp.p["a_log"])
    y_scan, h_scan = ssd.rglru_scan(x, r, i, a_log, 8.0, h0=to_dev(inp.p["h0"]), return_last_state=True)
    state = to_dev(inp.p["h0"]).clone()
    ys = [ssd.rglru_update(x[:, t].contiguous(), r[:, t].contiguous(), i[:, t].contiguous(), a_log, 8.0, state)
          for t in range(L)]
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, 1)
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                               8.0, f64(inp.p["h0"]))
    assert_close(host(y_dec), yr, TOL[synth.BF16], "decode y")
    assert_close(host(state), hr, TOL[synth.BF16], "decode state")
    assert_close(host(y_dec), host(y_scan), 1e-5, "decode vs scan")


@pytest.mark.parametrize("D", [1, 130, 258, 321, 2560])
@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_decode_channel_widths(D, dtype):
    """Decode steps at both widths of the decode kernel (two channels per lane for even D, one for odd
    D), fp32 and bf16 inputs, against the oracle."""
    import torch
    B, L = 3, 6
    inp = synth.rglru_inputs(B, L, D, dtype, 60 + D, with_h0=True)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    a_log = to_dev(inp.p["a_log"])
    state = to_dev(inp.p["h0"]).clone()
    ys = [ssd.rglru_update(x[:, t].contiguous(), r[:, t].contiguous(), i[:, t].contiguous(), a_log, 8.0, state)
          for t in range(L)]
    torch.cuda.synchronize()
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                               8.0, f64(inp.p["h0"]))
    assert_close(np.stack([host(v) for v in ys], axis=1), yr, TOL[dtype], "decode y")
    assert_close(host(state), hr, TOL[dtype], "decode state")


@pytest.mark.parametrize("L", [40, 100])
def test_short_scan_chunk_states(L):
    """Scans of at most 128 steps take the one-pass kernel; its chunk_states hold h0 and, past 64
    steps, the state after step 64, as the oracle gives them."""
    import torch
    B, D = 2, 130
    inp = synth.rglru_inputs(B, L, D, synth.F32, 70 + L, with_h0=True)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    cs = torch.full(ssd.chunk_states_shape(B, L, D), float("nan"), device="cuda")
    y, hl = ssd.rglru_scan(x, r, i, to_dev(inp.p["a_log"]), 8.0, h0=to_dev(inp.p["h0"]), return_last_state=True,
                           chunk_states=cs)
    torch.cuda.synchronize()
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                               8.0, f64(inp.p["h0"]))
    assert_close(host(y), yr, TOL[synth.F32], "y")
    assert_close(host(hl), hr, TOL[synth.F32], "h_last")
    states = host(cs)
    assert_close(states[:, 0], f64(inp.p["h0"]), TOL[synth.F32], "state entering chunk 0")
    if L > 64:
        assert_close(states[:, 1], yr[:, 63], TOL[synth.F32], "state entering chunk 1")


def test_decode_steps_replayed_from_a_hip_graph():
    """Decode steps captured once in a HIP graph: every replay, with eager work and synchronisations
    between replays, equals the same steps run eagerly."""
    import torch
    B, L, D = 4, 12, 320
    inp = synth.rglru_inputs(B, L, D, synth.BF16, 52, with_h0=True)
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    a_log, h0 = to_dev(inp.p["a_log"]), to_dev(inp.p["h0"])
    xs, rs, is_ = ([t[:, s].contiguous() for s in range(L)] for t in (x, r, i))
    state_e = h0.clone()
    y_e = torch.stack([ssd.rglru_update(xs[s], rs[s], is_[s], a_log, 8.0, state_e) for s in range(L)], 1)
    state = h0.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        ssd.rglru_update(xs[0], rs[0], is_[0], a_log, 8.0, h0.clone())  # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            ys = [ssd.rglru_update(xs[s], rs[s], is_[s], a_log, 8.0, state) for s in range(L)]
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(h0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.stack(ys, 1), y_e), f"replay {rep}: outputs differ from eager"
        assert torch.equal(state, state_e), f"replay {rep}: state differs from eager"
        ssd.rglru_update(xs[0], rs[0], is_[0], a_log, 8.0, h0.clone())  # eager work between replays


def test_split_scan_carries_state():
    import torch
    inp = synth.rglru_inputs(2, 250, 130, synth.F32, 61, with_h0=True)
    t = {n: to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit")}
    a_log, h0 = to_dev(inp.p["a_log"]), to_dev(inp.p["h0"])
    y, hl = ssd.rglru_scan(t["x"], t["r_logit"], t["i_logit"], a_log, 8.0, h0=h0, return_last_state=True)
    m = 97
    y1, h1 = ssd.rglru_scan(*(t[n][:, :m].contiguous() for n in ("x", "r_logit", "i_logit")), a_log, 8.0, h0=h0,
                            return_last_state=True)
    y2, h2 = ssd.rglru_scan(*(t[n][:, m:].contiguous() for n in ("x", "r_logit", "i_logit")), a_log, 8.0, h0=h1,
                            return_last_state=True)
    torch.cuda.synchronize()
    assert_close(host(torch.cat([y1, y2], 1)), host(y), 1e-5, "split y")
    assert_close(host(h2), host(hl), 1e-5, "split h_last")


def test_empty_sequence_copies_h0():
    import torch
    h0 = torch.randn(3, 64, device="cuda")
    e = torch.empty(3, 0, 64, device="cuda")
    y, hl = ssd.rglru_scan(e, e, e, torch.zeros(64, device="cuda"), 8.0, h0=h0, return_last_state=True)
    torch.cuda.synchronize()
    assert y.shape == (3, 0, 64) and torch.equal(hl, h0)


def test_rglru_workload_full_size_sampled_channels():
    """B=8, L=8192, D=2560 bf16 at full size; every output of 64 sampled (b, d) channels vs the oracle."""
    import torch
    cfg = synth.WORKLOADS["rglru"]
    inp = synth.workload_inputs("rglru")
    B, L, D = cfg["B"], cfg["L"], cfg["D"]
    x, r, i = (to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit"))
    a_log = to_dev(inp.p["a_log"])
    y, hl = ssd.rglru_scan(x, r, i, a_log, 8.0, return_last_state=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2024)
    bs = rng.integers(0, B, 64)
    ds = rng.integers(0, D, 64)
    g = lambda n: np.ascontiguousarray(synth.bf16_to_f64(inp.t[n].data[bs, :, ds]).T[None])    # [1, L, 64]
    yr, hr = oracle.rglru_scan(g("x"), g("r_logit"), g("i_logit"), inp.p["a_log"][ds].astype(np.float64), 8.0)
    yg = host(y[torch.as_tensor(bs, device="cuda"), :, torch.as_tensor(ds, device="cuda")]).T[None]
    assert_close(yg, yr, TOL[synth.BF16], "y sampled")
    assert_close(host(hl)[bs, ds][None], hr, TOL[synth.BF16], "h_last sampled")
    assert torch.isfinite(y).all()
