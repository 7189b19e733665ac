"""The workspace contract of the C ABI on the GPU: caller-owned workspaces reused across calls and
sizes, shared by host threads that call on one stream, and the timeout path of the bounded waits
between workgroups (forced from the host through the test hook, so every kernel still runs to its
end: the waits are bounded and give up after a few polls)."""
import threading

import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


def rglru_case(B, L, D, seed, dtype=synth.F32):
    inp = synth.rglru_inputs(B, L, D, dtype, seed, with_h0=True)
    dev = {n: to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit")}
    yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]), f64(inp.p["a_log"]),
                               8.0, h0=f64(inp.p["h0"]))
    return inp, dev, yr, hr


def test_explicit_workspace_reused_across_sizes():
    """One zero-filled workspace of the largest query size serves calls of several sizes in turn."""
    import torch
    shapes = [(2, 700, 130), (1, 64, 64), (3, 1000, 256), (2, 65, 66)]
    need = max(ssd._ws_bytes("rglru_scan", *s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for k, (B, L, D) in enumerate(shapes * 2):
        inp, dev, yr, hr = rglru_case(B, L, D, 50 + k)
        y, hl = ssd.rglru_scan(dev["x"], dev["r_logit"], dev["i_logit"], to_dev(inp.p["a_log"]), 8.0,
                               h0=to_dev(inp.p["h0"]), return_last_state=True, workspace=ws)
        torch.cuda.synchronize()
        assert_close(host(y), yr, TOL[synth.F32], f"y {B}x{L}x{D}")
        assert_close(host(hl), hr, TOL[synth.F32], f"h_last {B}x{L}x{D}")
    assert lib_check(ws) == 0


def lib_check(ws):
    import torch
    return ssd.lib().ssd_workspace_check(ws.data_ptr(), torch.cuda.current_stream().cuda_stream)


def test_two_host_threads_grow_one_stream_workspace():
    """Two host threads call the scan on the same (default) stream with sizes that keep growing, so the
    binding's workspace for that stream is replaced while the other thread's calls are queued; every
    result must still equal the oracle."""
    import torch
    cases = {t: [rglru_case(1 + (k % 2), 100 + 300 * k + 37 * t, 64 + 32 * t, 60 + 10 * t + k) for k in range(6)]
             for t in range(2)}
    errors, results = [], {}
    barrier = threading.Barrier(2)

    def worker(t):
        try:
            torch.cuda.set_device(0)
            outs = []
            barrier.wait()
            for inp, dev, _, _ in cases[t]:
                outs.append(ssd.rglru_scan(dev["x"], dev["r_logit"], dev["i_logit"], to_dev(inp.p["a_log"]), 8.0,
                                           h0=to_dev(inp.p["h0"]), return_last_state=True))
            results[t] = outs
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for (inp, _, yr, hr), (y, hl) in zip(cases[t], results[t]):
            assert_close(host(y), yr, TOL[synth.F32], f"thread {t} y")
            assert_close(host(hl), hr, TOL[synth.F32], f"thread {t} h_last")


def test_forced_timeout_is_reported_and_outputs_are_nan():
    """The test hook makes every bounded wait target words no launch writes and give up after 64 polls:
    the chunks that wait (all but the first 64 steps of each sequence) read NaN, the first chunk is exact,
    and workspace_check reports SSD_ERR_TIMEOUT once.  Afterwards the same workspace gives exact results."""
    import torch
    B, L, D = 2, 64 * 5 + 7, 130
    inp, dev, yr, hr = rglru_case(B, L, D, 70)
    args = (dev["x"], dev["r_logit"], dev["i_logit"], to_dev(inp.p["a_log"]), 8.0)
    ssd.workspace_check()
    try:
        ssd.testing_lookback(64, True)
        y = ssd.rglru_scan(*args, h0=to_dev(inp.p["h0"]))
        with pytest.raises(ssd.SSDError) as ei:
            ssd.workspace_check()
        assert ei.value.status == ssd.SSD_ERR_TIMEOUT
        # the forward's gradient pass waits the same way
        dy = torch.randn((B, L, D), device="cuda")
        g = ssd.rglru_scan_backward(*args, dy, h0=to_dev(inp.p["h0"]))
        with pytest.raises(ssd.SSDError):
            ssd.workspace_check()
    finally:
        ssd.testing_lookback(0, False)
    yh = host(y)
    assert np.all(np.isnan(yh[:, 64:])), "outputs after a wait that gave up must be NaN"
    assert_close(yh[:, :64], yr[:, :64], TOL[synth.F32], "first chunk (no wait)")
    assert torch.isnan(g["dx"][:, : L - 64 - 7]).all()
    ssd.workspace_check()  # the record was cleared
    y, hl = ssd.rglru_scan(*args, h0=to_dev(inp.p["h0"]), return_last_state=True)
    torch.cuda.synchronize()
    assert_close(host(y), yr, TOL[synth.F32], "y after the timeout")
    assert_close(host(hl), hr, TOL[synth.F32], "h_last after the timeout")


def test_forced_timeout_minmax():
    import torch
    inp = synth.minmax_inputs(2, 64 * 3 + 1, 66, synth.BF16, 71, with_x0=True)
    r, s = to_dev(inp.t["r"]), to_dev(inp.t["s"])
    try:
        ssd.testing_lookback(32, True)
        y = ssd.minmax_scan(r, s, x0=to_dev(inp.p["x0"]))
        with pytest.raises(ssd.SSDError):
            ssd.workspace_check()
    finally:
        ssd.testing_lookback(0, False)
    assert torch.isnan(y[:, 64:]).all()
    y = ssd.minmax_scan(r, s, x0=to_dev(inp.p["x0"]))
    yr, _ = oracle.minmax_scan(f64(inp.t["r"]), f64(inp.t["s"]), x0=f64(inp.p["x0"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(y), yr)
