"""ssd_rglru_scan_noalloc (the entry point for callers that cannot allocate) against ssd_rglru_scan,
through the C ABI: the same kernels on the library's fixed per-GPU scratch instead of a caller
workspace.  Two calls in a row (the second smaller, so it reuses scratch the first left behind) must
equal the workspace entry point bit for bit and the oracle within the fp32 tolerance; a problem whose
scratch exceeds the fixed array is rejected before anything is launched."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_noalloc_equals_workspace_entry_point_twice(dtype):
    import torch
    for k, (B, L, D) in enumerate([(3, 64 * 9 + 5, 258), (2, 100, 70)]):
        inp = synth.rglru_inputs(B, L, D, dtype, 8800 + k, with_h0=True, with_gate=(k == 1))
        args = [to_dev(inp.t[n]) for n in ("x", "r_logit", "i_logit")] + [to_dev(inp.p["a_log"]), 8.0]
        kw = dict(h0=to_dev(inp.p["h0"]), gate=to_dev(inp.t["gate"]) if "gate" in inp.t else None,
                  return_last_state=True)
        y1, h1 = ssd.rglru_scan_noalloc(*args, **kw)
        y2, h2 = ssd.rglru_scan(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(h1, h2), f"call {k}: noalloc differs from the workspace call"
        yr, hr = oracle.rglru_scan(f64(inp.t["x"]), f64(inp.t["r_logit"]), f64(inp.t["i_logit"]),
                                   f64(inp.p["a_log"]), 8.0, h0=f64(inp.p["h0"]),
                                   gate=f64(inp.t["gate"]) if "gate" in inp.t else None)
        assert_close(host(y1), yr, TOL[dtype], f"y call {k}")
        assert_close(host(h1), hr, TOL[dtype], f"h_last call {k}")


def test_noalloc_rejects_problems_beyond_its_scratch():
    import torch
    B, L, D = 8, 16384, 2560  # about 126 MB of lookback scratch, twice the fixed array
    need = ssd._ws_bytes("rglru_scan", B, L, D)
    assert need > ssd.NOALLOC_SCRATCH_BYTES
    x = torch.empty((B, L, D), dtype=torch.bfloat16, device="cuda")
    a_log = torch.full((D,), -0.01, device="cuda")
    with pytest.raises(ssd.SSDValueError) as ei:
        ssd.rglru_scan_noalloc(x, x, x, a_log, 8.0)
    assert ei.value.status == 2 and "fixed" in str(ei.value)
