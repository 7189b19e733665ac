"""GPU parity of the HGRN2 backward in its chunked MFMA form (bf16 inputs, d = 128) against the gradient
oracle (float64 autograd over the sequential row-gated forward), through the C ABI.  The adjoint passes
run the forward chunk kernels with exchanged inputs, two of them backward in time with the next token's
gate; these cases cover chunk boundaries and one-token sequences in both directions, both workgroup-to-head
mappings, with and without S0 and dS_last, gates saturated at the lower bound over whole chunks (chunks
that go token by token in every pass), and bf16 outputs.
Tolerance per gradient tensor: max|err| <= 2e-2 * RMS(oracle gradient)."""
import numpy as np
import pytest

from selective_state_space_diag_amd import synth
from tests.helpers import assert_close, host
from tests.test_gpu_hgrn2_backward import NAMES, TOLB, gpu_grads, make, oracle_grads

pytestmark = pytest.mark.gpu
TOL = TOLB[synth.BF16]


@pytest.mark.parametrize("B,L,H,lb,with_S0,with_dSl", [
    (1, 1, 2, 0.5, True, True),      # one token: the reversed passes start and end on it
    (2, 63, 4, 0.5, True, False),    # B*H = 8 (both halves of a head on one XCD), one short chunk
    (1, 64, 3, 0.9, False, True),    # exactly one chunk, plain mapping
    (1, 65, 3, 0.36, True, True),    # one token in the last chunk (the first one backward in time)
    (2, 130, 2, 0.0, True, True),    # lower bound 0: the decay check in every pass
    (1, 200, 2, 1.0, True, True),    # gates 1
])
def test_backward_chunked_shapes(B, L, H, lb, with_S0, with_dSl):
    inp, do, dSl = make(B, L, H, 128, synth.BF16, 7800 + L + 3 * H, lb=lb, with_S0=with_S0, with_dSl=with_dSl)
    G = gpu_grads(inp, do, dSl)
    R = oracle_grads(inp, do, dSl)
    for n in NAMES:
        assert_close(host(G[n]), R[n], TOL, n)


@pytest.mark.parametrize("lb", [0.36, 0.2, 0.0])
def test_backward_chunked_saturated_gates(lb):
    """Gates at the bound over whole chunks (in-chunk decay lb^64): at 0.36 the products hold it, at 0.2 and
    0 those chunks go token by token, in the forward pass, the reversed passes (whose gates are shifted by
    one token) and the key-axis pass alike.  dq, dk, dv and dS0 are also checked head by head; the gate
    gradient is not: as a suffix sum of do o - v dv it carries an absolute error of the order of those
    terms' rounding (~1e-9 here), while a head whose gates sit at 1e-13 has a true gate gradient of that
    order, so only the bound over the whole tensor applies to it (as for the register sweep)."""
    inp, do, dSl = make(2, 200, 2, 128, synth.BF16, 7900 + int(1000 * lb), lb=lb)
    g = synth.bf16_to_f32(inp.t["g_logit"].data).copy()
    g[:, 64:128] = -30.0
    g[:, 128:192, :, ::2] = -30.0
    g[0, :, 1] = -30.0
    inp.t["g_logit"] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g))
    G = gpu_grads(inp, do, dSl)
    R = oracle_grads(inp, do, dSl)
    for n in NAMES:
        assert_close(host(G[n]), R[n], TOL, n)
        if n == "dg_logit":
            continue
        for b in range(2):
            for h in range(2):
                sl = (slice(b, b + 1), slice(None), slice(h, h + 1)) if n != "dS0" else (slice(b, b + 1), slice(h, h + 1))
                assert_close(host(G[n][sl]), R[n][sl], TOL, f"{n} head {b},{h}")


def test_backward_chunked_bf16_outputs():
    """bf16 outputs are the fp32 results rounded (the gate gradient's sums take dv in fp32 either way); dS0
    is fp32 in both."""
    import torch
    inp, do, dSl = make(2, 150, 2, 128, synth.BF16, 7950)
    G32 = gpu_grads(inp, do, dSl)
    G16 = gpu_grads(inp, do, dSl, out_dtype=torch.bfloat16)
    for n in ("dq", "dk", "dv", "dg_logit"):
        assert torch.equal(G16[n], G32[n].to(torch.bfloat16)), n
    assert torch.equal(G16["dS0"], G32["dS0"])
    R = oracle_grads(inp, do, dSl)
    for n in NAMES:
        assert_close(host(G32[n]), R[n], TOL, n)
