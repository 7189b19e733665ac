"""GPU parity of the key-axis-gated HGRN2 scan in its chunked MFMA form (bf16 inputs, d = 128) against the
fp64 oracle, through the C ABI: shapes across chunk boundaries and both workgroup-to-head mappings, with
and without an initial state; gates saturated at the lower bound over whole chunks, at bounds where the
in-chunk decay lb^64 stays above 2^-96 and where it does not (those chunks go token by token); every
chunk token by token; NaN planted in each input, which must reach exactly the outputs and state entries
the recurrence sends it to, with and without the decay check compiled in.
Tolerance: max|err| <= 2e-2 * RMS(oracle) (bf16 inputs)."""
import numpy as np
import pytest

import oracle
import selective_state_space_diag_amd as ssd
from selective_state_space_diag_amd import synth
from tests.helpers import TOL, assert_close, f64, host, to_dev

pytestmark = pytest.mark.gpu


def run_key(inp, lb, out_dtype=None):
    import torch
    t = {n: to_dev(v) for n, v in inp.t.items()}
    kw = {} if out_dtype is None else {"out_dtype": out_dtype}
    o, S = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], lb, S0=to_dev(inp.p.get("S0")),
                          return_last_state=True, gate_axis="key", **kw)
    torch.cuda.synchronize()
    return host(o), host(S)


def oracle_key(inp, lb):
    t = inp.t
    return oracle.hgrn2_key_scan(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["g_logit"]), lb, f64(inp.p.get("S0")))


@pytest.mark.parametrize("B,L,H,lb,with_S0", [
    (2, 200, 4, 0.5, True),    # B*H = 8: the two halves of a head on one XCD; ragged last chunk
    (1, 65, 3, 0.36, True),    # B*H = 3: plain mapping; one token in the last chunk
    (3, 64, 1, 0.9, True),     # exactly one chunk
    (1, 1, 2, 1.0, True),      # one token, gates 1
    (2, 130, 2, 0.7, False),   # no initial state
    (1, 320, 2, 0.5, True),    # five chunks
])
def test_key_chunked_shapes(B, L, H, lb, with_S0):
    inp = synth.hgrn2_inputs(B, L, H, 128, synth.BF16, 9600 + L + 7 * H, lower_bound=lb, with_S0=with_S0)
    o, S = run_key(inp, lb)
    orf, Sr = oracle_key(inp, lb)
    assert_close(o, orf, TOL[synth.BF16], "o")
    assert_close(S, Sr, TOL[synth.BF16], "S_last")


@pytest.mark.parametrize("lb", [0.36, 0.354, 0.2, 0.0])
def test_key_chunked_saturated_gates(lb):
    """Gates at the bound over whole chunks: in-chunk decays lb^64, 2^-94.3 at 0.36 and 2^-95.9 at 0.354
    (K / Gamma reaches 2^94 |K| inside the products), 2^-148.6 at 0.2 and about 10^-830 at 0 (those
    chunks go token by token); chunk 0 has ordinary gates, so every sequence mixes the two ways."""
    inp = synth.hgrn2_inputs(2, 200, 3, 128, synth.BF16, 9700 + int(lb * 1000), lower_bound=lb, with_S0=True)
    g = synth.bf16_to_f32(inp.t["g_logit"].data).copy()
    g[:, 64:128] = -30.0                     # chunk 1: every gate at the bound
    g[:, 128:192, :, ::2] = -30.0            # chunk 2: half the key columns saturated
    g[0, :, 1] = -30.0                       # one whole head saturated over the whole sequence
    inp.t["g_logit"] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g))
    o, S = run_key(inp, lb)
    orf, Sr = oracle_key(inp, lb)
    assert_close(o, orf, TOL[synth.BF16], "o")
    assert_close(S, Sr, TOL[synth.BF16], "S_last")
    for b in range(o.shape[0]):
        for h in range(o.shape[2]):
            assert_close(o[b, :, h], orf[b, :, h], TOL[synth.BF16], f"o head {b},{h}")


def _plant(inp, name, idx):
    a = synth.bf16_to_f32(inp.t[name].data).copy()
    a[idx] = np.nan
    inp.t[name] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(a))


@pytest.mark.parametrize("name,idx", [
    ("v", (0, 70, 1, 9)),     # value row 9 of head (0, 1) from token 70 on, and that state row
    ("g_logit", (0, 70, 1, 9)),  # key column 9: every output of head (0, 1) from token 70, state column 9
    ("q", (0, 70, 1, 9)),     # token 70 of head (0, 1) only
    ("k", (0, 130, 0, 100)),  # every output of head (0, 0) from token 130 on, state column 100
    ("v", (0, 63, 0, 127)),   # last token of a chunk, last row of the second workgroup
])
@pytest.mark.parametrize("lb", [0.5, 0.0])
def test_key_chunked_nan_reaches_what_the_recurrence_reaches(name, idx, lb):
    inp = synth.hgrn2_inputs(1, 150, 2, 128, synth.BF16, 9800, lower_bound=lb, with_S0=True)
    _plant(inp, name, idx)
    o, S = run_key(inp, lb)
    orf, Sr = oracle_key(inp, lb)
    assert np.isnan(orf).any()
    assert np.array_equal(np.isnan(o), np.isnan(orf)), "NaN pattern of o"
    assert np.array_equal(np.isnan(S), np.isnan(Sr)), "NaN pattern of S_last"
    ok, okS = ~np.isnan(orf), ~np.isnan(Sr)
    assert_close(o[ok], orf[ok], TOL[synth.BF16], "o outside the NaN entries")
    assert_close(S[okS], Sr[okS], TOL[synth.BF16], "S_last outside the NaN entries")


def test_key_chunked_all_chunks_token_by_token():
    """Every gate at the bound 0 (logit -30) but one key column near 1: every chunk of every head fails the
    decay check; with an S0 and a ragged last chunk."""
    inp = synth.hgrn2_inputs(2, 64 * 3 + 9, 2, 128, synth.BF16, 9850, lower_bound=0.0, with_S0=True)
    g = np.full(inp.t["g_logit"].shape, -30.0, dtype=np.float32)
    g[:, :, :, 5] = 3.0
    inp.t["g_logit"] = synth.Tensor(synth.BF16, synth.f32_to_bf16_bits(g))
    o, S = run_key(inp, 0.0)
    orf, Sr = oracle_key(inp, 0.0)
    assert_close(o, orf, TOL[synth.BF16], "o")
    assert_close(S, Sr, TOL[synth.BF16], "S_last")


@pytest.mark.parametrize("lb", [0.5, 0.0])
def test_key_chunked_bf16_output_is_rounded_fp32(lb):
    import torch
    inp = synth.hgrn2_inputs(2, 100, 2, 128, synth.BF16, 9870, lower_bound=lb, with_S0=True)
    o32, _ = run_key(inp, lb)
    o16, _ = run_key(inp, lb, out_dtype=torch.bfloat16)
    ref = torch.from_numpy(o32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(o16, ref)


def test_key_chunked_decode_continues_scan():
    """Decode steps at d = 128 started from the chunked scan's final state agree with one longer scan."""
    import torch
    B, L, H, d, extra = 1, 100, 2, 128, 5
    inp = synth.hgrn2_inputs(B, L + extra, H, d, synth.BF16, 9900, lower_bound=0.5, with_S0=True)
    t = {n: to_dev(v) for n, v in inp.t.items()}
    o_all, S_all = ssd.hgrn2_scan(t["q"], t["k"], t["v"], t["g_logit"], 0.5, S0=to_dev(inp.p["S0"]),
                                  return_last_state=True, gate_axis="key")
    _, S = ssd.hgrn2_scan(*(t[n][:, :L].contiguous() for n in ("q", "k", "v", "g_logit")), 0.5,
                          S0=to_dev(inp.p["S0"]), return_last_state=True, gate_axis="key")
    outs = [ssd.hgrn2_update(*(t[n][:, s].contiguous() for n in ("q", "k", "v", "g_logit")), 0.5, S,
                             gate_axis="key") for s in range(L, L + extra)]
    torch.cuda.synchronize()
    orf, Sr = oracle_key(inp, 0.5)
    assert_close(host(torch.stack(outs, 1)), orf[:, L:], TOL[synth.BF16], "decode o")
    assert_close(host(S), Sr, TOL[synth.BF16], "decode S")
    assert_close(host(o_all), orf, TOL[synth.BF16], "scan o")
    assert_close(host(S_all), Sr, TOL[synth.BF16], "scan S")
