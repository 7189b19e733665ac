#!/usr/bin/env python3
"""Throughput of the gfx950 gated diagonal linear-recurrence scans on one MI355X.

Headline (the JSON ``value``): the multi-scale selective scan at B=4, L=2048, D=1536, N=16,
bf16 inputs, fp32 state and output, in state updates per second.  One step is one full
selective scan (softplus, discretisation, recurrence, readout, skip and silu gate) over one
batch of synthetic input already resident in HBM.  Three input sets rotate so the 256 MB
Infinity Cache cannot serve the 126 MB working set.

The JSON line also carries:
  roofline      the dominant kernel against its roofline, with per-step HIP-event timing on
                the stream the kernels run on;
  cpu_baseline  the fp64 CPU oracle timed on the host (reported baseline, not a target);
  forms         the other workloads (RG-LRU fp32 and bf16, RG-LRU decode, HGRN2, packed
                variable-length selective scan) with their own throughput and GB/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-forms] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
FP32_VECTOR_TFLOPS = 157.3   # MI355X fp32 vector, published (counts packed two-wide FMA)
# fp32 vector peak without packed instructions, which this library does not use: 256 CUs x 4 SIMDs x
# 16 lanes x 2 flops per FMA x 2.4 GHz
FP32_SCALAR_FMA_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
BF16_MFMA_TFLOPS = 2500.0    # MI355X dense bf16 matrix, published


# ----------------------------------------------------------------------------- algorithmic sizes
def selective_bytes(B, L, D, N, in_b=2, out_b=4, z=True, skip=True, nseq=None):
    act = B * L * D
    b = act * in_b * (3 if z else 2) + 2 * B * L * N * in_b + D * N * 4 + act * out_b
    if skip:
        b += D * 4
    if nseq is not None:
        b += (nseq + 1) * 4
    return b


# Algorithmic flops per selective state update: delta*A (1), exp (1), (delta*x)*B_n (1),
# h = abar*h + bbar (2), y += C_n*h (2).
SELECTIVE_FLOPS_PER_UPDATE = 7


def rglru_bytes(B, L, D, in_b=2, out_b=4):
    return B * L * D * (3 * in_b + out_b) + D * 4


def rglru_gated_bytes(B, L, D, in_b=2, out_b=4):
    return B * L * D * (4 * in_b + out_b) + D * 4


def rglru_bwd_bytes(B, L, D, in_b=2, out_b=4):
    # x, r, i, dy read once; dx, dr_logit, di_logit written; a_log in, d a_log out
    return B * L * D * (4 * in_b + 3 * out_b) + 2 * D * 4


def minmax_bytes(B, L, D, in_b=2, out_b=4):
    return B * L * D * (2 * in_b + out_b)


def minmax_bwd_bytes(B, L, D, in_b=2, out_b=4):
    # r, s, dy read once; dr, ds written
    return B * L * D * (3 * in_b + 2 * out_b)


def selective_bwd_bytes(B, L, D, N, in_b=2, out_b=4):
    # x, dt, z, dy read, dx, ddt, dz written; Bm, Cm read, dBm, dCm written; A, Dskip, dt_bias and
    # their gradients
    return B * L * D * (4 * in_b + 3 * out_b) + B * L * N * (2 * in_b + 2 * out_b) + D * N * 8 + D * 16


def conv_bytes(B, L, D, W, in_b=2, out_b=4):
    return B * L * D * (in_b + out_b) + D * (W + 1) * 4


def hgrn2_bytes(B, L, H, d, in_b=2, out_b=4):
    return B * L * H * d * (4 * in_b + out_b)


def hgrn2_bwd_bytes(B, L, H, d, in_b=2, out_b=4):
    # q, k, v, g_logit, do read (in dtype) and the forward's fp32 o; dq, dk, dv, dg_logit written
    return B * L * H * d * (5 * in_b + 4 + 4 * out_b)


def profiled_traffic(profile, sources):
    """HBM bytes per call recorded by rocprofv3 counter runs in profiles/<profile>, if the kernel
    sources are unchanged since (their sha256 is stored with the figure); else None."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- profile-data: (\{.*\}) -->", open(path).read())
    if not m:
        return None
    data = json.loads(m.group(1))
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return data["traffic_bytes_per_call"] if h.hexdigest() == data["kernel_sources_sha256"] else None


# ----------------------------------------------------------------------------- timing helpers
WARM_SECONDS = 0.3  # untimed running before each timed region, so clocks have left their idle state


def time_calls(fn, n_sets, steps, warmup):
    """Run ``fn(i % n_sets)`` at least ``warmup`` times and for at least WARM_SECONDS, then time
    ``steps`` back-to-back calls between one pair of HIP events on torch's current stream (the stream
    the library launches on), synchronizing before and after.  Returns (ms per step from the events,
    ms per step from the host clock)."""
    import torch
    t_warm = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_warm < WARM_SECONDS:
        fn(i % n_sets)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i % n_sets)
    end.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end) / steps, wall / steps


def dev_bf16(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


# ----------------------------------------------------------------------------- headline
def headline(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    from selective_state_space_diag_amd import synth

    cfg = synth.WORKLOADS["selective"]
    B, L, D, N = cfg["B"], cfg["L"], cfg["D"], cfg["N"]
    n_sets = 3
    sets = []
    host_inputs = None
    for k in range(n_sets):
        inp = synth.workload_inputs("selective", seed=1001 + 100 * k)
        if k == 0:
            host_inputs = inp
        t = {n: dev_bf16(v.data, device) for n, v in inp.t.items()}
        sets.append(dict(t=t, A=torch.from_numpy(inp.p["A"]).to(device),
                         Dskip=torch.from_numpy(inp.p["Dskip"]).to(device)))

    def step(i):
        s = sets[i]
        t = s["t"]
        return ssd.selective_scan(t["x"], t["dt"], s["A"], t["Bm"], t["Cm"], Dskip=s["Dskip"], z=t["z"],
                                  dt_softplus=True)

    ms, wall = time_calls(step, n_sets, args.steps, args.warmup)
    updates = B * L * D * N
    nbytes = selective_bytes(B, L, D, N)
    res = dict(ms=ms, updates=updates, bytes=nbytes, host_ms=wall)
    return res, host_inputs


def cpu_baseline(host_inputs, min_seconds: float = 10.0):
    """The fp64 oracle on the whole headline workload (4 x 2048 x 1536 x 16), run back to back until
    at least ``min_seconds`` have passed (one pass takes about a second)."""
    import oracle
    t = host_inputs.t
    x, dt, z, Bm, Cm = (t[n].f64() for n in ("x", "dt", "z", "Bm", "Cm"))
    A = host_inputs.p["A"].astype(np.float64)
    Dskip = host_inputs.p["Dskip"].astype(np.float64)
    oracle.lib()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.selective_scan(x, dt, A, Bm, Cm, Dskip=Dskip, z=z, dt_softplus=True)
        reps += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds:
            break
    updates = reps * x.shape[0] * x.shape[1] * x.shape[2] * A.shape[1]
    return dict(value=updates / sec, unit="state-updates/s", cores=1, kind="oracle",
                sample=f"the whole headline workload (4x2048x1536 channels x 16 states) {reps} times back to back, "
                       f"{updates} updates in {sec:.1f} s, single-threaded fp64")


# ----------------------------------------------------------------------------- other workloads
def forms(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    from selective_state_space_diag_amd import synth

    out = {}
    gen = torch.Generator(device=device)
    gen.manual_seed(7)

    def randn(shape, std=1.0, mean=0.0, dtype=torch.bfloat16):
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return (t * std + mean).to(dtype)

    def record(name, ms, updates, nbytes, extra=None):
        d = dict(ms=round(ms, 5), state_updates_per_s=updates / (ms * 1e-3),
                 hbm_gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 algorithmic_bytes=nbytes, state_updates=updates)
        if extra:
            d.update(extra)
        out[name] = d
        print(f"# {name}: {ms:.4f} ms  {d['state_updates_per_s']:.3e} upd/s  {d['hbm_gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)

    # --- headline shape with unstructured A (no integer-multiple rows): one exponential per state
    B, L, D, N = 4, 2048, 1536, 16
    x, z = randn((B, L, D)), randn((B, L, D))
    A = -torch.exp(torch.empty(D, N, device=device).uniform_(np.log(0.5), np.log(64.0), generator=gen))
    delta0 = torch.exp(torch.empty(D, device=device).uniform_(np.log(1e-3), np.log(1e-1), generator=gen))
    delta = torch.exp(randn((B, L, D), std=0.1, dtype=torch.float32)) * delta0
    dt = (delta + torch.log(-torch.expm1(-delta))).to(torch.bfloat16)
    del delta
    Bm, Cm = randn((B, L, N), std=1.0 / N), randn((B, L, N), std=1.0 / N)
    Dskip = torch.ones(D, device=device)
    ms = time_calls(lambda kk: ssd.selective_scan(x, dt, A, Bm, Cm, Dskip=Dskip, z=z), 1, 30, 3)[0]
    record("selective_unstructured_A_B4_L2048_D1536_N16", ms, B * L * D * N, selective_bytes(B, L, D, N))

    # --- gradients of the selective scan on the headline shape (dy ~ N(0, 1), h0 and dh_last zero)
    dy = randn((B, L, D))
    ms = time_calls(lambda kk: ssd.selective_scan_backward(x, dt, A, Bm, Cm, dy, Dskip=Dskip, z=z), 1, 10, 2)[0]
    record("selective_backward_bf16_B4_L2048_D1536_N16", ms, B * L * D * N, selective_bwd_bytes(B, L, D, N))
    del x, z, dt, Bm, Cm, dy

    # --- RG-LRU fp32, B=2 L=128 D=64 (latency bound)
    B, L, D = 2, 128, 64
    x, r, i = (randn((B, L, D), dtype=torch.float32) for _ in range(3))
    a_log = torch.log(torch.empty(D, device=device).uniform_(0.9, 0.999, generator=gen))
    ms = time_calls(lambda k: ssd.rglru_scan(x, r, i, a_log, 8.0), 1, 50, 5)[0]
    record("rglru_fp32_B2_L128_D64", ms, B * L * D, rglru_bytes(B, L, D, 4, 4))

    # --- RG-LRU bf16, B=8 L=8192 D=2560
    B, L, D = 8, 8192, 2560
    x, r, i = (randn((B, L, D)) for _ in range(3))
    a_log = torch.log(torch.empty(D, device=device).uniform_(0.9, 0.999, generator=gen))
    ms = time_calls(lambda k: ssd.rglru_scan(x, r, i, a_log, 8.0), 1, 10, 2)[0]
    record("rglru_bf16_B8_L8192_D2560", ms, B * L * D, rglru_bytes(B, L, D))

    # --- the same scan with the block's gelu(gate) output multiply fused into its stores
    gt = randn((B, L, D))
    ms = time_calls(lambda k: ssd.rglru_scan(x, r, i, a_log, 8.0, gate=gt), 1, 10, 2)[0]
    record("rglru_gated_bf16_B8_L8192_D2560", ms, B * L * D, rglru_gated_bytes(B, L, D))
    del gt

    # --- gradients of the RG-LRU scan on the same shape (dy ~ N(0, 1)): with the chunk states a
    #     training forward saves (1/64 of the states), and recomputing them from the inputs
    dy = randn((B, L, D))
    cs = torch.empty(ssd.chunk_states_shape(B, L, D), device=device)
    ssd.rglru_scan(x, r, i, a_log, 8.0, chunk_states=cs)
    ms = time_calls(lambda k: ssd.rglru_scan_backward(x, r, i, a_log, 8.0, dy, chunk_states=cs), 1, 5, 1)[0]
    record("rglru_backward_bf16_B8_L8192_D2560", ms, B * L * D, rglru_bwd_bytes(B, L, D) + cs.numel() * 4)
    ms = time_calls(lambda k: ssd.rglru_scan_backward(x, r, i, a_log, 8.0, dy), 1, 5, 1)[0]
    record("rglru_backward_recompute_bf16_B8_L8192_D2560", ms, B * L * D, rglru_bwd_bytes(B, L, D))
    del dy

    # --- MinMax scan on the same shape (r, s ~ N(0, 1))
    ms = time_calls(lambda k: ssd.minmax_scan(r, i), 1, 10, 2)[0]
    record("minmax_bf16_B8_L8192_D2560", ms, B * L * D, minmax_bytes(B, L, D))

    # --- gradients of the MinMax scan on the same shape (dy ~ N(0, 1)), with and without the
    #     forward's chunk states
    dy = randn((B, L, D))
    ssd.minmax_scan(r, i, chunk_states=cs)
    ms = time_calls(lambda k: ssd.minmax_scan_backward(r, i, dy, chunk_states=cs), 1, 5, 1)[0]
    record("minmax_backward_bf16_B8_L8192_D2560", ms, B * L * D, minmax_bwd_bytes(B, L, D) + cs.numel() * 4)
    ms = time_calls(lambda k: ssd.minmax_scan_backward(r, i, dy), 1, 5, 1)[0]
    record("minmax_backward_recompute_bf16_B8_L8192_D2560", ms, B * L * D, minmax_bwd_bytes(B, L, D))
    del dy, cs

    # --- causal depthwise conv (width 4) in front of the RG-LRU, same shape
    W = 4
    wconv = torch.empty(D, W, device=device).uniform_(-0.5, 0.5, generator=gen)
    bconv = torch.empty(D, device=device).uniform_(-0.5, 0.5, generator=gen)
    ms = time_calls(lambda k: ssd.causal_conv1d(x, wconv, bias=bconv), 1, 10, 2)[0]
    record("causal_conv1d_bf16_B8_L8192_D2560_W4", ms, B * L * D, conv_bytes(B, L, D, W))
    del x, r, i

    # --- RG-LRU decode, B=256 D=2560, 256 steps carrying the state (one launch per step)
    B, D, S = 256, 2560, 256
    xs, rs, is_ = (randn((S, B, D)) for _ in range(3))
    state = torch.zeros(B, D, device=device)

    def decode(k):
        for s in range(S):
            ssd.rglru_update(xs[s], rs[s], is_[s], a_log, 8.0, state)

    ms = time_calls(decode, 1, 3, 1)[0]
    per_step_bytes = B * D * (3 * 2 + 4 + 4 + 4)
    record("rglru_decode_B256_D2560_256steps", ms, B * D * S, per_step_bytes * S,
           dict(us_per_step=ms * 1e3 / S))

    # --- the same 256 decode steps captured once in a HIP graph and replayed (identical kernels)
    state_g = torch.zeros(B, D, device=device)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        decode_g = lambda: [ssd.rglru_update(xs[s], rs[s], is_[s], a_log, 8.0, state_g) for s in range(S)]
        decode_g()  # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            decode_g()
    torch.cuda.synchronize()
    ms = time_calls(lambda k: graph.replay(), 1, 5, 1)[0]
    record("rglru_decode_B256_D2560_256steps_hipgraph", ms, B * D * S, per_step_bytes * S,
           dict(us_per_step=ms * 1e3 / S))
    del xs, rs, is_, graph

    # --- HGRN2 bf16, B=8 H=16 d=128 L=4096, lower bound 0.5
    B, L, H, dd = 8, 4096, 16, 128
    q, k, v = (randn((B, L, H, dd), std=dd ** -0.5) for _ in range(3))
    g = randn((B, L, H, dd), mean=2.0)
    ms = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.5), 1, 5, 1)[0]
    flops = 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)  # chunked form at chunk 64
    record("hgrn2_bf16_B8_H16_d128_L4096", ms, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
           dict(mfma_equiv_tflops=flops / (ms * 1e-3) / 1e12,
                mfma_util=flops / (ms * 1e-3) / 1e12 / BF16_MFMA_TFLOPS))

    # --- the same scan at the page's default lower bound 0 (the register sweep: 5 d^2 fp32 flops per
    #     token and head; the chunked MFMA form needs lower bounds >= 2^-1.5)
    ms = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.0), 1, 3, 1)[0]
    rflops = 5 * B * L * H * dd * dd
    record("hgrn2_lb0_bf16_B8_H16_d128_L4096", ms, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
           dict(valu_tflops=rflops / (ms * 1e-3) / 1e12, valu_frac=rflops / (ms * 1e-3) / 1e12 / FP32_SCALAR_FMA_TFLOPS))

    # --- gradients of the HGRN2 scan on the same shape (do ~ N(0, 1/d)), given the forward's fp32
    #     output; the three sweeps execute 15 d^2 fp32 flops per token and head (two state updates of
    #     3 d^2, the adjoint update twice, three d^2 matrix-vector products)
    do = randn((B, L, H, dd), std=dd ** -0.5)
    o = ssd.hgrn2_scan(q, k, v, g, 0.5)
    ms = time_calls(lambda kk: ssd.hgrn2_scan_backward(q, k, v, g, 0.5, do, o=o), 1, 3, 1)[0]
    vflops = 15 * B * L * H * dd * dd
    record("hgrn2_backward_bf16_B8_H16_d128_L4096", ms, B * L * H * dd * dd, hgrn2_bwd_bytes(B, L, H, dd),
           dict(valu_tflops=vflops / (ms * 1e-3) / 1e12, valu_frac=vflops / (ms * 1e-3) / 1e12 / FP32_SCALAR_FMA_TFLOPS))
    del do

    # --- the key-axis gate reading on the same inputs (a register sweep: 5 d^2 fp32 flops per token
    #     and head, the state update and the readout)
    ms = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.5, gate_axis="key"), 1, 3, 1)[0]
    kflops = 5 * B * L * H * dd * dd
    record("hgrn2_key_gate_bf16_B8_H16_d128_L4096", ms, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
           dict(valu_tflops=kflops / (ms * 1e-3) / 1e12, valu_frac=kflops / (ms * 1e-3) / 1e12 / FP32_SCALAR_FMA_TFLOPS))

    # --- readout LayerNorm over the hidden size (H d = 2048) with the silu output gate, on the scan's
    #     fp32 output: o read (fp32), gate read (bf16), y written (fp32)
    ogate = randn((B, L, H * dd))
    wn, bn = torch.ones(H * dd, device=device), torch.zeros(H * dd, device=device)
    o2 = o.view(B, L, H * dd)
    ms = time_calls(lambda kk: ssd.readout_norm(o2, gate=ogate, weight=wn, bias=bn), 1, 10, 2)[0]
    record("readout_norm_B8_L4096_width2048", ms, B * L * H * dd, B * L * H * dd * (4 + 2 + 4) + H * dd * 8)
    del q, k, v, g, o, o2, ogate

    # --- packed varlen selective, L=131072, 32 sequences, D=4096, N=16
    Lt, D, N, ns = 131072, 4096, 16, 32
    lengths = synth.varlen_lengths(Lt, ns, 1004)
    cu = torch.from_numpy(synth.cu_seqlens_from_lengths(lengths)).to(device)
    x, z = randn((1, Lt, D)), randn((1, Lt, D))
    A = torch.from_numpy(synth.multiscale_A(D, N, 4)).to(device)
    delta0 = torch.exp(torch.empty(D, device=device).uniform_(np.log(1e-3), np.log(1e-1), generator=gen))
    delta = torch.exp(randn((1, Lt, D), std=0.1, dtype=torch.float32)) * delta0
    dt = (delta + torch.log(-torch.expm1(-delta))).to(torch.bfloat16)
    del delta
    Bm, Cm = randn((1, Lt, N), std=1.0 / N), randn((1, Lt, N), std=1.0 / N)
    Dskip = torch.ones(D, device=device)
    ms = time_calls(lambda kk: ssd.selective_scan(x, dt, A, Bm, Cm, Dskip=Dskip, z=z, cu_seqlens=cu,
                                                  check_cu_seqlens=False), 1, 5, 1)[0]
    record("selective_varlen_L131072_D4096_N16_32seq", ms, Lt * D * N, selective_bytes(1, Lt, D, N, nseq=ns))

    # --- gradients of the packed varlen scan (dy ~ N(0, 1))
    dy = randn((1, Lt, D))
    ms = time_calls(lambda kk: ssd.selective_scan_backward(x, dt, A, Bm, Cm, dy, Dskip=Dskip, z=z, cu_seqlens=cu,
                                                           check_cu_seqlens=False), 1, 2, 1)[0]
    record("selective_backward_varlen_L131072_D4096_N16_32seq", ms, Lt * D * N, selective_bwd_bytes(1, Lt, D, N))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-forms", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="first run a plain device-to-device tensor copy of this many MiB three times (a known-size "
                         "kernel for scaling hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the scans shard with no communication across channels, batches "
              "and heads, and this build runs on a single MI355X; use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head, host_inputs = headline(args, device)
    ms = head["ms"]
    value = head["updates"] / (ms * 1e-3)
    call_s = ms * 1e-3
    achieved_tflops = head["updates"] * SELECTIVE_FLOPS_PER_UPDATE / call_s / 1e12
    hbm_gbs = head["bytes"] / call_s / 1e9
    print(f"# headline: {ms:.4f} ms/step (host clock {head['host_ms']:.4f}), {value:.3e} upd/s, "
          f"{hbm_gbs:.0f} GB/s", file=sys.stderr, flush=True)

    line = {
        "metric": "scan state-updates/s + achieved HBM GB/s (% of peak), fwd, 1 MI355X",
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "multi-scale selective scan, B=4 L=2048 D=1536 N=16, 4 scales, bf16 in, "
                               "fp32 state and out, softplus dt, skip D=1, silu(z) gate",
                   "B": 4, "L": 2048, "D": 1536, "N": 16, "input_dtype": "bf16", "output_dtype": "f32"},
        "hbm": {"achieved_gbs": hbm_gbs, "peak_gbs": HBM_PEAK_GBS, "frac": hbm_gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": head["bytes"]},
        "roofline": {"bound": "alu", "achieved": achieved_tflops, "peak": FP32_SCALAR_FMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tflops / FP32_SCALAR_FMA_TFLOPS,
                     "peak_basis": "fp32 FMA without packed instructions: 256 CU x 64 lanes x 2 flop x 2.4 GHz; "
                                   "published 157.3 counts packed FMA",
                     "published_peak": FP32_VECTOR_TFLOPS,
                     "traffic": profiled_traffic("selective_scan_B4_L2048_D1536_N16.md",
                                                 ["selective_state_space_diag_amd/csrc/selective.hip",
                                                  "selective_state_space_diag_amd/csrc/common.hpp"]),
                     "kernel": "selective scan call: aggregate + carry + scan kernels",
                     "flops_per_update": SELECTIVE_FLOPS_PER_UPDATE, "ms_per_call": ms},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(host_inputs)
    if not args.no_forms:
        line["forms"] = forms(args, device)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
