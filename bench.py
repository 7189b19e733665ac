#!/usr/bin/env python3
"""Throughput of the gfx950 gated diagonal linear-recurrence scans on one MI355X.

Headline (the JSON ``value``): the packed variable-length multi-scale selective scan, L = 131072
tokens in 32 sequences (lengths log-uniform in [512, 16384], rescaled to sum to L), D = 4096 channels,
N = 16 states, 4 scales, bf16 inputs, fp32 state and output, in state updates per second.  One step is
one full scan (softplus of dt, discretisation, recurrence with a state reset at every sequence start,
readout, skip and silu gate) over inputs already resident in HBM.  The 5.4 GB it moves per step is 21
times the 256 MB Infinity Cache, so one input set suffices.

The JSON line also carries:
  roofline      the headline call against the HBM roofline (algorithmic bytes / time), with per-step
                HIP-event timing on the stream the kernels run on, median and min, the fraction of the
                measured device-copy rate, the fp32 ALU fraction beside it, and the HBM traffic recorded
                by rocprofv3 counters (profiles/), null once the kernel sources changed;
  cpu_baseline  the fp64 CPU oracle on a sample of the same workload (512 channels, every sequence),
                timed with one thread and with every host thread it may use (reported, not a target);
  forms         the other workloads with their own throughput, GB/s, median and min.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-forms] [--no-cpu-baseline]
                       [--only NAME] [--copy-calibration-mb MB]
``--only NAME`` runs one workload (``headline`` or a form name) and prints its record alone: the
profiling commands under profiles/ use it.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
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

HEADLINE = dict(L=131072, D=4096, N=16, nseq=32, scales=4, seed=1004)

_CSRC = "selective_state_space_diag_amd/csrc/"
_SEL_SOURCES = [_CSRC + f for f in ("selective.hip", "common.hpp", "kernels.hpp")]
_H2_SOURCES = [_CSRC + f for f in ("hgrn2.hip", "h2_layout.hpp", "common.hpp", "kernels.hpp")]
_SCAN1_SOURCES = [_CSRC + f for f in ("scan1.hip", "common.hpp", "kernels.hpp")]
_SWEEP_SOURCES = [_CSRC + f for f in ("hgrn2_sweep.hip", "common.hpp", "kernels.hpp")]
_CONV_SOURCES = [_CSRC + f for f in ("conv1d.hip", "common.hpp", "kernels.hpp")]
_NORM_SOURCES = [_CSRC + f for f in ("norm.hip", "common.hpp", "kernels.hpp")]
# Workload -> (summary file under profiles/, what one call is, the kernel sources the summary's counter
# figures hold for: a figure is used only while the sha256 of these files is the one stored with it).
PROFILES = {
    "headline": ("selective_varlen_L131072_D4096_N16.md",
                 "Packed varlen selective scan, L=131072 tokens in 32 sequences, D=4096, N=16, bf16 in, fp32 out; "
                 "one call = planner + phase 1 (first pieces and aggregate units) + piece fold + phase 2 scan kernels", _SEL_SOURCES),
    "selective_B4_L2048_D1536_N16": ("selective_scan_B4_L2048_D1536_N16.md",
                                     "Batched selective scan B=4 L=2048 D=1536 N=16, bf16 in, fp32 out; one call = "
                                     "aggregate + carry + scan kernels", _SEL_SOURCES),
    "hgrn2_bf16_B8_H16_d128_L4096": ("hgrn2_scan_B8_H16_d128_L4096.md",
                                     "HGRN2 scan B=8 H=16 d=128 L=4096, bf16 in, fp32 out, lower bound 0.5; one call "
                                     "= one chunked MFMA kernel", _H2_SOURCES),
    "hgrn2_lb0_bf16_B8_H16_d128_L4096": ("hgrn2_lb0_scan_B8_H16_d128_L4096.md",
                                         "HGRN2 scan B=8 H=16 d=128 L=4096, bf16 in, fp32 out, lower bound 0 (the "
                                         "chunked MFMA kernel with the per-chunk decay check)", _H2_SOURCES),
    "rglru_bf16_B8_L8192_D2560": ("rglru_scan_B8_L8192_D2560.md",
                                  "RG-LRU scan B=8 L=8192 D=2560, bf16 in, fp32 out; one call = one lookback kernel",
                                  _SCAN1_SOURCES),
    "rglru_gated_bf16_B8_L8192_D2560": ("rglru_gated_scan_B8_L8192_D2560.md",
                                        "RG-LRU scan with the gelu(gate) output multiply, B=8 L=8192 D=2560, bf16 in, "
                                        "fp32 out; one call = one lookback kernel", _SCAN1_SOURCES),
    "rglru_fp32_B2_L128_D64": ("rglru_scan_B2_L128_D64_fp32.md",
                               "RG-LRU scan B=2 L=128 D=64 fp32 (one-pass short kernel), called from Python and 64 "
                               "times from a HIP graph", _SCAN1_SOURCES),
    "rglru_backward": ("rglru_backward_B8_L8192_D2560.md",
                       "RG-LRU backward B=8 L=8192 D=2560 bf16: a forward with chunk states, then the backward with "
                       "them and without them (record pass)", _SCAN1_SOURCES),
    "minmax": ("minmax_B8_L8192_D2560.md",
               "MinMax scan B=8 L=8192 D=2560 bf16, a forward with chunk states, and the backward with them and "
               "without them (record pass)", _SCAN1_SOURCES),
    "rglru_decode": ("rglru_update_B256_D2560.md",
                     "RG-LRU decode steps B=256 D=2560 bf16: 256 steps from Python, then from a HIP graph, then a "
                     "same-size device copy from a graph", _SCAN1_SOURCES),
    "causal_conv1d_bf16_B8_L8192_D2560_W4": ("causal_conv1d_B8_L8192_D2560_W4.md",
                                             "Causal depthwise conv W=4, B=8 L=8192 D=2560 bf16; one call = one "
                                             "kernel", _CONV_SOURCES),
    "selective_backward_bf16_B4_L2048_D1536_N16": ("selective_backward_B4_L2048_D1536_N16.md",
                                                   "Selective scan backward B=4 L=2048 D=1536 N=16 bf16 in, fp32 "
                                                   "gradients", _SEL_SOURCES),
    "selective_backward_varlen_L131072_D4096_N16_32seq": ("selective_backward_varlen_L131072_D4096_N16.md",
                                                          "Packed varlen selective scan backward, L=131072 in 32 "
                                                          "sequences, D=4096 N=16 bf16", _SEL_SOURCES),
    "hgrn2_backward_bf16_B8_H16_d128_L4096": ("hgrn2_backward_B8_H16_d128_L4096.md",
                                              "HGRN2 backward B=8 H=16 d=128 L=4096 bf16, the forward output given "
                                              "(one forward call first); one call = transposes, three chunked "
                                              "MFMA passes, the gate-gradient sums",
                                              _H2_SOURCES + [_CSRC + "hgrn2_sweep.hip"]),
    "hgrn2_key_gate_bf16_B8_H16_d128_L4096": ("hgrn2_key_gate_scan_B8_H16_d128_L4096.md",
                                              "HGRN2 scan with the gate on the key axis, B=8 H=16 d=128 L=4096 bf16 "
                                              "in, fp32 out, lower bound 0.5; one call = one chunked MFMA kernel",
                                              _H2_SOURCES + [_CSRC + "hgrn2_sweep.hip"]),
    "readout_norm_B8_L4096_width2048": ("readout_norm_B8_L4096_width2048.md",
                                        "Readout LayerNorm and silu gate over 32768 rows of 2048 features (one HGRN2 "
                                        "forward call first)", _NORM_SOURCES),
}


def sources_sha256(sources):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


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


def profiled_traffic(workload):
    """HBM bytes per call recorded by rocprofv3 counter runs in the workload's summary under profiles/,
    if its kernel sources are unchanged since (their sha256 is stored with the figure); else None."""
    import re
    if workload not in PROFILES:
        return None
    fname, _, sources = PROFILES[workload]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- profile-data: (\{.*\}) -->", open(path).read())
    if not m:
        return None
    data = json.loads(m.group(1))
    if data.get("kernel_sources_sha256") != sources_sha256(sources):
        return None
    return data.get("traffic_bytes_per_call")


# ----------------------------------------------------------------------------- timing helpers
WARM_SECONDS = 0.3  # untimed running before each timed region, so clocks have left their idle state


def time_calls(fn, n_sets, steps, warmup):
    """Run ``fn(i % n_sets)`` at least ``warmup`` times and for at least WARM_SECONDS, then time ``steps``
    back-to-back calls with a HIP event between consecutive calls, on torch's current stream (the stream
    the library launches on), synchronizing before and after.  Returns a dict: ms (mean per step over the
    timed region), median_ms, min_ms (per step), host_ms (host clock per step)."""
    import torch
    t_warm = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_warm < WARM_SECONDS:
        fn(i % n_sets)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn(i % n_sets)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return dict(ms=ev[0].elapsed_time(ev[-1]) / steps, median_ms=statistics.median(per), min_ms=min(per),
                host_ms=wall / steps)


def copy_rate_gbs(device, mib=2048, reps=10):
    """Device-to-device copy rate (read + write bytes / time) of a plain torch copy of ``mib`` MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=device)
    dst = torch.empty_like(src)
    t = time_calls(lambda k: dst.copy_(src), 1, reps, 2)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (t["median_ms"] * 1e-3) / 1e9


def dev_bf16(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class Gen:
    """Seeded normal / uniform draws on the GPU (torch's Philox generator), for the large workloads."""

    def __init__(self, device, seed):
        import torch
        self.torch = torch
        self.device = device
        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed)

    def randn(self, shape, std=1.0, mean=0.0, dtype=None):
        t = self.torch.randn(shape, generator=self.g, device=self.device, dtype=self.torch.float32)
        t = t * std + mean
        return t.to(dtype or self.torch.bfloat16)

    def uniform(self, shape, lo, hi):
        return self.torch.empty(shape, device=self.device).uniform_(lo, hi, generator=self.g)


def selective_gpu_inputs(gen, B, L, D, N, scales=4, structured_A=True):
    """The selective workload's distributions drawn on the GPU: A multi-scale (or unstructured),
    delta = delta0[d] exp(N(0, 0.1)) passed as dt = softplus^-1(delta) in bf16, x, z ~ N(0, 1),
    B, C ~ N(0, 1/N), skip D = 1."""
    import torch
    from selective_state_space_diag_amd import synth
    x, z = gen.randn((B, L, D)), gen.randn((B, L, D))
    if structured_A:
        A = torch.from_numpy(synth.multiscale_A(D, N, scales)).to(gen.device)
    else:
        A = -torch.exp(gen.uniform((D, N), np.log(0.5), np.log(64.0)))
    delta0 = torch.exp(gen.uniform((D,), np.log(1e-3), np.log(1e-1)))
    dt = torch.empty((B, L, D), device=gen.device, dtype=torch.bfloat16)
    for b in range(B):  # row by row: the fp32 intermediates of one batch row at a time
        delta = torch.exp(gen.randn((1, L, D), std=0.1, dtype=torch.float32)) * delta0
        dt[b] = (delta + torch.log(-torch.expm1(-delta))).to(torch.bfloat16)[0]
        del delta
    Bm, Cm = gen.randn((B, L, N), std=1.0 / N), gen.randn((B, L, N), std=1.0 / N)
    return dict(x=x, z=z, A=A, dt=dt, Bm=Bm, Cm=Cm, Dskip=torch.ones(D, device=gen.device))


def record_of(t, updates, nbytes, extra=None, name=None):
    d = dict(ms=round(t["ms"], 5), median_ms=round(t["median_ms"], 5), min_ms=round(t["min_ms"], 5),
             state_updates_per_s=updates / (t["ms"] * 1e-3), hbm_gbs=nbytes / (t["ms"] * 1e-3) / 1e9,
             hbm_frac=nbytes / (t["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, algorithmic_bytes=nbytes,
             state_updates=updates)
    if extra:
        d.update(extra)
    if name:
        print(f"# {name}: {t['ms']:.4f} ms (median {t['median_ms']:.4f}, min {t['min_ms']:.4f})  "
              f"{d['state_updates_per_s']:.3e} upd/s  {d['hbm_gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    return d


# ----------------------------------------------------------------------------- headline
def headline(args, device):
    """The packed varlen selective scan (L = 131072, 32 sequences, D = 4096, N = 16)."""
    import torch
    import selective_state_space_diag_amd as ssd
    from selective_state_space_diag_amd import synth

    c = HEADLINE
    Lt, D, N, ns = c["L"], c["D"], c["N"], c["nseq"]
    lengths = synth.varlen_lengths(Lt, ns, c["seed"])
    cu_host = synth.cu_seqlens_from_lengths(lengths)
    cu = torch.from_numpy(cu_host).to(device)
    inp = selective_gpu_inputs(Gen(device, c["seed"]), 1, Lt, D, N, c["scales"])

    def step(i):
        return ssd.selective_scan(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], Dskip=inp["Dskip"],
                                  z=inp["z"], cu_seqlens=cu, check_cu_seqlens=False)

    t = time_calls(step, 1, args.steps, args.warmup)
    updates = Lt * D * N
    nbytes = selective_bytes(1, Lt, D, N, nseq=ns)
    return dict(t=t, updates=updates, bytes=nbytes, inputs=inp, cu=cu_host, lengths=lengths)


def cpu_baseline(head, max_threads=16):
    """The fp64 oracle (unchanged, as the tests use it) on a bounded sample of the headline workload:
    512 channels (every 8th, so all four scale blocks) over all 131072 rows and all 32 sequences, the
    same input bits as the GPU run; timed once with one thread and once split over the host threads
    this process may use (at most 16, the host share of one GPU), one thread per channel group."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    inp = head["inputs"]
    D = inp["x"].shape[2]
    ds = torch.arange(0, D, 8, device=inp["x"].device)
    h = lambda t: t[:, :, ds].double().cpu().numpy()
    x, dt, z = h(inp["x"]), h(inp["dt"]), h(inp["z"])
    Bm, Cm = inp["Bm"].double().cpu().numpy(), inp["Cm"].double().cpu().numpy()
    A = inp["A"][ds].double().cpu().numpy()
    Dskip = inp["Dskip"][ds].double().cpu().numpy()
    cu = head["cu"]
    oracle.lib()
    nch = len(ds)
    updates = x.shape[1] * nch * A.shape[1]

    def run(sl):
        oracle.selective_scan(np.ascontiguousarray(x[:, :, sl]), np.ascontiguousarray(dt[:, :, sl]), A[sl], Bm, Cm,
                              Dskip=Dskip[sl], z=np.ascontiguousarray(z[:, :, sl]), dt_softplus=True, cu_seqlens=cu)

    t0 = time.perf_counter()
    run(slice(0, nch))
    one = time.perf_counter() - t0
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    nthr = max(1, min(avail, max_threads))
    groups = [slice(i * nch // nthr, (i + 1) * nch // nthr) for i in range(nthr)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(run, groups))
    many = time.perf_counter() - t0
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return dict(value=updates / many, unit="state-updates/s", cores=nthr, kind="oracle",
                sample=f"512 of 4096 channels (every 8th) of the headline workload, all 131072 rows and 32 "
                       f"sequences, {updates} state updates, fp64; {many:.2f} s on {nthr} threads, "
                       f"{one:.2f} s on 1 thread",
                single_thread_value=updates / one, host_nproc=os.cpu_count(), host_threads_allowed=avail,
                cpu_model=model)


# ----------------------------------------------------------------------------- other workloads
def form_selective_cfg(args, device):
    """The batched selective scan B=4 L=2048 D=1536 N=16, three rotating input sets (126 MB each, so the
    256 MB Infinity Cache cannot hold the working set)."""
    import torch
    import selective_state_space_diag_amd as ssd
    from selective_state_space_diag_amd import synth
    B, L, D, N = 4, 2048, 1536, 16
    sets = []
    for k in range(3):
        inp = synth.workload_inputs("selective", seed=1001 + 100 * k)
        t = {n: dev_bf16(v.data, device) for n, v in inp.t.items()}
        sets.append(dict(t=t, A=torch.from_numpy(inp.p["A"]).to(device),
                         Dskip=torch.from_numpy(inp.p["Dskip"]).to(device)))

    def step(i):
        s = sets[i]
        t = s["t"]
        return ssd.selective_scan(t["x"], t["dt"], s["A"], t["Bm"], t["Cm"], Dskip=s["Dskip"], z=t["z"])

    t = time_calls(step, 3, 50, 5)
    return record_of(t, B * L * D * N, selective_bytes(B, L, D, N),
                     dict(alu_tflops=B * L * D * N * SELECTIVE_FLOPS_PER_UPDATE / (t["ms"] * 1e-3) / 1e12),
                     "selective_B4_L2048_D1536_N16")


def form_selective_unstructured(args, device):
    import selective_state_space_diag_amd as ssd
    B, L, D, N = 4, 2048, 1536, 16
    inp = selective_gpu_inputs(Gen(device, 7), B, L, D, N, structured_A=False)
    t = time_calls(lambda k: ssd.selective_scan(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"],
                                                Dskip=inp["Dskip"], z=inp["z"]), 1, 30, 3)
    return record_of(t, B * L * D * N, selective_bytes(B, L, D, N), None,
                     "selective_unstructured_A_B4_L2048_D1536_N16")


def form_selective_backward(args, device):
    import selective_state_space_diag_amd as ssd
    B, L, D, N = 4, 2048, 1536, 16
    gen = Gen(device, 8)
    inp = selective_gpu_inputs(gen, B, L, D, N)
    dy = gen.randn((B, L, D))
    t = time_calls(lambda k: ssd.selective_scan_backward(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], dy,
                                                         Dskip=inp["Dskip"], z=inp["z"]), 1, 10, 2)
    return record_of(t, B * L * D * N, selective_bwd_bytes(B, L, D, N), None, "selective_backward_bf16_B4_L2048_D1536_N16")


def form_rglru_small(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    B, L, D = 2, 128, 64
    gen = Gen(device, 9)
    x, r, i = (gen.randn((B, L, D), dtype=torch.float32) for _ in range(3))
    a_log = torch.log(gen.uniform((D,), 0.9, 0.999))
    t = time_calls(lambda k: ssd.rglru_scan(x, r, i, a_log, 8.0), 1, 50, 5)
    out = {"rglru_fp32_B2_L128_D64": record_of(t, B * L * D, rglru_bytes(B, L, D, 4, 4), None,
                                               "rglru_fp32_B2_L128_D64")}
    # the same call 64 times from one HIP graph: the device time of a call without the host's
    # per-call cost
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        ssd.rglru_scan(x, r, i, a_log, 8.0)  # workspace for the capture stream, outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(64):
                ssd.rglru_scan(x, r, i, a_log, 8.0)
    torch.cuda.synchronize()
    t = time_calls(lambda k: graph.replay(), 1, 10, 2)
    t = {k: v / 64 for k, v in t.items()}
    out["rglru_fp32_B2_L128_D64_hipgraph"] = record_of(t, B * L * D, rglru_bytes(B, L, D, 4, 4),
                                                       dict(us_per_call=t["ms"] * 1e3),
                                                       "rglru_fp32_B2_L128_D64_hipgraph")
    return out


def _rglru_big(device, seed):
    import torch
    B, L, D = 8, 8192, 2560
    gen = Gen(device, seed)
    x, r, i = (gen.randn((B, L, D)) for _ in range(3))
    a_log = torch.log(gen.uniform((D,), 0.9, 0.999))
    return gen, (B, L, D), x, r, i, a_log


def form_rglru(args, device):
    import selective_state_space_diag_amd as ssd
    _, (B, L, D), x, r, i, a_log = _rglru_big(device, 10)
    t = time_calls(lambda k: ssd.rglru_scan(x, r, i, a_log, 8.0), 1, 10, 2)
    return record_of(t, B * L * D, rglru_bytes(B, L, D), None, "rglru_bf16_B8_L8192_D2560")


def form_rglru_gated(args, device):
    import selective_state_space_diag_amd as ssd
    gen, (B, L, D), x, r, i, a_log = _rglru_big(device, 11)
    gt = gen.randn((B, L, D))
    t = time_calls(lambda k: ssd.rglru_scan(x, r, i, a_log, 8.0, gate=gt), 1, 10, 2)
    return record_of(t, B * L * D, rglru_gated_bytes(B, L, D), None, "rglru_gated_bf16_B8_L8192_D2560")


def form_rglru_noalloc(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    _, (B, L, D), x, r, i, a_log = _rglru_big(device, 10)
    y = torch.empty((B, L, D), device=device)
    t = time_calls(lambda k: ssd.rglru_scan_noalloc(x, r, i, a_log, 8.0, y=y), 1, 10, 2)
    return record_of(t, B * L * D, rglru_bytes(B, L, D), None, "rglru_noalloc_bf16_B8_L8192_D2560")


def form_rglru_backward(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    gen, (B, L, D), x, r, i, a_log = _rglru_big(device, 12)
    dy = gen.randn((B, L, D))
    cs = torch.empty(ssd.chunk_states_shape(B, L, D), device=device)
    ssd.rglru_scan(x, r, i, a_log, 8.0, chunk_states=cs)
    out = {}
    t = time_calls(lambda k: ssd.rglru_scan_backward(x, r, i, a_log, 8.0, dy, chunk_states=cs), 1, 5, 1)
    out["rglru_backward_bf16_B8_L8192_D2560"] = record_of(t, B * L * D, rglru_bwd_bytes(B, L, D) + cs.numel() * 4,
                                                          None, "rglru_backward_bf16_B8_L8192_D2560")
    t = time_calls(lambda k: ssd.rglru_scan_backward(x, r, i, a_log, 8.0, dy), 1, 5, 1)
    out["rglru_backward_recompute_bf16_B8_L8192_D2560"] = record_of(
        t, B * L * D, rglru_bwd_bytes(B, L, D), None, "rglru_backward_recompute_bf16_B8_L8192_D2560")
    return out


def form_minmax(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    gen, (B, L, D), x, r, i, a_log = _rglru_big(device, 13)
    out = {}
    t = time_calls(lambda k: ssd.minmax_scan(r, i), 1, 10, 2)
    out["minmax_bf16_B8_L8192_D2560"] = record_of(t, B * L * D, minmax_bytes(B, L, D), None,
                                                  "minmax_bf16_B8_L8192_D2560")
    dy = gen.randn((B, L, D))
    cs = torch.empty(ssd.chunk_states_shape(B, L, D), device=device)
    ssd.minmax_scan(r, i, chunk_states=cs)
    t = time_calls(lambda k: ssd.minmax_scan_backward(r, i, dy, chunk_states=cs), 1, 5, 1)
    out["minmax_backward_bf16_B8_L8192_D2560"] = record_of(t, B * L * D, minmax_bwd_bytes(B, L, D) + cs.numel() * 4,
                                                           None, "minmax_backward_bf16_B8_L8192_D2560")
    t = time_calls(lambda k: ssd.minmax_scan_backward(r, i, dy), 1, 5, 1)
    out["minmax_backward_recompute_bf16_B8_L8192_D2560"] = record_of(
        t, B * L * D, minmax_bwd_bytes(B, L, D), None, "minmax_backward_recompute_bf16_B8_L8192_D2560")
    return out


def form_conv(args, device):
    import selective_state_space_diag_amd as ssd
    gen, (B, L, D), x, r, i, a_log = _rglru_big(device, 14)
    W = 4
    wconv = gen.uniform((D, W), -0.5, 0.5)
    bconv = gen.uniform((D,), -0.5, 0.5)
    t = time_calls(lambda k: ssd.causal_conv1d(x, wconv, bias=bconv), 1, 10, 2)
    return record_of(t, B * L * D, conv_bytes(B, L, D, W), None, "causal_conv1d_bf16_B8_L8192_D2560_W4")


def form_rglru_decode(args, device):
    """256 RG-LRU decode steps at B = 256, D = 2560 carrying the state: one launch per step from Python,
    and the same 256 launches captured once in a HIP graph and replayed."""
    import torch
    import selective_state_space_diag_amd as ssd
    B, D, S = 256, 2560, 256
    gen = Gen(device, 15)
    xs, rs, is_ = (gen.randn((S, B, D)) for _ in range(3))
    a_log = torch.log(gen.uniform((D,), 0.9, 0.999))
    state = torch.zeros(B, D, device=device)

    def decode(k):
        for s in range(S):
            ssd.rglru_update(xs[s], rs[s], is_[s], a_log, 8.0, state)

    per_step_bytes = B * D * (3 * 2 + 4 + 4 + 4)
    out = {}
    t = time_calls(decode, 1, 3, 1)
    out["rglru_decode_B256_D2560_256steps"] = record_of(t, B * D * S, per_step_bytes * S,
                                                        dict(us_per_step=t["ms"] * 1e3 / S),
                                                        "rglru_decode_B256_D2560_256steps")
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
    t = time_calls(lambda k: graph.replay(), 1, 5, 1)
    # reference: a plain device copy moving the same bytes per step (half read, half written), 256
    # times from one HIP graph: the latency floor of one round trip to memory at this size
    src = torch.empty(per_step_bytes // 8, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    cgraph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        dst.copy_(src)
        torch.cuda.synchronize()
        with torch.cuda.graph(cgraph, stream=cap):
            for _ in range(S):
                dst.copy_(src)
    torch.cuda.synchronize()
    tc = time_calls(lambda k: cgraph.replay(), 1, 5, 1)
    out["rglru_decode_B256_D2560_256steps_hipgraph"] = record_of(
        t, B * D * S, per_step_bytes * S, dict(us_per_step=t["ms"] * 1e3 / S, same_bytes_copy_us=tc["ms"] * 1e3 / S),
        "rglru_decode_B256_D2560_256steps_hipgraph")
    print(f"#   same-size device copy from a graph: {tc['ms'] * 1e3 / S:.2f} us per step", file=sys.stderr, flush=True)
    return out


def _hgrn2_inputs(device, seed):
    B, L, H, dd = 8, 4096, 16, 128
    gen = Gen(device, seed)
    q, k, v = (gen.randn((B, L, H, dd), std=dd ** -0.5) for _ in range(3))
    g = gen.randn((B, L, H, dd), mean=2.0)
    return gen, (B, L, H, dd), q, k, v, g


def form_hgrn2(args, device):
    import selective_state_space_diag_amd as ssd
    _, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    t = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.5), 1, 10, 2)
    flops = 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)  # chunked form at chunk 64
    return record_of(t, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
                     dict(mfma_equiv_tflops=flops / (t["ms"] * 1e-3) / 1e12,
                          mfma_util=flops / (t["ms"] * 1e-3) / 1e12 / BF16_MFMA_TFLOPS),
                     "hgrn2_bf16_B8_H16_d128_L4096")


def form_hgrn2_lb0(args, device):
    import selective_state_space_diag_amd as ssd
    _, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    t = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.0), 1, 10, 2)
    flops = 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)  # chunked form at chunk 64
    return record_of(t, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
                     dict(mfma_equiv_tflops=flops / (t["ms"] * 1e-3) / 1e12,
                          mfma_util=flops / (t["ms"] * 1e-3) / 1e12 / BF16_MFMA_TFLOPS),
                     "hgrn2_lb0_bf16_B8_H16_d128_L4096")


def form_hgrn2_backward(args, device):
    import selective_state_space_diag_amd as ssd
    gen, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    do = gen.randn((B, L, H, dd), std=dd ** -0.5)
    o = ssd.hgrn2_scan(q, k, v, g, 0.5)
    t = time_calls(lambda kk: ssd.hgrn2_scan_backward(q, k, v, g, 0.5, do, o=o), 1, 10, 2)
    # three adjoint passes in the chunked form (dq, dv, dk), each the forward's products at chunk 64
    flops = 3 * 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)
    return record_of(t, B * L * H * dd * dd, hgrn2_bwd_bytes(B, L, H, dd),
                     dict(mfma_equiv_tflops=flops / (t["ms"] * 1e-3) / 1e12,
                          mfma_util=flops / (t["ms"] * 1e-3) / 1e12 / BF16_MFMA_TFLOPS),
                     "hgrn2_backward_bf16_B8_H16_d128_L4096")


def form_hgrn2_backward_lb0(args, device):
    import selective_state_space_diag_amd as ssd
    gen, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    do = gen.randn((B, L, H, dd), std=dd ** -0.5)
    o = ssd.hgrn2_scan(q, k, v, g, 0.0)
    t = time_calls(lambda kk: ssd.hgrn2_scan_backward(q, k, v, g, 0.0, do, o=o), 1, 10, 2)
    flops = 3 * 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)
    return record_of(t, B * L * H * dd * dd, hgrn2_bwd_bytes(B, L, H, dd),
                     dict(mfma_equiv_tflops=flops / (t["ms"] * 1e-3) / 1e12,
                          mfma_util=flops / (t["ms"] * 1e-3) / 1e12 / BF16_MFMA_TFLOPS),
                     "hgrn2_backward_lb0_bf16_B8_H16_d128_L4096")


def form_hgrn2_key(args, device):
    import selective_state_space_diag_amd as ssd
    _, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    t = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.5, gate_axis="key"), 1, 10, 2)
    flops = 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)  # chunked form at chunk 64, as for the row gate
    return record_of(t, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
                     dict(mfma_equiv_tflops=flops / (t["ms"] * 1e-3) / 1e12,
                          mfma_util=flops / (t["ms"] * 1e-3) / 1e12 / BF16_MFMA_TFLOPS),
                     "hgrn2_key_gate_bf16_B8_H16_d128_L4096")


def form_hgrn2_key_lb0(args, device):
    import selective_state_space_diag_amd as ssd
    _, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    t = time_calls(lambda kk: ssd.hgrn2_scan(q, k, v, g, 0.0, gate_axis="key"), 1, 10, 2)
    flops = 2 * B * L * H * (2 * 64 * dd + 2 * dd * dd)  # chunked form at chunk 64
    return record_of(t, B * L * H * dd * dd, hgrn2_bytes(B, L, H, dd),
                     dict(mfma_equiv_tflops=flops / (t["ms"] * 1e-3) / 1e12,
                          mfma_util=flops / (t["ms"] * 1e-3) / 1e12 / BF16_MFMA_TFLOPS),
                     "hgrn2_key_gate_lb0_bf16_B8_H16_d128_L4096")


def form_readout_norm(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    gen, (B, L, H, dd), q, k, v, g = _hgrn2_inputs(device, 16)
    o = ssd.hgrn2_scan(q, k, v, g, 0.5)
    del q, k, v, g
    ogate = gen.randn((B, L, H * dd))
    wn, bn = torch.ones(H * dd, device=device), torch.zeros(H * dd, device=device)
    o2 = o.view(B, L, H * dd)
    t = time_calls(lambda kk: ssd.readout_norm(o2, gate=ogate, weight=wn, bias=bn), 1, 10, 2)
    return record_of(t, B * L * H * dd, B * L * H * dd * (4 + 2 + 4) + H * dd * 8, None,
                     "readout_norm_B8_L4096_width2048")


def form_selective_varlen_backward(args, device):
    import torch
    import selective_state_space_diag_amd as ssd
    from selective_state_space_diag_amd import synth
    c = HEADLINE
    Lt, D, N, ns = c["L"], c["D"], c["N"], c["nseq"]
    cu = torch.from_numpy(synth.cu_seqlens_from_lengths(synth.varlen_lengths(Lt, ns, c["seed"]))).to(device)
    gen = Gen(device, 17)
    inp = selective_gpu_inputs(gen, 1, Lt, D, N)
    dy = gen.randn((1, Lt, D))
    t = time_calls(lambda kk: ssd.selective_scan_backward(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["Cm"], dy,
                                                          Dskip=inp["Dskip"], z=inp["z"], cu_seqlens=cu,
                                                          check_cu_seqlens=False), 1, 2, 1)
    return record_of(t, Lt * D * N, selective_bwd_bytes(1, Lt, D, N), None,
                     "selective_backward_varlen_L131072_D4096_N16_32seq")


FORMS = {
    "selective_B4_L2048_D1536_N16": form_selective_cfg,
    "selective_unstructured_A_B4_L2048_D1536_N16": form_selective_unstructured,
    "selective_backward_bf16_B4_L2048_D1536_N16": form_selective_backward,
    "rglru_fp32_B2_L128_D64": form_rglru_small,
    "rglru_bf16_B8_L8192_D2560": form_rglru,
    "rglru_gated_bf16_B8_L8192_D2560": form_rglru_gated,
    "rglru_noalloc_bf16_B8_L8192_D2560": form_rglru_noalloc,
    "rglru_backward": form_rglru_backward,
    "minmax": form_minmax,
    "causal_conv1d_bf16_B8_L8192_D2560_W4": form_conv,
    "rglru_decode": form_rglru_decode,
    "hgrn2_bf16_B8_H16_d128_L4096": form_hgrn2,
    "hgrn2_lb0_bf16_B8_H16_d128_L4096": form_hgrn2_lb0,
    "hgrn2_backward_bf16_B8_H16_d128_L4096": form_hgrn2_backward,
    "hgrn2_backward_lb0_bf16_B8_H16_d128_L4096": form_hgrn2_backward_lb0,
    "hgrn2_key_gate_bf16_B8_H16_d128_L4096": form_hgrn2_key,
    "hgrn2_key_gate_lb0_bf16_B8_H16_d128_L4096": form_hgrn2_key_lb0,
    "readout_norm_B8_L4096_width2048": form_readout_norm,
    "selective_backward_varlen_L131072_D4096_N16_32seq": form_selective_varlen_backward,
}


def run_form(name, args, device):
    """Records of one form (a dict name -> record); frees its device memory afterwards."""
    import torch
    r = FORMS[name](args, device)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    recs = r if isinstance(r, dict) and "ms" not in r else {name: r}
    for n, rec in recs.items():
        if n in PROFILES:
            rec["traffic_bytes"] = profiled_traffic(n)
    return recs


# ----------------------------------------------------------------------------- profile summaries
def _csv_rows(folder, suffix):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _short_kernel(name):
    """Kernel name without 'void', the library's namespaces and the parameter list."""
    n = name.replace("void ", "", 1).replace("ssd::(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def _last_json(path):
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            try:
                rec = json.loads(line)
            except ValueError:
                pass
    return rec


def summarize_profile(folder, workload):
    """Markdown summary of the rocprofv3 runs of one workload in ``folder``:
    trace/ (--kernel-trace --stats, csv) with the bench output in trace.log, pmc_FETCH_SIZE/ and
    pmc_WRITE_SIZE/ (each run started with --copy-calibration-mb, the size printed in its log),
    optionally pmc_SQ/ (instruction counters), and commands.txt (the commands that made them).
    Only the library's kernels (namespace ssd) are listed.  Per-call figures count each kernel as many
    times per call as its dispatches divided by those of the kernel with the largest total time."""
    import re
    fname, title, sources = PROFILES[workload]
    lib = lambda n: "ssd::" in (n or "")
    # durations: kernel trace and rocprofv3's own statistics
    dur, shape = {}, {}
    for r in _csv_rows(os.path.join(folder, "trace"), "kernel_trace.csv"):
        n = r.get("Kernel_Name")
        if not lib(n):
            continue
        dur.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        shape[n] = (r.get("Grid_Size") or r.get("Grid_Size_X"), r.get("Workgroup_Size") or r.get("Workgroup_Size_X"),
                    r.get("VGPR_Count") or r.get("Arch_VGPR_Count"), r.get("LDS_Block_Size") or r.get("LDS_Size"))
    stats = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in _csv_rows(os.path.join(folder, "trace"), "kernel_stats.csv")
             if lib(r.get("Name"))}
    if not dur:
        raise SystemExit(f"no library kernels in {folder}/trace")
    dom = max(dur, key=lambda n: sum(dur[n]))
    mult = {n: int(round(len(v) / len(dur[dom]))) for n, v in dur.items()}

    def counters(sub):
        """{kernel: {counter: [per-dispatch value]}} and the ordered copy-kernel dispatches."""
        per, names = {}, {}
        for r in _csv_rows(os.path.join(folder, sub), "counter_collection.csv"):
            d = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
            names[d] = r.get("Kernel_Name")
            per.setdefault(d, {}).setdefault(r["Counter_Name"], 0.0)
            per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        out, copies = {}, []
        for d in sorted(per):
            n = names[d]
            if "copyBuffer" in (n or ""):
                copies.append(per[d])
            for c, v in per[d].items():
                out.setdefault(n, {}).setdefault(c, []).append(v)
        return out, copies

    med = lambda v: statistics.median(v) if v else float("nan")
    lines = [f"# {title}", ""]
    cmd_path = os.path.join(folder, "commands.txt")
    if os.path.exists(cmd_path):
        lines += ["Commands (on one MI355X, from the repository root `$REPO`; `$OUT` = an output folder):", ""]
        lines += [f"* `{c.strip().replace('<file>.md', fname)}`" for c in open(cmd_path) if c.strip()]
        lines += [""]
    rec = _last_json(os.path.join(folder, "trace.log"))
    call = None  # the run's one record (per-call figures are given only when the run has exactly one)
    if rec is not None:
        if "metric" in rec:
            call = rec
        elif len(rec.get("forms", {})) == 1:
            call = next(iter(rec["forms"].values()))
    lines += ["## Kernel durations (kernel trace)", "",
              "| kernel | grid threads | wg | VGPRs | LDS B | dispatches | per call | avg µs (--stats) | median µs | min µs |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    order = sorted(dur, key=lambda n: -sum(dur[n]))
    for n in order:
        g, w, vg, lds = shape[n]
        lines.append(f"| `{_short_kernel(n)}` | {g} | {w} | {vg} | {lds} | {len(dur[n])} | {mult[n]} | "
                     f"{stats.get(n, float('nan')):.2f} | {med(dur[n]):.2f} | {min(dur[n]):.2f} |")
    per_call_us = sum(mult[n] * stats.get(n, sum(dur[n]) / len(dur[n])) for n in dur)
    if call is not None:
        lines += ["", f"Sum of the average kernel durations per call: {per_call_us:.1f} µs."]
    elif rec is not None:
        lines += ["", "The run times several calls (the bench's records below); the kernel rows cover them all:", ""]
        lines += [f"* `{n}`: {r.get('ms', float('nan')) * 1e3:.1f} µs per step (median "
                  f"{r.get('median_ms', float('nan')) * 1e3:.1f} µs)" for n, r in rec.get("forms", {}).items()]
    if call is not None:
        lines += [f"The bench's HIP-event timing of the same command: {call.get('ms_per_step', call.get('ms')) * 1e3:.1f} µs "
                  f"per call (mean over the timed steps; median {call.get('median_ms_per_step', call.get('median_ms')) * 1e3:.1f} µs)."]
    data = {"kernel_sources_sha256": sources_sha256(sources)}
    # traffic
    fetch, fcopies = counters("pmc_FETCH_SIZE")
    write, wcopies = counters("pmc_WRITE_SIZE")
    if fetch and write:
        def calib(sub, copies, counter):
            m = re.search(r"# copy calibration: (\d+) copies of (\d+) bytes", open(os.path.join(folder, sub + ".log")).read())
            k, nbytes = int(m.group(1)), int(m.group(2))
            kib = statistics.median(c[counter] for c in copies[:k])
            return nbytes / (kib * 1024.0), kib, nbytes
        ff, fkib, cb = calib("pmc_FETCH_SIZE", fcopies, "FETCH_SIZE")
        fw, wkib, _ = calib("pmc_WRITE_SIZE", wcopies, "WRITE_SIZE")
        lines += ["", "## HBM traffic (FETCH_SIZE and WRITE_SIZE, one counter per run)", "",
                  f"A plain device copy of {cb} bytes run first in the same processes reads back {fkib:.0f} KiB "
                  f"FETCH_SIZE and {wkib:.0f} KiB WRITE_SIZE per dispatch, so bytes read = FETCH_SIZE × 1024 × {ff:.3f} "
                  f"and bytes written = WRITE_SIZE × 1024 × {fw:.3f}.", "",
                  "| kernel | FETCH_SIZE KiB / dispatch (median) | WRITE_SIZE KiB / dispatch | read MB / dispatch | "
                  "written MB / dispatch |", "|---|---|---|---|---|"]
        traffic = 0.0  # per call: meaningful only for a run with one record
        for n in order:
            fk, wk = med(fetch.get(n, {}).get("FETCH_SIZE", [])), med(write.get(n, {}).get("WRITE_SIZE", []))
            rd, wr = fk * 1024 * ff, wk * 1024 * fw
            lines.append(f"| `{_short_kernel(n)}` | {fk:.1f} | {wk:.1f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
            traffic += mult[n] * (rd + wr)
        if call is not None:
            data["traffic_bytes_per_call"] = int(traffic)
        alg = None
        if call is not None:
            alg = call["roofline"]["algorithmic_bytes_per_call"] if "roofline" in call else call.get("algorithmic_bytes")
        if alg:
            data["algorithmic_bytes_per_call"] = int(alg)
            lines += ["", f"Algorithmic bytes per call: {int(alg):,}. Measured HBM traffic per call: {int(traffic):,} B "
                          f"({traffic / alg:.2f}× algorithmic)."]
    # instruction counters
    sq, _ = counters("pmc_SQ")
    if sq:
        lines += ["", "## Instruction counters (one run; medians per dispatch)", "",
                  "SQ counters are summed over the chip; GRBM_GUI_ACTIVE is summed over the 8 XCDs, so cycles = "
                  "GRBM_GUI_ACTIVE / 8 (the implied clock is cycles / kernel duration). VALU issue = (SQ_INSTS_VALU − "
                  "SQ_INSTS_MFMA) × 4 / (1024 SIMDs × cycles): a wave64 instruction occupies a 16-lane SIMD for 4 "
                  "cycles (transcendentals included, which issue at a lower rate); MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (1024 × cycles), rocprofv3's MfmaUtil.", "",
                  "| kernel | waves | VALU instr | of which transcendental | MFMA instr | bf16 MFMA flops | LDS instr | "
                  "cycles | implied GHz | VALU issue | MFMA busy |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        for n in order:
            c = {k: med(v) for k, v in sq.get(n, {}).items()}
            if not c:
                continue
            cyc = c.get("GRBM_GUI_ACTIVE", float("nan")) / 8
            ghz = cyc / (stats.get(n, med(dur[n])) * 1e3)
            valu, mfma = c.get("SQ_INSTS_VALU", 0.0), c.get("SQ_INSTS_MFMA", 0.0)
            lines.append(
                f"| `{_short_kernel(n)}` | {c.get('SQ_WAVES', 0):.0f} | {valu:.3e} | {c.get('SQ_INSTS_VALU_TRANS_F32', 0):.3e} | "
                f"{mfma:.3e} | {c.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0) * 512:.3e} | {c.get('SQ_INSTS_LDS', 0):.3e} | "
                f"{cyc:.3e} | {ghz:.2f} | {100 * (valu - mfma) * 4 / (1024 * cyc):.1f} % | "
                f"{100 * c.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (1024 * cyc):.1f} % |")
            data.setdefault("counters", {})[_short_kernel(n)] = {k: round(v, 1) for k, v in c.items()}
    lines += ["", f"Kernel sources these figures hold for: {', '.join('`' + f + '`' for f in sources)} "
                  f"(sha256 below; the bench reports the traffic only while it matches).", "",
              "<!-- profile-data: " + json.dumps({k: v for k, v in data.items() if k != "counters"}) + " -->"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-forms", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="run one workload: 'headline' or a form name " + ", ".join(FORMS))
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="write the markdown summary of the rocprofv3 runs of workload --only in DIR (no GPU use)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="first run a plain device-to-device tensor copy of this many MiB three times (a known-size "
                         "kernel for scaling hardware traffic counters)")
    args = ap.parse_args()
    if args.summarize is not None:
        sys.stdout.write(summarize_profile(args.summarize, args.only or "headline"))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X (the scans shard with no "
              "communication across channels, sequences and heads; see DESIGN.md); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.only is not None and args.only != "headline" and args.only not in FORMS:
        print(f"unknown workload {args.only!r}; choose 'headline' or one of: {', '.join(FORMS)}", file=sys.stderr)
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
        print(f"# copy calibration: 3 copies of {n * 4} bytes", file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()

    if args.only is not None and args.only != "headline":
        print(json.dumps({"only": args.only, "forms": run_form(args.only, args, device)}), flush=True)
        return

    copy_gbs = copy_rate_gbs(device)
    head = headline(args, device)
    t = head["t"]
    ms = t["ms"]
    value = head["updates"] / (ms * 1e-3)
    call_s = ms * 1e-3
    hbm_gbs = head["bytes"] / call_s / 1e9
    alu_tflops = head["updates"] * SELECTIVE_FLOPS_PER_UPDATE / call_s / 1e12
    print(f"# headline: {ms:.4f} ms/step (median {t['median_ms']:.4f}, min {t['min_ms']:.4f}, host clock "
          f"{t['host_ms']:.4f}), {value:.3e} upd/s, {hbm_gbs:.0f} GB/s; device copy {copy_gbs:.0f} GB/s",
          file=sys.stderr, flush=True)
    c = HEADLINE
    line = {
        "metric": "scan state-updates/s + achieved HBM GB/s (% of peak), fwd, 1 MI355X",
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "median_ms_per_step": t["median_ms"],
        "min_ms_per_step": t["min_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "packed variable-length multi-scale selective scan, L=131072 tokens in 32 sequences "
                               "(lengths log-uniform in [512, 16384], rescaled to sum to L; state reset at each "
                               "start), D=4096, N=16, 4 scales, bf16 in, fp32 state and out, softplus dt, skip D=1, "
                               "silu(z) gate",
                   "L": c["L"], "nseq": c["nseq"], "D": c["D"], "N": c["N"], "input_dtype": "bf16",
                   "output_dtype": "f32"},
        "hbm": {"achieved_gbs": hbm_gbs, "peak_gbs": HBM_PEAK_GBS, "frac": hbm_gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": head["bytes"], "device_copy_gbs": copy_gbs,
                "frac_of_device_copy": hbm_gbs / copy_gbs},
        "roofline": {"bound": "hbm", "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hbm_gbs / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("headline"),
                     "kernel": "one packed varlen selective scan call (its kernels, back to back)",
                     "algorithmic_bytes_per_call": head["bytes"], "ms_per_call": ms,
                     "median_ms_per_call": t["median_ms"], "min_ms_per_call": t["min_ms"],
                     "frac_of_device_copy": hbm_gbs / copy_gbs,
                     "alu": {"achieved_tflops": alu_tflops, "flops_per_update": SELECTIVE_FLOPS_PER_UPDATE,
                             "frac_of_published_fp32": alu_tflops / FP32_VECTOR_TFLOPS,
                             "frac_of_non_packed_fma": alu_tflops / FP32_SCALAR_FMA_TFLOPS,
                             "published_peak_tflops": FP32_VECTOR_TFLOPS,
                             "non_packed_peak_tflops": FP32_SCALAR_FMA_TFLOPS}},
    }
    if args.only == "headline":
        print(json.dumps(line), flush=True)
        return
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head)
        print(f"# cpu_baseline: {line['cpu_baseline']['value']:.3e} upd/s on {line['cpu_baseline']['cores']} "
              f"threads ({line['cpu_baseline']['single_thread_value']:.3e} on one)", file=sys.stderr, flush=True)
    del head
    torch.cuda.empty_cache()
    if not args.no_forms:
        forms = {}
        for name in FORMS:
            forms.update(run_form(name, args, device))
        line["forms"] = forms
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
