"""Shared helpers of the GPU parity tests: moving synthetic inputs to the device and the error
measure  max|gpu - oracle| / RMS(oracle)."""
import numpy as np

from selective_state_space_diag_amd import synth

# Tolerances on max |err| / RMS(reference): fp32 inputs and bf16 inputs with fp32 state.
TOL = {synth.F32: 1e-5, synth.BF16: 2e-2}


def to_dev(t, device="cuda"):
    """synth.Tensor or float32 numpy array -> torch tensor on the GPU with the same bits."""
    import torch
    if isinstance(t, synth.Tensor):
        if t.dtype == synth.BF16:
            return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    if t is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def f64(t):
    if t is None:
        return None
    if isinstance(t, synth.Tensor):
        return t.f64()
    return np.asarray(t, dtype=np.float64)


def rel_err(gpu, ref):
    """max |gpu - ref| / RMS(ref) (0 when both are empty)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(g - r))) / max(rms, 1e-30)


def assert_close(gpu, ref, tol, what=""):
    e = rel_err(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), f"{what}: non-finite GPU output"
    assert e <= tol, f"{what}: max|err|/RMS = {e:.3e} > {tol:.1e}"
    return e


def elem_err(gpu, ref):
    """max_i |gpu_i - ref_i| / max(|ref_i|, RMS(ref)): each element against its own magnitude, with the
    RMS as the floor for the small ones."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    den = np.maximum(np.abs(r), max(float(np.sqrt(np.mean(r * r))), 1e-30))
    return float(np.max(np.abs(g - r) / den))


def assert_close_elem(gpu, ref, tol, what=""):
    e = elem_err(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), f"{what}: non-finite GPU output"
    assert e <= tol, f"{what}: max|err|/max(|ref|, RMS) = {e:.3e} > {tol:.1e}"
    return e


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def parallel_map(fn, items):
    """fn over items on a small thread pool (the oracle's C loops release the GIL), results in order."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        return list(ex.map(fn, items))


def spread_heads(B, H):
    """(b, h) pairs of the full-size HGRN2 checks: every head of four batch rows of both parities, so
    every head index, every (b, h) parity and every position of a head's workgroups modulo the 8 XCDs
    is covered (64 heads at B = 8, H = 16)."""
    rows = sorted({0, min(3, B - 1), min(5, B - 1), B - 1})
    return [(b, h) for b in rows for h in range(H)]


def spread_channels(D, n_random, seed, block=256, scale_blocks=4):
    """Channels of the full-size selective checks: the first and last channel of every 256-channel
    workgroup (which include the edges of every scale block) plus seeded random ones."""
    import numpy as np
    edges = set()
    for c0 in range(0, D, block):
        edges.update((c0, min(c0 + block, D) - 1))
    for s in range(scale_blocks):
        edges.update((s * D // scale_blocks, (s + 1) * D // scale_blocks - 1))
    rng = np.random.default_rng(seed)
    rest = [c for c in rng.permutation(D) if c not in edges][:n_random]
    return np.array(sorted(edges | set(int(c) for c in rest)))
