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


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)
