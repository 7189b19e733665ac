"""Seeded synthetic inputs shaped like the source pages' workloads.

This module draws random inputs only; it contains none of the scans'
arithmetic.  The same bits feed both the GPU library and the CPU oracle:
bf16 inputs are produced here as raw bit patterns (``uint16``), and
:func:`bf16_to_f64` gives their exact float64 values for the oracle.

Every generator takes an explicit ``seed`` and uses numpy's PCG64.  Normal
draws are made in float32 and rounded to bf16 with round-to-nearest-even.
``N(mu, s)`` below always means mean ``mu`` and standard deviation ``s``.

Workloads (sizes as named by the five benchmark configurations):

* ``rglru``: x, r_logit, i_logit ~ N(0,1); ``a_log[d] = ln U(0.9, 0.999)``
  (the RG-LRU base ``a`` initialised in [0.9, 0.999]); c = 8.
* ``selective``: A[d][n] = -(n+1) * 2**s for scale s = floor(d * S / D) (the
  multi-scale A of the cortexnet MultiScaleSSM, scales in contiguous channel
  blocks); per-channel step delta0 = exp(U[ln 1e-3, ln 1e-1]) times
  exp(N(0, 0.1)) per token; passed either raw (``dt_softplus=False``) or as
  ``dt = softplus^-1(delta)`` (``dt_softplus=True``); x, z ~ N(0,1);
  B, C ~ N(0, 1/N); skip D = 1.
* ``hgrn2``: q, k, v ~ N(0, 1/sqrt(d)); g_logit ~ N(2, 1); lower bound 0.5.
* ``varlen``: sequence lengths log-uniform in [512, 16384], rescaled to sum to
  the packed length (largest-remainder rounding).
* ``rglru`` with a gate: the block's gate pre-activation ~ N(0,1).
* ``minmax``: r, s ~ N(0,1) (the neuron's two linear maps of the input), gate
  ~ N(0,1), x0 ~ N(0,1); or, with ``ties=True``, values drawn from
  {-2, -1, -0, +0, 1, 2} so that equal values and both zeros occur.
* ``conv``: x ~ N(0,1); weight and bias ~ U(-1/sqrt(W), 1/sqrt(W)) (torch's
  default Conv1d initialisation for a depthwise kernel of width W); carried
  window ~ N(0,1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


# ----------------------------------------------------------------------------- bit-level conversions
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of each bf16 bit pattern."""
    return bf16_to_f32(bits).astype(np.float64)


@dataclass
class Tensor:
    """One synthetic input: its storage (``bits`` for bf16, ``f32`` for float32)."""
    dtype: str
    data: np.ndarray  # uint16 bit patterns (bf16) or float32

    @property
    def shape(self):
        return self.data.shape

    def f64(self) -> np.ndarray:
        return bf16_to_f64(self.data) if self.dtype == BF16 else self.data.astype(np.float64)

    def slice(self, index) -> "Tensor":
        return Tensor(self.dtype, np.ascontiguousarray(self.data[index]))


def _store(a32: np.ndarray, dtype: str) -> Tensor:
    if dtype == BF16:
        return Tensor(BF16, f32_to_bf16_bits(a32))
    if dtype == F32:
        return Tensor(F32, np.ascontiguousarray(a32, dtype=np.float32))
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, mean=0.0, std=1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


@dataclass
class Inputs:
    """A named bundle of inputs plus scalar parameters."""
    kind: str
    dims: Dict[str, int]
    t: Dict[str, Tensor] = field(default_factory=dict)        # bf16 / f32 activations
    p: Dict[str, np.ndarray] = field(default_factory=dict)    # float32 parameters (A, a_log, Dskip, ...)
    s: Dict[str, object] = field(default_factory=dict)        # scalars / flags / cu_seqlens


# ----------------------------------------------------------------------------- RG-LRU
def rglru_inputs(B: int, L: int, D: int, dtype: str = BF16, seed: int = 0, c: float = 8.0,
                 with_h0: bool = False, with_gate: bool = False) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.uniform(0.9, 0.999, size=D)
    inp = Inputs("rglru", dict(B=B, L=L, D=D))
    inp.p["a_log"] = np.log(a).astype(np.float32)
    for name in ("x", "r_logit", "i_logit"):
        inp.t[name] = _store(_normal(rng, (B, L, D)), dtype)
    inp.s["c"] = float(c)
    if with_h0:
        inp.p["h0"] = _normal(rng, (B, D))
    if with_gate:
        inp.t["gate"] = _store(_normal(rng, (B, L, D)), dtype)
    return inp


# ----------------------------------------------------------------------------- MinMax
_TIE_VALUES = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)


def minmax_inputs(B: int, L: int, D: int, dtype: str = BF16, seed: int = 0, with_x0: bool = False,
                  with_gate: bool = False, ties: bool = False) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    inp = Inputs("minmax", dict(B=B, L=L, D=D))
    draw = (lambda shape: _TIE_VALUES[rng.integers(0, _TIE_VALUES.size, size=shape)]) if ties else \
        (lambda shape: _normal(rng, shape))
    for name in ("r", "s"):
        inp.t[name] = _store(draw((B, L, D)), dtype)
    if with_x0:
        inp.p["x0"] = draw((B, D)).astype(np.float32)
    if with_gate:
        inp.t["gate"] = _store(_normal(rng, (B, L, D)), dtype)
    return inp


# ----------------------------------------------------------------------------- causal conv
def conv_inputs(B: int, L: int, D: int, W: int = 4, dtype: str = BF16, seed: int = 0, with_bias: bool = True,
                with_state: bool = False) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    inp = Inputs("conv", dict(B=B, L=L, D=D, W=W))
    bound = 1.0 / math.sqrt(W)
    inp.p["weight"] = rng.uniform(-bound, bound, size=(D, W)).astype(np.float32)
    if with_bias:
        inp.p["bias"] = rng.uniform(-bound, bound, size=D).astype(np.float32)
    inp.t["x"] = _store(_normal(rng, (B, L, D)), dtype)
    if with_state:
        inp.p["state"] = _normal(rng, (B, D, W))
    return inp


def rglru_decode_inputs(B: int, D: int, steps: int, dtype: str = BF16, seed: int = 0, c: float = 8.0) -> Inputs:
    """Per-step fresh x, r_logit, i_logit of shape [steps, B, D] for the decode benchmark."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.uniform(0.9, 0.999, size=D)
    inp = Inputs("rglru_decode", dict(B=B, D=D, steps=steps))
    inp.p["a_log"] = np.log(a).astype(np.float32)
    for name in ("x", "r_logit", "i_logit"):
        inp.t[name] = _store(_normal(rng, (steps, B, D)), dtype)
    inp.s["c"] = float(c)
    return inp


# ----------------------------------------------------------------------------- selective
def multiscale_A(D: int, N: int, num_scales: int = 4) -> np.ndarray:
    """A[d][n] = -(n+1) * 2**s, scale s = floor(d * num_scales / D) (equal contiguous channel blocks
    when num_scales divides D)."""
    s = ((np.arange(D) * num_scales) // max(D, 1)).astype(np.float64)
    n = np.arange(1, N + 1, dtype=np.float64)
    return (-(n[None, :] * (2.0 ** s)[:, None])).astype(np.float32)


def _softplus_inverse(delta: np.ndarray) -> np.ndarray:
    # input preparation only: the dt that a softplus maps onto the drawn step size
    d = delta.astype(np.float64)
    return d + np.log(-np.expm1(-d))


def selective_inputs(B: int, L: int, D: int, N: int = 16, dtype: str = BF16, seed: int = 0,
                     num_scales: int = 4, dt_softplus: bool = True, with_z: bool = True,
                     with_skip: bool = True, cu_seqlens: Optional[np.ndarray] = None,
                     with_h0: bool = False) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    inp = Inputs("selective", dict(B=B, L=L, D=D, N=N))
    inp.p["A"] = multiscale_A(D, N, num_scales)
    log_lo, log_hi = math.log(1e-3), math.log(1e-1)
    delta0 = np.exp(rng.uniform(log_lo, log_hi, size=D)).astype(np.float32)
    eps = _normal(rng, (B, L, D), 0.0, 0.1)
    delta = np.exp(eps) * delta0[None, None, :]
    dt = _softplus_inverse(delta).astype(np.float32) if dt_softplus else delta
    del eps, delta
    inp.t["dt"] = _store(dt, dtype)
    del dt
    inp.t["x"] = _store(_normal(rng, (B, L, D)), dtype)
    inp.t["Bm"] = _store(_normal(rng, (B, L, N), 0.0, 1.0 / N), dtype)
    inp.t["Cm"] = _store(_normal(rng, (B, L, N), 0.0, 1.0 / N), dtype)
    if with_z:
        inp.t["z"] = _store(_normal(rng, (B, L, D)), dtype)
    if with_skip:
        inp.p["Dskip"] = np.ones(D, dtype=np.float32)
    inp.s["dt_softplus"] = bool(dt_softplus)
    if cu_seqlens is not None:
        inp.s["cu_seqlens"] = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if with_h0:
        nseq = (len(cu_seqlens) - 1) if cu_seqlens is not None else B
        inp.p["h0"] = _normal(rng, (nseq, D, N))
    return inp


def varlen_lengths(total: int, nseq: int, seed: int, lo: float = 512.0, hi: float = 16384.0) -> np.ndarray:
    """Lengths log-uniform in [lo, hi], scaled to sum to ``total`` (largest remainder, ties by index)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = np.exp(rng.uniform(math.log(lo), math.log(hi), size=nseq))
    scaled = raw * (total / raw.sum())
    base = np.floor(scaled).astype(np.int64)
    rem = total - int(base.sum())
    frac = scaled - base
    order = sorted(range(nseq), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    return base


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


# ----------------------------------------------------------------------------- HGRN2
def hgrn2_inputs(B: int, L: int, H: int, d: int, dtype: str = BF16, seed: int = 0, lower_bound: float = 0.5,
                 with_S0: bool = False) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    inp = Inputs("hgrn2", dict(B=B, L=L, H=H, d=d))
    std = 1.0 / math.sqrt(d)
    for name in ("q", "k", "v"):
        inp.t[name] = _store(_normal(rng, (B, L, H, d), 0.0, std), dtype)
    inp.t["g_logit"] = _store(_normal(rng, (B, L, H, d), 2.0, 1.0), dtype)
    inp.s["lower_bound"] = float(lower_bound)
    if with_S0:
        inp.p["S0"] = _normal(rng, (B, H, d, d), 0.0, 0.1)
    return inp


# ----------------------------------------------------------------------------- the five workloads
# Named workloads with the shapes and distributions described above; each has a fixed seed.
WORKLOADS = {
    "rglru_small": dict(kind="rglru", B=2, L=128, D=64, dtype=F32, c=8.0, seed=1000),
    "selective": dict(kind="selective", B=4, L=2048, D=1536, N=16, dtype=BF16, scales=4, seed=1001),
    "rglru": dict(kind="rglru", B=8, L=8192, D=2560, dtype=BF16, c=8.0, decode_B=256, decode_steps=256, seed=1002),
    "hgrn2": dict(kind="hgrn2", B=8, L=4096, H=16, d=128, dtype=BF16, lower_bound=0.5, chunk=64, seed=1003),
    "selective_varlen": dict(kind="varlen", L=131072, nseq=32, D=4096, N=16, dtype=BF16, scales=4, seed=1004),
}


def workload_inputs(name: str, seed: Optional[int] = None, **overrides) -> Inputs:
    """Inputs of the named workload (seed defaults to the workload's own)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    seed = cfg["seed"] if seed is None else seed
    k = cfg["kind"]
    if k == "rglru":
        return rglru_inputs(cfg["B"], cfg["L"], cfg["D"], cfg["dtype"], seed, cfg["c"])
    if k == "selective":
        return selective_inputs(cfg["B"], cfg["L"], cfg["D"], cfg["N"], cfg["dtype"], seed, cfg["scales"],
                                dt_softplus=cfg.get("dt_softplus", True))
    if k == "hgrn2":
        return hgrn2_inputs(cfg["B"], cfg["L"], cfg["H"], cfg["d"], cfg["dtype"], seed, cfg["lower_bound"])
    if k == "varlen":
        lengths = varlen_lengths(cfg["L"], cfg["nseq"], seed)
        cu = cu_seqlens_from_lengths(lengths)
        return selective_inputs(1, cfg["L"], cfg["D"], cfg["N"], cfg["dtype"], seed + 1, cfg["scales"],
                                dt_softplus=cfg.get("dt_softplus", True), cu_seqlens=cu)
    raise ValueError(k)
