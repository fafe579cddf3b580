"""Seeded synthetic inputs for the chunked gated delta rule.

This module is shared by the CPU oracle and by the GPU path's tests and benchmark.
It holds none of the method's arithmetic: it only draws random numbers, shapes them
into the distributions of the five workloads, and rounds them once to the storage
precision.  Nothing here computes a state, a gate product, a triangular inverse or
an output.

Workloads (the distributions follow the Gated DeltaNet layers the pages discuss:
Preconditioned DeltaNet, technical summary section 2; Gated DeltaNet-2 news item,
"Como DeltaNet-2 Redesenhou"; MatMul-only inversion summary, "Problema"):

* ``plain``  - plain delta rule, B1 H1 T256 d64, fp32, C64.
* ``gdn``    - scalar-gated delta rule, B4 H16 T4096 d128, bf16 inputs, C64.
* ``gdn2``   - channel-wise erase/write gates, B2 H16 T8192 d128, bf16, C64.
* ``pdn``    - diagonal-preconditioned write key, B4 H16 T4096 d128, bf16, C64.
* ``long``   - scalar-gated, B1 H32 T32768 d128, bf16, C64, then decode steps at
               batch 64 (step ``s`` drawn from seed ``5001 + s``).
* ``kda``    - one decay per key channel (the diagonal gate of Kimi Delta Attention),
               otherwise as ``gdn``: B4 H16 T4096 d128, bf16, C64.

Recipe (one generator per call, ``numpy.random.Generator(PCG64(seed))``, draws in
the order q, k, v, then the gate logits):

* q, k ~ N(0, 1), L2-normalised per token in fp64 (no epsilon);
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1))                      [B, T, H]     (scalar gain);
* log_alpha = -0.1 * softplus(N(0, 1))         [B, T, H]     (scalar decay);
* log_alpha = -0.1 * softplus(N(0, 1))         [B, T, H, Dk] (per-channel decay);
* erase = sigmoid(N(2, 1))                     [B, T, H, Dk] (channel gain, key axis);
* write = sigmoid(N(0, 1))                     [B, T, H, Dv] (channel gain, value axis).

Stress options (off by default; a default spec draws exactly the stream above):

* ``key_corr = c > 0``: queries, keys (and an explicit write key) share one direction per
  (batch, head) stream, q = normalise(z_q + c * u), k = normalise(z_k + c * u), u ~ N(0, I)
  drawn from its own generator (seed ``seed + 104729``), so every decode step of a stream
  sees the same u.  Real keys are correlated; this is the regime where the chunk's
  triangular inverse is ill-conditioned;
* ``beta_shift = s``: beta = s + sigmoid(N(0, 1)) (s = 1 gives beta in (1, 2), the range where
  the transition I - beta k k^T has a negative eigenvalue);
* ``decay_law = "strong"``: log_alpha = -5 U(0, 1) per token (per channel for a per-channel
  decay) in place of -0.1 softplus(N(0, 1)).

Loss gradients for the backward pass (``make_cotangents``, seed ``spec.seed + 7919`` unless
given): d_out ~ N(0, 1) [B, T, H, Dv] stored like v, and d_state_out ~ N(0, 1) [B, H, Dv, Dk]
fp32, drawn in that order.

Every value is produced in fp64, cast to fp32, then (for bf16 workloads, and only
for q, k, v, erase, write) rounded to bf16 with round-to-nearest-even, once.  Both
the oracle and the GPU path consume exactly those bits.  beta and log_alpha stay
fp32 on both sides.  Arrays are numpy float32 in ``[B, T, H, D]`` / ``[B, T, H]``
layout; bf16 values are held exactly in float32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Spec", "WORKLOADS", "spec", "make_inputs", "make_decode_inputs", "make_cotangents",
    "round_to_bf16", "round_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape, precision and variant of one synthetic workload."""
    name: str
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    chunk: int = 64
    dtype: str = "bf16"          # storage dtype of q, k, v, o (and erase/write gates)
    gain: str = "scalar"         # "scalar" (beta) | "channel" (erase, write)
    decay: str = "none"          # "none" | "scalar" (log_alpha [B,T,H]) | "channel" ([B,T,H,Dk])
    wkey: str = "same"           # "same" | "precond" | "explicit"
    seed: int = 0
    # diagonal preconditioner constants (used when wkey == "precond")
    pc_rho: float = 0.99
    pc_eps: float = 1e-3
    pc_h0: float = 1.0
    # decode phase (``long`` workload only)
    decode_batch: int = 0
    decode_steps: int = 0
    # stress options (see the module docstring); the defaults leave the draws unchanged
    key_corr: float = 0.0
    beta_shift: float = 0.0
    decay_law: str = "mild"      # "mild" | "strong"

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Spec] = {
    "plain": Spec("plain", B=1, H=1, T=256, Dk=64, Dv=64, dtype="f32",
                  gain="scalar", decay="none", seed=1000),
    "gdn": Spec("gdn", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16",
                gain="scalar", decay="scalar", seed=2000),
    "gdn2": Spec("gdn2", B=2, H=16, T=8192, Dk=128, Dv=128, dtype="bf16",
                 gain="channel", decay="none", seed=3000),
    "pdn": Spec("pdn", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16",
                gain="scalar", decay="none", wkey="precond", seed=4000),
    "long": Spec("long", B=1, H=32, T=32768, Dk=128, Dv=128, dtype="bf16",
                 gain="scalar", decay="scalar", seed=5000,
                 decode_batch=64, decode_steps=1024),
    "kda": Spec("kda", B=4, H=16, T=4096, Dk=128, Dv=128, dtype="bf16",
                gain="scalar", decay="channel", seed=6000),
}


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally with fields overridden (smaller test shapes)."""
    s = WORKLOADS[name]
    return s.replace(**overrides) if overrides else s


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even); returned as float32 holding bf16 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return bits.astype(np.uint32).view(np.float32).reshape(f.shape)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = round_to_f32(x64)
    return round_to_bf16(x32) if dtype == "bf16" else x32


def _l2n(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _shared_direction(s: Spec, seed: int, lead: tuple) -> np.ndarray:
    """One direction per (batch, head) stream, broadcast over tokens: shape of ``lead`` with the
    token axis (if any) set to 1, plus the key axis."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    if len(lead) == 3:   # (B, T, H)
        return rng.standard_normal((lead[0], 1, lead[2], s.Dk))
    return rng.standard_normal(lead + (s.Dk,))   # (B, H): decode


def _draw(rng: np.random.Generator, s: Spec, lead: tuple, base_seed: int) -> Dict[str, np.ndarray]:
    """Draw one batch of inputs with leading dims ``lead`` (e.g. (B, T, H))."""
    out: Dict[str, np.ndarray] = {}
    zq = rng.standard_normal(lead + (s.Dk,))
    zk = rng.standard_normal(lead + (s.Dk,))
    out["v"] = _store(rng.standard_normal(lead + (s.Dv,)), s.dtype)
    if s.gain == "scalar":
        out["beta"] = round_to_f32(s.beta_shift + _sigmoid(rng.standard_normal(lead)))
    else:
        out["erase"] = _store(_sigmoid(rng.normal(2.0, 1.0, lead + (s.Dk,))), s.dtype)
        out["write"] = _store(_sigmoid(rng.standard_normal(lead + (s.Dv,))), s.dtype)
    if s.decay != "none":
        shape = lead if s.decay == "scalar" else lead + (s.Dk,)
        if s.decay_law == "strong":
            out["log_alpha"] = round_to_f32(-5.0 * rng.random(shape))
        else:
            out["log_alpha"] = round_to_f32(-0.1 * _softplus(rng.standard_normal(shape)))
    zw = rng.standard_normal(lead + (s.Dk,)) if s.wkey == "explicit" else None
    if s.key_corr > 0.0:
        u = s.key_corr * _shared_direction(s, base_seed, lead)
        zq, zk = zq + u, zk + u
        zw = None if zw is None else zw + u
    out["q"] = _store(_l2n(zq), s.dtype)
    out["k"] = _store(_l2n(zk), s.dtype)
    if zw is not None:
        out["write_key"] = _store(zw / np.sqrt(s.Dk), s.dtype)
    return {k: out[k] for k in ("q", "k", "v", "beta", "erase", "write", "log_alpha", "write_key") if k in out}


def make_inputs(s: Spec, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of one chunked-forward call: arrays in [B, T, H, D] / [B, T, H] layout."""
    base = s.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(base))
    return _draw(rng, s, (s.B, s.T, s.H), base)


def make_decode_inputs(s: Spec, step: int) -> Dict[str, np.ndarray]:
    """Inputs of decode step ``step`` at batch ``decode_batch``: [Bd, H, D] / [Bd, H].

    Step ``s`` uses seed ``s.seed + 1 + step`` (5001 + step for the long workload).
    """
    rng = np.random.Generator(np.random.PCG64(s.seed + 1 + step))
    return _draw(rng, s, (s.decode_batch, s.H), s.seed)


def make_cotangents(s: Spec, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Loss gradients of one forward call's outputs: d_out [B, T, H, Dv] (stored like v) and
    d_state_out [B, H, Dv, Dk] fp32."""
    rng = np.random.Generator(np.random.PCG64(s.seed + 7919 if seed is None else seed))
    d_out = _store(rng.standard_normal((s.B, s.T, s.H, s.Dv)), s.dtype)
    d_state_out = round_to_f32(rng.standard_normal((s.B, s.H, s.Dv, s.Dk)))
    return {"d_out": d_out, "d_state_out": d_state_out}
