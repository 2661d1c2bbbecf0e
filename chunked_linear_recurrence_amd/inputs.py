"""Seeded synthetic inputs, shared by the library's tests, its benchmark and the oracle.

This module only draws random numbers and casts them to the storage dtype; it holds
none of the recurrence's arithmetic.  All draws use numpy's PCG64 generator
(``np.random.default_rng(seed)``) in float32, in a fixed order:

  single layer:  x, dt_raw, A_raw, B, C, D, init_state (init_state only when random)
  layer stack:   x0, dt_raw, B, C, then for each layer l: A_raw[l], D[l]

Distributions:
  x ~ N(0, 1);  dt = clamp(softplus(N(-2, 0.5)), dt_min, dt_max);
  A_h = -exp(U(0, ln 16))  (so A in [-16, -1]);  B, C ~ N(0, 1) / sqrt(N);
  D ~ U(0, 1);  init_state ~ N(0, init_std^2) when requested, else zeros.
Activations (x, dt, B, C) are stored as float32 or bfloat16; the float32 -> bfloat16 cast
is torch's round-to-nearest-even.  A, D and states are always float32.
"""
import math

import numpy as np
import torch

from .workloads import Workload


def _softplus(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z) in float32, written to avoid overflow for large z
    return (np.maximum(z, 0) + np.log1p(np.exp(-np.abs(z)))).astype(np.float32)


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def draw_dt(rng, shape, dt_min, dt_max, dist="softplus"):
    if dist == "softplus":
        z = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.5) - np.float32(2.0)
        return np.clip(_softplus(z), dt_min, dt_max).astype(np.float32)
    if dist == "loguniform":
        u = rng.random(shape, dtype=np.float32)
        lo, hi = math.log(dt_min), math.log(dt_max)
        return np.exp(np.float32(lo) + u * np.float32(hi - lo)).astype(np.float32)
    raise ValueError("unknown dt distribution %r" % dist)


def make_layer(batch, seqlen, nheads, headdim, dstate, ngroups, dtype="bf16", seed=0,
               dt_min=1e-3, dt_max=0.1, init="zero", init_std=0.1, dt_dist="softplus"):
    """Inputs of one layer as CPU tensors: x, dt, A, B, C, D, init_state (None if zero)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32)
    dt = draw_dt(rng, (batch, seqlen, nheads), dt_min, dt_max, dt_dist)
    A = -np.exp(rng.random(nheads, dtype=np.float32) * np.float32(math.log(16.0)))
    scale = np.float32(1.0 / math.sqrt(dstate))
    B = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32) * scale
    C = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32) * scale
    D = rng.random(nheads, dtype=np.float32)
    init_state = None
    if init == "normal":
        init_state = torch.from_numpy(
            rng.standard_normal((batch, nheads, headdim, dstate), dtype=np.float32)
            * np.float32(init_std))
    return dict(x=_store(x, dtype), dt=_store(dt, dtype),
                A=torch.from_numpy(A.astype(np.float32)), B=_store(B, dtype),
                C=_store(C, dtype), D=torch.from_numpy(D), init_state=init_state)


def make_stack(batch, seqlen, nheads, headdim, dstate, ngroups, layers, dtype="bf16", seed=0,
               dt_min=1e-3, dt_max=0.1):
    """Inputs of a layer stack: x0, dt, B, C shared by every layer; A, D per layer [layers, H]."""
    rng = np.random.default_rng(seed)
    x0 = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32)
    dt = draw_dt(rng, (batch, seqlen, nheads), dt_min, dt_max)
    scale = np.float32(1.0 / math.sqrt(dstate))
    B = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32) * scale
    C = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=np.float32) * scale
    A = np.empty((layers, nheads), dtype=np.float32)
    D = np.empty((layers, nheads), dtype=np.float32)
    for l in range(layers):
        A[l] = -np.exp(rng.random(nheads, dtype=np.float32) * np.float32(math.log(16.0)))
        D[l] = rng.random(nheads, dtype=np.float32)
    return dict(x0=_store(x0, dtype), dt=_store(dt, dtype), B=_store(B, dtype),
                C=_store(C, dtype), A=torch.from_numpy(A), D=torch.from_numpy(D))


def make(w: Workload, seed=None):
    """Inputs of a named workload (seed defaults to the workload's own)."""
    s = w.seed if seed is None else seed
    if w.layers > 1:
        return make_stack(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                          w.layers, w.dtype, s, w.dt_min, w.dt_max)
    return make_layer(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype, s,
                      w.dt_min, w.dt_max, w.init, w.init_std)
