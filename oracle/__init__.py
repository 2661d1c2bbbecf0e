"""fp64 CPU oracle for the chunked linear recurrence.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import, call, link or execute anything in this package.  The
product path (the HIP library and its Python binding) never touches it, and the two
share no code: no kernels, headers, helpers, tables or pre/post-processing.  Inputs
reach both sides from the seeded generators, which hold none of the method's
arithmetic.

Method source: the page "分块推理：解锁循环模型并行计算，实现长序列高效处理"
(chunked inference for recurrent models), cited as [分块推理 §n]:
  seq()      the recurrence of [分块推理 §2], token by token (the plain definition);
  chunked()  the decomposition of [分块推理 §2.1-§2.2] with its intermediates;
  stack_horizontal(), stack_vertical()
             the two cross-layer schedules of [分块推理 §3.1] and [分块推理 §3.2];
  brute      a numpy closed form of the unrolled recurrence, for tiny lengths.

Pins: every function here is checked in tests/test_oracle.py against facts fixed by the
pages and by mathematics (brute force, closed forms, scipy's IIR filter, invariants and
hand-worked fixtures under tests/golden/).
"""
import ctypes
import os

import numpy as np

from . import brute  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "libssdoracle.so")
_lib = None

_DP = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_seq.argtypes = [_I64] * 6 + [_DP] * 9 + [ctypes.c_int]
        lib.oracle_seq.restype = ctypes.c_int
        lib.oracle_chunked.argtypes = [_I64] * 7 + [_DP] * 14 + [ctypes.c_int]
        lib.oracle_chunked.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [_DP, _DP, _I64]
        lib.oracle_round_bf16.restype = None
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def to_f64(t) -> np.ndarray:
    """Decode a tensor or array exactly into a C-contiguous float64 array.

    bfloat16 values are the upper 16 bits of an IEEE binary32 value, so the decode
    shifts the raw bits left by 16 and reinterprets them; float32 widens exactly.
    """
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                bits = t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16
                return np.ascontiguousarray(bits.view(np.float32).astype(np.float64))
            return np.ascontiguousarray(t.numpy().astype(np.float64))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_DP)


def _dims(x, B):
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return batch, L, H, P, N, G


def seq(x, dt, A, B, C, D=None, init=None, nthreads=None):
    """Token-by-token recurrence [分块推理 §2] over all (batch, head) pairs.

    x [b,L,H,P], dt [b,L,H], A [H], B/C [b,L,G,N], D [H] or None, init [b,H,P,N] or None.
    Returns (y [b,L,H,P], final_state [b,H,P,N]) in float64.
    """
    x, dt, A, B, C = (to_f64(v) for v in (x, dt, A, B, C))
    D = None if D is None else to_f64(D)
    init = None if init is None else to_f64(init)
    batch, L, H, P, N, G = _dims(x, B)
    y = np.zeros((batch, L, H, P))
    fin = np.zeros((batch, H, P, N))
    rc = _load().oracle_seq(batch, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                            _ptr(D), _ptr(init), _ptr(y), _ptr(fin),
                            nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_seq failed with code %d" % rc)
    return y, fin


def chunked(x, dt, A, B, C, D, init, Q, nthreads=None):
    """Chunked decomposition [分块推理 §2.1-§2.2] with every intermediate.

    Returns a dict with y, final_state, logcum [b,H,nc,Q] (NaN past a short last chunk),
    b_intra and b_in [b,nc,H,P,N], by_intra and by_inter [b,L,H,P].
    """
    x, dt, A, B, C = (to_f64(v) for v in (x, dt, A, B, C))
    D = None if D is None else to_f64(D)
    init = None if init is None else to_f64(init)
    batch, L, H, P, N, G = _dims(x, B)
    nc = (L + Q - 1) // Q
    out = dict(
        y=np.zeros((batch, L, H, P)), final_state=np.zeros((batch, H, P, N)),
        logcum=np.full((batch, H, nc, Q), np.nan), b_intra=np.zeros((batch, nc, H, P, N)),
        b_in=np.zeros((batch, nc, H, P, N)), by_intra=np.zeros((batch, L, H, P)),
        by_inter=np.zeros((batch, L, H, P)))
    rc = _load().oracle_chunked(batch, L, H, P, N, G, Q, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                _ptr(C), _ptr(D), _ptr(init), _ptr(out["y"]),
                                _ptr(out["final_state"]), _ptr(out["logcum"]),
                                _ptr(out["b_intra"]), _ptr(out["b_in"]), _ptr(out["by_intra"]),
                                _ptr(out["by_inter"]), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_chunked failed with code %d" % rc)
    return out


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (as float64)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty_like(v)
    _load().oracle_round_bf16(_ptr(v), _ptr(out), v.size)
    return out


def stack_horizontal(x0, dt, A_layers, B, C, D_layers, layer_init=None, residual=True,
                     store_bf16=True, nthreads=None):
    """Layer-serial stack [分块推理 §3.1]: every token of layer l, then layer l+1.

    Layer l maps activations u to out = y_l(u) (+ u when residual), where y_l is the
    recurrence with A_layers[l], D_layers[l] and initial state layer_init[l].  When the
    library stores activations in bfloat16, out is rounded once to bfloat16 at each layer
    boundary (store_bf16), as the stored tensor is.  dt, B and C are shared by all layers.
    Returns (stack output [b,L,H,P], final states [layers,b,H,P,N]).
    """
    u = to_f64(x0)
    A_layers, D_layers = to_f64(A_layers), to_f64(D_layers)
    finals = []
    for l in range(A_layers.shape[0]):
        init = None if layer_init is None else to_f64(layer_init)[l]
        y, fin = seq(u, dt, A_layers[l], B, C, D_layers[l], init, nthreads)
        out = y + u if residual else y
        u = round_bf16(out) if store_bf16 else out
        finals.append(fin)
    return u, np.stack(finals)


def stack_vertical(x0, dt, A_layers, B, C, D_layers, V, layer_init=None, residual=True,
                   store_bf16=True, nthreads=None):
    """Segment-serial stack [分块推理 §3.2]: V tokens through every layer, each layer's
    state saved per layer and reused by the next segment.  Must equal stack_horizontal.
    """
    x0, dt, B, C = (to_f64(v) for v in (x0, dt, B, C))
    A_layers, D_layers = to_f64(A_layers), to_f64(D_layers)
    nl = A_layers.shape[0]
    batch, L, H, P = x0.shape
    N = B.shape[3]
    states = (np.zeros((nl, batch, H, P, N)) if layer_init is None
              else to_f64(layer_init).copy())
    out = np.zeros_like(x0)
    for s0 in range(0, L, V):
        s1 = min(s0 + V, L)
        u = np.ascontiguousarray(x0[:, s0:s1])
        for l in range(nl):
            seg = (np.ascontiguousarray(dt[:, s0:s1]), np.ascontiguousarray(B[:, s0:s1]),
                   np.ascontiguousarray(C[:, s0:s1]))
            y, fin = seq(u, seg[0], A_layers[l], seg[1], seg[2], D_layers[l],
                         np.ascontiguousarray(states[l]), nthreads)
            states[l] = fin
            o = y + u if residual else y
            u = round_bf16(o) if store_bf16 else o
        out[:, s0:s1] = u
    return out, states
