"""GPU parity of the decode step (ssd_step): one token of the recurrence of [分块推理 §2]
of the page "分块推理：解锁循环模型并行计算，实现长序列高效处理", continuing from a carried
state.  The fp64 oracle runs the whole sequence token by token; the GPU runs a chunked
prefill (ssd_chunk_scan_fwd) and then decode steps from its final_state."""
import numpy as np
import pytest
import torch

import oracle
from chunked_linear_recurrence_amd import inputs, ssd

from helpers import err_bf16, err_f32, err_for, tol_for, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _token(d, t):
    """Token t of a layer's inputs, in the step's layouts."""
    return (d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["B"][:, t].contiguous(),
            d["C"][:, t].contiguous())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_then_decode_matches_sequential(dtype):
    """Chunked prefill over L tokens, then T single-token steps: every decoded output and
    the final state match the fp64 recurrence over all L + T tokens."""
    b, L, T, H, P, N, G, Q = 2, 3 * 256 + 40, 24, 4, 64, 128, 2, 256
    if dtype == "f32":
        P, N, Q = 32, 64, 64
    d = inputs.make_layer(b, L + T, H, P, N, G, dtype, seed=11, init="normal", init_std=0.3)
    g = to_dev(d, DEV)
    pre = {k: (v[:, :L].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in g.items()}
    y_pre, state = ssd.fwd(pre["x"], pre["dt"], pre["A"], pre["B"], pre["C"], pre["D"], pre["init_state"], Q)
    ys = []
    for t in range(L, L + T):
        x, dt, B, C = _token(g, t)
        ys.append(ssd.step(x, dt, g["A"], B, C, g["D"], state))
    torch.cuda.synchronize()
    yr, fr = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"])
    err = err_for(dtype)
    assert err(y_pre, yr[:, :L]) <= tol_for(dtype)
    assert err(torch.stack(ys, dim=1), yr[:, L:]) <= tol_for(dtype)
    assert err(state, fr) <= tol_for(dtype)


@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_steps_every_dstate(dtype, N):
    """Decode only (from a random state), every supported N, P not a power of two, G = 2."""
    b, T, H, P, G = 3, 6, 4, 24, 2
    d = inputs.make_layer(b, T, H, P, N, G, dtype, seed=N, init="normal", init_std=0.5)
    g = to_dev(d, DEV)
    state = g["init_state"].clone()
    ys = []
    for t in range(T):
        x, dt, B, C = _token(g, t)
        ys.append(ssd.step(x, dt, g["A"], B, C, g["D"], state))
    torch.cuda.synchronize()
    yr, fr = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"])
    err = err_for(dtype)
    assert err(torch.stack(ys, dim=1), yr) <= tol_for(dtype)
    assert err(state, fr) <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_residual_and_no_skip(dtype):
    b, H, P, N = 1, 2, 64, 64
    d = inputs.make_layer(b, 1, H, P, N, 1, dtype, seed=3, init="normal", init_std=0.5)
    g = to_dev(d, DEV)
    x, dt, B, C = _token(g, 0)
    s1 = g["init_state"].clone()
    y1 = ssd.step(x, dt, g["A"], B, C, g["D"], s1, residual=True)
    s2 = g["init_state"].clone()
    y2 = ssd.step(x, dt, g["A"], B, C, None, s2)
    torch.cuda.synchronize()
    yr1, fr = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"])
    yr1 = yr1 + oracle.to_f64(d["x"])
    yr2, _ = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], None, d["init_state"])
    err = err_for(dtype)
    assert err(y1, yr1[:, 0]) <= tol_for(dtype)
    assert err(y2, yr2[:, 0]) <= tol_for(dtype)
    assert torch.equal(s1, s2)                      # the state does not depend on D or the flag
    assert err(s1, fr) <= tol_for(dtype)


def test_step_long_context_shape():
    """The 128K-token layer's shape (H = 48, P = 64, N = 128) at batch 1 and 8: 50 steps."""
    for b in (1, 8):
        d = inputs.make_layer(b, 50, 48, 64, 128, 1, "bf16", seed=b, init="normal", init_std=0.5,
                              dt_max=1e-2)
        g = to_dev(d, DEV)
        state = g["init_state"].clone()
        ys = []
        for t in range(50):
            x, dt, B, C = _token(g, t)
            ys.append(ssd.step(x, dt, g["A"], B, C, g["D"], state))
        torch.cuda.synchronize()
        yr, fr = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"])
        assert err_bf16(torch.stack(ys, dim=1), yr) <= 2e-2
        assert err_bf16(state, fr) <= 2e-2
