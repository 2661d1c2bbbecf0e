"""GPU parity of the associative-scan form of the chunk outputs (SSD_FLAG_SCAN_FORM): the
log-depth tree over (a_t, x_t B_t) of [分块推理 §2.1] of the page
"分块推理：解锁循环模型并行计算，实现长序列高效处理", run in place of the matrix-core
chunk_scan, against the fp64 oracle and against the matrix-core form."""
import pytest
import torch

import oracle
from chunked_linear_recurrence_amd import inputs, ssd

from helpers import err_bf16, err_for, tol_for, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SHAPES = [("bf16", 32, 64, 64), ("bf16", 64, 32, 64), ("bf16", 64, 64, 128), ("bf16", 128, 64, 128),
          ("bf16", 256, 64, 128), ("f32", 64, 32, 64), ("f32", 64, 64, 64)]


@pytest.mark.parametrize("dtype,Q,P,N", SHAPES)
def test_scan_form_matches_oracle(dtype, Q, P, N):
    code = 1 if dtype == "bf16" else 0
    assert ssd.scan_form_supported(code, Q, P, N)
    d = inputs.make_layer(2, 3 * Q + 13, 4, P, N, 2, dtype, seed=Q + P, init="normal", init_std=0.5)
    g = to_dev(d, DEV)
    y, fin = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], Q, scan_form=True)
    torch.cuda.synchronize()
    yr, fr = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"])
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype)
    assert err(fin, fr) <= tol_for(dtype)


def test_scan_form_residual_and_against_matrix_form():
    d = inputs.make_layer(1, 1000, 3, 64, 128, 1, "bf16", seed=4)
    g = to_dev(d, DEV)
    ys, _ = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, 256, residual=True, scan_form=True)
    ym, _ = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, 256, residual=True)
    torch.cuda.synchronize()
    yr, _ = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None)
    yr = yr + oracle.to_f64(d["x"])
    assert err_bf16(ys, yr) <= 2e-2
    assert err_bf16(ys, ym) <= 2e-2
