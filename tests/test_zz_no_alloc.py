"""ssd_chunk_scan_fwd_noalloc (the entry point for callers that cannot allocate) against
ssd_chunk_scan_fwd with a caller workspace: the same kernels, so the outputs must agree
bit for bit (stronger than the parity tolerance).  Calls run back to back on one GPU and
share the library's scratch: a large call close to the scratch limit, then smaller ones,
whose results must not depend on what the earlier call left behind."""
import pytest
import torch

from chunked_linear_recurrence_amd import inputs, ssd

from helpers import err_for, tol_for, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # (batch, L, H, P, N, G, dtype, Q, init)
    (1, 65536, 7, 64, 128, 1, "bf16", 256, "zero"),     # ~60 MB of workspace (limit 64 MiB)
    (2, 3000, 24, 64, 128, 1, "bf16", 256, "normal"),   # smaller, nonzero init
    (1, 700, 4, 32, 64, 2, "bf16", 64, "normal"),       # smaller still, two groups, ragged
    (2, 300, 2, 16, 16, 1, "f32", 64, "normal"),        # fp32
]


def _run(case, residual=False):
    b, L, H, P, N, G, dtype, Q, init = case
    d = inputs.make_layer(b, L, H, P, N, G, dtype, seed=L + H, init=init, init_std=0.5)
    g = to_dev(d, DEV)
    dims = ssd.dims_of(g["x"], g["B"])
    assert ssd.workspace_bytes(dims, Q) <= ssd.NOALLOC_SCRATCH_BYTES
    y_ref, f_ref = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], Q,
                           residual=residual)
    y = torch.full_like(g["x"], float("nan"))
    fin = torch.full((b, H, P, N), float("nan"), device=DEV)
    ssd.fwd_noalloc(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], Q, y=y,
                    final_state=fin, residual=residual)
    torch.cuda.synchronize()
    return dtype, y, fin, y_ref, f_ref


def test_noalloc_equals_workspace_entry_point_in_sequence():
    for k, case in enumerate(CASES):
        print("[noalloc case %d] %s" % (k, case), flush=True)
        dtype, y, fin, y_ref, f_ref = _run(case, residual=(k == 2))
        assert torch.equal(y, y_ref), case
        assert torch.equal(fin, f_ref), case
        assert err_for(dtype)(y, y_ref) <= tol_for(dtype)


def test_noalloc_second_call_smaller_after_larger():
    """Two calls in a row, the second with a smaller input than the first."""
    for case in (CASES[1], CASES[2]):
        dtype, y, fin, y_ref, f_ref = _run(case)
        assert torch.equal(y, y_ref) and torch.equal(fin, f_ref), case


def test_noalloc_rejects_oversized_call_on_the_gpu():
    d = inputs.make_layer(1, 256 * 300, 7, 64, 128, 1, "bf16", seed=1)
    g = to_dev(d, DEV)
    assert ssd.workspace_bytes(ssd.dims_of(g["x"], g["B"]), 256) > ssd.NOALLOC_SCRATCH_BYTES
    y = torch.empty_like(g["x"])
    with pytest.raises(ssd.SSDError, match="SSD_ERR_WORKSPACE"):
        ssd.fwd_noalloc(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, 256, y=y)
