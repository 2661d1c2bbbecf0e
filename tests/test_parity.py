"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Same seeded inputs on both sides; every comparison is element by element, at the
tolerance of the activation dtype (see helpers.py).  Sizes span several chunks and a
ragged last chunk; the named workloads run at their full sizes, every output element
compared.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from chunked_linear_recurrence_amd import inputs, ssd, WORKLOADS

from helpers import err_f32, err_bf16, err_for, tol_for, to_dev, as_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gpu(d, Q, residual=False, last_stage=ssd.NSTAGES, with_final=True):
    g = to_dev(d, DEV)
    y, fin = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g.get("init_state"), Q,
                     residual=residual, want_final=with_final, last_stage=last_stage)
    torch.cuda.synchronize()
    return y, fin


def oracle_layer(d, residual=False):
    y, fin = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d.get("init_state"))
    if residual:
        y = y + oracle.to_f64(d["x"])
    return y, fin


def small(batch, L, H, P, N, G, dtype, seed, init=True, dt_max=0.1):
    return inputs.make_layer(batch, L, H, P, N, G, dtype, seed=seed, dt_max=dt_max,
                             init="normal" if init else "zero", init_std=0.5)


# --------------------------------------------------------------------- per stage

@pytest.mark.parametrize("dtype,b,L,H,P,N,G,Q", [
    ("f32", 2, 3 * 64 + 17, 4, 32, 64, 2, 64),
    ("bf16", 2, 3 * 64 + 17, 4, 32, 64, 2, 64),
    ("bf16", 2, 3 * 256 + 37, 3, 64, 128, 1, 256),     # the shape of the 128K-token layer
    ("f32", 2, 2 * 256 + 9, 2, 64, 128, 1, 256),
])
def test_stages_match_oracle_intermediates(dtype, b, L, H, P, N, G, Q):
    """dA_cum, b_intra and b_in left in the workspace match the oracle's chunked
    decomposition (logcum, b_intra, b_in) of [分块推理 §2.1-§2.2]."""
    d = small(b, L, H, P, N, G, dtype, seed=5 + Q)
    ref = oracle.chunked(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init_state"], Q)
    g = to_dev(d, DEV)
    dims = ssd.dims_of(g["x"], g["B"])
    offs = ssd.workspace_layout(dims, Q)
    ws = torch.zeros(ssd.workspace_bytes(dims, Q), dtype=torch.uint8, device=DEV)
    ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], Q, workspace=ws,
            last_stage=3)
    torch.cuda.synchronize()
    nc = (L + Q - 1) // Q
    cdt, ce = (torch.float64, 8) if dtype == "f32" else (torch.float32, 4)
    cum = ws[offs[0]:offs[0] + b * H * nc * Q * ce].view(cdt).reshape(b, H, nc, Q)
    cum = as_np(cum) * math.log(2.0)        # the library keeps base-2 sums (dt A / ln 2)
    lc = ref["logcum"]
    valid = ~np.isnan(lc)
    ctol = 1e-12 if dtype == "f32" else 1e-5      # fp64 sums for fp32 activations
    assert np.abs(cum[valid] - lc[valid]).max() <= ctol * (1 + np.abs(lc[valid]).max())
    # past the short last chunk: the chunk total
    qlast = L - (nc - 1) * Q
    assert np.allclose(cum[:, :, -1, qlast:], cum[:, :, -1, qlast - 1:qlast], rtol=0, atol=0)
    e = 4 if dtype == "f32" else 2
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    bint = ws[offs[1]:offs[1] + b * nc * H * P * N * e].view(tdt)
    bint = as_np(ssd.tile_order_to_pn(bint.reshape(b, nc, H, P * N), P, N))
    bin_ = ws[offs[2]:offs[2] + b * nc * H * P * N * e].view(tdt)
    bin_ = as_np(ssd.tile_order_to_pn(bin_.reshape(b, nc, H, P * N), P, N))
    err = err_for(dtype)
    tol = tol_for(dtype)
    for c in range(nc):
        assert err(bint[:, c], ref["b_intra"][:, c]) <= tol, ("b_intra", c)
        assert err(bin_[:, c], ref["b_in"][:, c]) <= tol, ("b_in", c)


# ------------------------------------------------------------------ full layers

@pytest.mark.parametrize("name", ["tiny_fp32_L256", "mamba2_130m_layer_b2_L2048",
                                  "throughput_b8_L4096_h32"])
def test_workload_parity(name):
    w = WORKLOADS[name]
    d = inputs.make(w)
    y, fin = run_gpu(d, w.chunk)
    yr, fr = oracle_layer(d)
    err = err_for(w.dtype)
    assert err(y, yr) <= tol_for(w.dtype)
    assert err(fin, fr) <= tol_for(w.dtype)


def _err_bf16_by_head(got, ref, head_axis):
    """The bf16 metric over a whole tensor, max |got - ref| / max |ref|, accumulated one
    head at a time (the full 128K-token tensors are 400 M elements)."""
    num = den = 0.0
    for h in range(ref.shape[head_axis]):
        r = np.take(ref, h, axis=head_axis)
        gh = as_np(got.select(head_axis, h))
        num = max(num, float(np.abs(gh - r).max()))
        den = max(den, float(np.abs(r).max()))
    return num / (den if den > 0 else 1.0)


@pytest.fixture(scope="module")
def long_context():
    """Inputs of the 128K-token layer and the fp64 recurrence over all of it (computed once
    for the tests below)."""
    w = WORKLOADS["long_context_b1_L131072_h48"]
    d = inputs.make(w)
    yr, fr = oracle_layer(d)
    return w, d, yr, fr


@pytest.mark.slow
@pytest.mark.parametrize("Q", [256, 128, 64])
def test_long_context_parity_every_head(long_context, Q):
    """128K tokens, 48 heads: every output and every final-state element against the fp64
    recurrence over the whole sequence, at the workload's Q = 256 (512 chunks) and at
    Q = 128 and 64 (1024 and 2048 chunks).  For Q < 256 a chunk's decay rows are less than
    one wave of 16-byte pieces, and the per-lane guard on their DMA keeps every read inside
    the workspace (whose end coincides with the allocation's at this size)."""
    w, d, yr, fr = long_context
    y, fin = run_gpu(d, Q)
    ycpu = y.cpu()
    del y
    e_y = _err_bf16_by_head(ycpu, yr, 2)
    e_f = err_bf16(fin, fr)
    print("long context Q=%d: y err %.3g, final_state err %.3g" % (Q, e_y, e_f))
    assert e_y <= 2e-2
    assert e_f <= 2e-2
    assert torch.isfinite(ycpu.float()).all()


@pytest.mark.parametrize("case", range(12))
def test_random_shapes(case):
    rng = np.random.default_rng(1000 + case)
    dtype = ["f32", "bf16"][case % 2]
    Q = [64, 128, 256][case % 3]
    P = int(rng.choice([16, 32, 64])) if Q == 256 else int(rng.choice([32, 64]))
    N = int(rng.choice([32, 64, 128]))
    code = 0 if dtype == "f32" else 1
    if not ssd.shape_supported(code, Q, P, N):
        P, N = next((pp, nn) for pp, nn in ((64, 64), (32, 64), (16, 32), (16, 16))
                    if ssd.shape_supported(code, Q, pp, nn))
    G = int(rng.choice([1, 2]))
    H = G * int(rng.integers(1, 4))
    b = int(rng.integers(1, 3))
    L = int(rng.integers(1, 4)) * Q + int(rng.integers(1, Q))      # ragged last chunk
    d = small(b, L, H, P, N, G, dtype, seed=case, init=bool(case % 3))
    y, fin = run_gpu(d, Q)
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype), (dtype, Q, P, N, G, H, b, L)
    assert err(fin, fr) <= tol_for(dtype)


@pytest.mark.parametrize("nc", [7, 8, 9, 16, 17])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_pass_chain_lengths(nc, dtype):
    """Chains on both sides of the state pass's short-chain kernels (at most 8 and at most
    16 chunks, several element groups per wave) and of its streaming kernel beyond, with a
    ragged last chunk and a nonzero initial state: y and final_state against the oracle."""
    Q, P, N = 64, 32, 64
    d = small(2, (nc - 1) * Q + 5, 3, P, N, 1, dtype, seed=300 + nc, init=True)
    y, fin = run_gpu(d, Q)
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype), (dtype, nc)
    assert err(fin, fr) <= tol_for(dtype), (dtype, nc)


# ------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("L", [1, 17, 64, 65, 255, 256, 257])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_short_and_ragged_lengths(L, dtype):
    Q, P, N = (64, 16, 16) if dtype == "f32" else (256, 32, 64)
    d = small(2, L, 2, P, N, 1, dtype, seed=L)
    y, fin = run_gpu(d, Q)
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype)
    assert err(fin, fr) <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_residual_flag_and_no_skip(dtype):
    d = small(1, 300, 2, 64, 64, 1, dtype, seed=3)
    y, _ = run_gpu(d, 64, residual=True)
    yr, _ = oracle_layer(d, residual=True)
    assert err_for(dtype)(y, yr) <= tol_for(dtype)
    d["D"] = None
    y2, _ = run_gpu(d, 64)
    yr2, _ = oracle.seq(d["x"], d["dt"], d["A"], d["B"], d["C"], None, d["init_state"])
    assert err_for(dtype)(y2, yr2) <= tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_special_cases(dtype):
    """a = 1 (A = 0): prefix sums; a = 0 (A very negative): only the current token."""
    d = small(1, 200, 2, 32, 32, 1, dtype, seed=9)
    d["A"] = torch.zeros_like(d["A"])
    y, fin = run_gpu(d, 64)
    yr, fr = oracle_layer(d)
    assert err_for(dtype)(y, yr) <= tol_for(dtype)
    assert err_for(dtype)(fin, fr) <= tol_for(dtype)
    d["A"] = torch.full_like(d["A"], -1e4)
    y, fin = run_gpu(d, 64)
    yr, fr = oracle_layer(d)
    assert err_for(dtype)(y, yr) <= tol_for(dtype)
    assert err_for(dtype)(fin, fr) <= tol_for(dtype)


def test_final_state_in_place_and_determinism():
    d = small(2, 600, 4, 64, 128, 1, "bf16", seed=4)
    g = to_dev(d, DEV)
    st = g["init_state"].clone()
    y1, _ = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], st, 256, final_state=st)
    y2, f2 = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], 256)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(st, f2)
    y3, f3 = ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], 256)
    torch.cuda.synchronize()
    assert torch.equal(y2, y3) and torch.equal(f2, f3)


def test_narrow_dt_variant():
    """Per-token dt variation in the narrow range (log-uniform in [1e-3, 1e-2])."""
    d = inputs.make_layer(1, 4096 + 100, 4, 64, 128, 1, "bf16", seed=2, dt_min=1e-3, dt_max=1e-2,
                          dt_dist="loguniform")
    y, fin = run_gpu(d, 256)
    yr, fr = oracle_layer(d)
    assert err_bf16(y, yr) <= 2e-2
    assert err_bf16(fin, fr) <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("P,N", [(32, 64), (64, 64), (64, 128)])
def test_chunk_length_32(dtype, P, N):
    """Q = 32 (the smallest chunk the pages list, for other model families): several chunks,
    a ragged tail, two groups, a nonzero initial state."""
    d = small(2, 5 * 32 + 11, 4, P, N, 2, dtype, seed=P + N)
    y, fin = run_gpu(d, 32)
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype)
    assert err(fin, fr) <= tol_for(dtype)


def test_head_grouping_does_not_change_the_result(monkeypatch):
    """Heads per workgroup only split the work: every split gives bit-identical outputs
    (ngroups 4, heads per group 3, so some splits leave a short last group)."""
    d = small(2, 700, 12, 64, 128, 4, "bf16", seed=21)
    outs = []
    for hs, hc in (("1", "1"), ("2", "3"), ("3", "2"), ("64", "64")):
        monkeypatch.setenv("SSD_HEADS_PER_WG_STATE", hs)
        monkeypatch.setenv("SSD_HEADS_PER_WG_SCAN", hc)
        outs.append(run_gpu(d, 256))
    for y, fin in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(fin, outs[0][1])
    yr, fr = oracle_layer(d)
    assert err_bf16(outs[0][0], yr) <= 2e-2


@pytest.mark.parametrize("dtype,Q,P,N", [
    ("bf16", 256, 64, 128),      # separate staging rows (the tuned shape)
    ("bf16", 256, 64, 256),      # outputs staged in place
    ("f32", 128, 64, 128),       # outputs staged in place
    ("bf16", 256, 128, 128),     # each head as two channel units
    ("f32", 256, 64, 64),        # each head as two channel units
])
def test_staging_modes_over_several_heads(monkeypatch, dtype, Q, P, N):
    """chunk_scan's staging modes and channel units, and chunk_state's wave split, with
    several heads per workgroup (the outputs of one head are staged and stored while the
    next is computed): against the oracle, and bit-identical to one head per workgroup."""
    code = 0 if dtype == "f32" else 1
    if not ssd.shape_supported(code, Q, P, N):
        pytest.skip("shape not compiled")
    d = small(2, 2 * Q + 37, 6, P, N, 2, dtype, seed=Q + P + N)
    outs = []
    for hc in ("1", "3"):
        monkeypatch.setenv("SSD_HEADS_PER_WG_SCAN", hc)
        monkeypatch.setenv("SSD_HEADS_PER_WG_STATE", hc)
        outs.append(run_gpu(d, Q))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(outs[1][0], yr) <= tol_for(dtype), (dtype, Q, P, N)
    assert err(outs[1][1], fr) <= tol_for(dtype), (dtype, Q, P, N)


def _compiled_shapes():
    try:
        return [(dt, Q, P, N) for dt in (0, 1) for Q in (32, 64, 128, 256) for P in (16, 32, 64, 128)
                for N in (16, 32, 64, 128, 256) if ssd.shape_supported(dt, Q, P, N)]
    except Exception:            # library not built: nothing to parametrize over
        return []


@pytest.mark.parametrize("code,Q,P,N", _compiled_shapes())
def test_every_compiled_shape(code, Q, P, N):
    """Every (dtype, Q, P, N) the library compiles, including the largest (P = 128,
    N = 256) and the single-buffer fp32 ones: three chunks with a ragged tail, two groups,
    a nonzero initial state."""
    dtype = "f32" if code == 0 else "bf16"
    d = small(1, 2 * Q + 5, 4, P, N, 2, dtype, seed=Q * 7 + P + N)
    y, fin = run_gpu(d, Q)
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype), (dtype, Q, P, N)
    assert err(fin, fr) <= tol_for(dtype), (dtype, Q, P, N)


@pytest.mark.parametrize("b,L,H,G,dtype", [
    (33, 300, 3, 1, "bf16"),      # large odd batch, three heads
    (5, 700, 20, 4, "bf16"),      # heads split unevenly over cumsum blocks and head groups
    (2, 1100, 96, 2, "bf16"),     # many heads
    (17, 150, 5, 5, "f32"),       # fp32, one head per group, every chunk short
])
def test_batch_and_head_counts(b, L, H, G, dtype):
    Q, P, N = (256, 64, 128) if dtype == "bf16" else (64, 32, 64)
    d = small(b, L, H, P, N, G, dtype, seed=b * 100 + H)
    y, fin = run_gpu(d, Q)
    yr, fr = oracle_layer(d)
    err = err_for(dtype)
    assert err(y, yr) <= tol_for(dtype)
    assert err(fin, fr) <= tol_for(dtype)
