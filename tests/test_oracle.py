"""Pins of the fp64 CPU oracle (no GPU, no HIP library).

Each test fixes part of the oracle with something other than the oracle itself: values
worked by hand (tests/golden/), a textbook routine (scipy's IIR filter), closed forms,
a brute-force unrolling, invariants of the method and torch's bfloat16 cast.  The method
is the one of the page "分块推理：解锁循环模型并行计算，实现长序列高效处理" (§2-§3).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import torch

import oracle
from oracle import brute
from chunked_linear_recurrence_amd import inputs, WORKLOADS

from conftest import GOLDEN


def _gold(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / scale)


def _scalar_problem(xs, a, B=1.0, C=1.0, D=0.0):
    L = len(xs)
    x = np.asarray(xs, dtype=np.float64).reshape(1, L, 1, 1)
    # a = exp(dt * A) with A = -1, dt = -ln(a)
    dt = np.full((1, L, 1), -math.log(a))
    A = np.array([-1.0])
    Bv = np.full((1, L, 1, 1), B)
    Cv = np.full((1, L, 1, 1), C)
    return x, dt, A, Bv, Cv, np.array([D])


def _random_problem(rng, batch, L, H, P, N, G, h0=True, dt_range=(0.01, 0.5)):
    x = rng.standard_normal((batch, L, H, P))
    dt = rng.uniform(*dt_range, size=(batch, L, H))
    A = -np.exp(rng.uniform(0, math.log(16), size=H))
    B = rng.standard_normal((batch, L, G, N)) / math.sqrt(N)
    C = rng.standard_normal((batch, L, G, N)) / math.sqrt(N)
    D = rng.uniform(0, 1, size=H)
    init = rng.standard_normal((batch, H, P, N)) * 0.3 if h0 else None
    return x, dt, A, B, C, D, init


# ----------------------------------------------------------------------------- golden

def test_golden_scalar_halving():
    g = _gold("scalar_halving.json")
    for case in g["cases"]:
        x, dt, A, B, C, D = _scalar_problem([1.0] * 4, 0.5)
        init = np.full((1, 1, 1, 1), case["h0"])
        y, fin = oracle.seq(x, dt, A, B, C, D, init)
        assert np.allclose(y.ravel(), case["y"], rtol=0, atol=1e-14)
        assert abs(fin.item() - case["final"]) < 1e-14
        for Q in (1, 2, 3, 4, 5):
            o = oracle.chunked(x, dt, A, B, C, D, init, Q)
            assert np.allclose(o["y"].ravel(), case["y"], rtol=0, atol=1e-14)
            assert abs(o["final_state"].item() - case["final"]) < 1e-14


def test_golden_chunked_intermediates():
    g = _gold("chunked_L4_Q2.json")
    x, dt, A, B, C, D = _scalar_problem(g["x"], 0.5)
    o = oracle.chunked(x, dt, A, B, C, D, None, g["Q"])
    tol = dict(rtol=0, atol=1e-14)
    assert np.allclose(o["by_intra"].ravel(), g["by_intra"], **tol)
    assert np.allclose(o["b_intra"].ravel(), g["b_intra"], **tol)
    assert np.allclose(o["b_in"].ravel(), g["b_in"], **tol)
    assert np.allclose(o["by_inter"].ravel(), g["by_inter"], **tol)
    assert np.allclose(o["y"].ravel(), g["y"], **tol)
    assert abs(o["final_state"].item() - g["final"]) < 1e-14
    assert np.allclose(o["logcum"][0, 0] / math.log(2.0), g["logcum_over_ln2"], **tol)
    y, fin = oracle.seq(x, dt, A, B, C, D)
    assert np.allclose(y.ravel(), g["y"], **tol)


def test_golden_outer_product_orientation():
    g = _gold("outer_product_P2_N3.json")
    x = np.array(g["x"]).reshape(1, 1, 1, 2)
    dt = np.ones((1, 1, 1))
    A = np.array([-1.0])
    B = np.array(g["B"]).reshape(1, 1, 1, 3)
    C = np.array(g["C"]).reshape(1, 1, 1, 3)
    D = np.array([g["D"]])
    for fn in ("seq", "chunked"):
        if fn == "seq":
            y, fin = oracle.seq(x, dt, A, B, C, D)
        else:
            o = oracle.chunked(x, dt, A, B, C, D, None, 1)
            y, fin = o["y"], o["final_state"]
        assert np.array_equal(y.ravel(), g["y"])
        assert np.array_equal(fin[0, 0], np.array(g["final"]))


def test_golden_two_layer_stack():
    g = _gold("stack_2layer_residual.json")
    x0 = np.array(g["x0"]).reshape(1, 2, 1, 1)
    dt = np.full((1, 2, 1), math.log(2.0))
    B = np.ones((1, 2, 1, 1))
    C = np.ones((1, 2, 1, 1))
    A = np.full((2, 1), -1.0)
    D = np.zeros((2, 1))
    out_h, fin_h = oracle.stack_horizontal(x0, dt, A, B, C, D)
    out_v, fin_v = oracle.stack_vertical(x0, dt, A, B, C, D, V=1)
    for out, fin in ((out_h, fin_h), (out_v, fin_v)):
        assert np.allclose(out.ravel(), g["out"], rtol=0, atol=1e-14)
        assert np.allclose(fin.ravel(), g["finals"], rtol=0, atol=1e-14)


# ----------------------------------------------------------------- P1: brute force

@pytest.mark.parametrize("seed", range(6))
def test_seq_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    batch = 1 + seed % 2
    G = 1 + seed % 2
    H = G * (1 + (seed // 2) % 3)
    P, N = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    L = int(rng.integers(1, 20))
    prob = _random_problem(rng, batch, L, H, P, N, G)
    y, fin = oracle.seq(*prob)
    yb, finb = brute.closed_form(*prob)
    assert _rel(y, yb) < 1e-12
    assert _rel(fin, finb) < 1e-12


def test_group_mapping_contiguous():
    """Heads 0..H/G-1 read group 0, the next H/G heads group 1 (per the brute-force rule);
    swapping the groups' B/C must change exactly the heads that read them."""
    rng = np.random.default_rng(7)
    x, dt, A, B, C, D, init = _random_problem(rng, 1, 9, 4, 3, 5, 2)
    y, _ = oracle.seq(x, dt, A, B, C, D, init)
    B2, C2 = B[:, :, ::-1].copy(), C[:, :, ::-1].copy()
    y2, _ = oracle.seq(x, dt, A, B2, C2, D, init)
    # heads 0,1 now read the former group 1 and heads 2,3 the former group 0
    yb, _ = brute.closed_form(x[:, :, [2, 3, 0, 1]], dt[:, :, [2, 3, 0, 1]], A[[2, 3, 0, 1]],
                              B, C, D[[2, 3, 0, 1]], init[:, [2, 3, 0, 1]])
    assert _rel(y2[:, :, [2, 3, 0, 1]], yb) < 1e-12
    assert _rel(y, y2) > 1e-3


# --------------------------------------------------- P2: chunked == sequential, all Q

@pytest.mark.parametrize("L", [1, 7, 16, 37])
def test_chunked_equals_sequential_every_Q(L):
    rng = np.random.default_rng(L)
    prob = _random_problem(rng, 2, L, 2, 3, 4, 1)
    y, fin = oracle.seq(*prob)
    for Q in range(1, L + 2):
        o = oracle.chunked(*prob, Q)
        assert _rel(o["y"], y) < 1e-12, Q
        assert _rel(o["final_state"], fin) < 1e-12, Q
        # y is the sum of its parts [分块推理 §2.2]
        x, D = prob[0], prob[5]
        assert _rel(o["by_intra"] + o["by_inter"] + D[None, None, :, None] * x, y) < 1e-12


@pytest.mark.parametrize("name,Q,heads", [("tiny_fp32_L256", 64, None),
                                           ("tiny_fp32_L256", 256, None),
                                           ("mamba2_130m_layer_b2_L2048", 256, 3),
                                           ("mamba2_130m_layer_b2_L2048", 64, 3)])
def test_chunked_equals_sequential_workload_shapes(name, Q, heads):
    d = inputs.make(WORKLOADS[name])
    x, dt, A, D = d["x"], d["dt"], d["A"], d["D"]
    if heads:
        x, dt, A, D = x[:, :, :heads], dt[:, :, :heads], A[:heads], D[:heads]
    y, fin = oracle.seq(x, dt, A, d["B"], d["C"], D)
    o = oracle.chunked(x, dt, A, d["B"], d["C"], D, None, Q)
    assert _rel(o["y"], y) < 1e-12
    assert _rel(o["final_state"], fin) < 1e-12


def test_chunk_states_compose():
    """b_in of chunk c+1 is the end state of running tokens [0, (c+1)Q) sequentially."""
    rng = np.random.default_rng(3)
    prob = _random_problem(rng, 1, 23, 2, 3, 4, 1)
    Q = 5
    o = oracle.chunked(*prob, Q)
    x, dt, A, B, C, D, init = prob
    for c in range(1, 5):
        t = c * Q
        _, fin = oracle.seq(x[:, :t], dt[:, :t], A, B[:, :t], C[:, :t], D, init)
        assert _rel(o["b_in"][:, c], fin) < 1e-12


def _intermediate_mismatches(o, prob, Q):
    """Names of the chunked intermediates in `o` that differ from a computation sharing no
    step with the decomposition [分块推理 §2.1-§2.2]:
      b_intra(c)  = final state of the sequential recurrence run from a zero state over
                    chunk c's tokens alone;
      by_intra(c) = that run's output without the skip term;
      logcum      = numpy's cumulative sum of dt * A within each chunk (NaN past the end);
      b_in(c)     = final state of the recurrence run from init_state over tokens [0, cQ);
      by_inter_i  = (product of exp(dt A) from the chunk start to token i, by np.prod)
                    times C_i contracted with b_in(c)."""
    x, dt, A, B, C, D, init = prob
    b, L, H, P = x.shape
    G = B.shape[2]
    bad = set()
    for c in range(-(-L // Q)):
        t0, t1 = c * Q, min(c * Q + Q, L)
        sl = slice(t0, t1)
        y0, f0 = oracle.seq(x[:, sl], dt[:, sl], A, B[:, sl], C[:, sl], None, None)
        if _rel(o["b_intra"][:, c], f0) > 1e-12:
            bad.add("b_intra")
        if _rel(o["by_intra"][:, sl], y0) > 1e-12:
            bad.add("by_intra")
        if c == 0:
            ref_in = init
        else:
            _, ref_in = oracle.seq(x[:, :t0], dt[:, :t0], A, B[:, :t0], C[:, :t0], D, init)
        if _rel(o["b_in"][:, c], ref_in) > 1e-12:
            bad.add("b_in")
        for bb in range(b):
            for h in range(H):
                ref = np.cumsum(dt[bb, sl, h] * A[h])
                lc = o["logcum"][bb, h, c]
                if not (np.allclose(lc[:t1 - t0], ref, rtol=1e-13, atol=1e-15)
                        and np.isnan(lc[t1 - t0:]).all()):
                    bad.add("logcum")
                g = h // (H // G)
                a = np.exp(dt[bb, sl, h] * A[h])
                for i, t in enumerate(range(t0, t1)):
                    ref = np.prod(a[:i + 1]) * (ref_in[bb, h] @ C[bb, t, g])
                    if not np.allclose(o["by_inter"][bb, t, h], ref, rtol=1e-12, atol=1e-14):
                        bad.add("by_inter")
    return bad


def _intermediates_problem(Q):
    rng = np.random.default_rng(40 + Q)
    return _random_problem(rng, 2, 23, 4, 3, 5, 2)      # b 2, L 23, H 4 in 2 groups, P 3, N 5


@pytest.mark.parametrize("Q", [4, 5, 9])
def test_chunked_intermediates_against_per_chunk_runs(Q):
    """Every intermediate oracle.chunked exports, at batch 2, 4 heads in 2 groups, P = 3,
    N = 5, a nonzero initial state and a ragged last chunk, equals its independent
    computation (_intermediate_mismatches)."""
    prob = _intermediates_problem(Q)
    o = oracle.chunked(*prob, Q)
    nc = -(-23 // Q)
    assert o["b_intra"].shape == (2, nc, 4, 3, 5) and o["logcum"].shape == (2, 4, nc, Q)
    assert _intermediate_mismatches(o, prob, Q) == set()


def test_intermediates_pin_catches_planted_index_slips():
    """Index slips planted in a copy of the oracle's exports (on the CPU): heads swapped,
    batch rows swapped, chunk index shifted, a transposed P x N state, an exclusive
    prefix.  Each is seen by the per-chunk pin above."""
    Q = 5
    prob = _intermediates_problem(Q)
    o = oracle.chunked(*prob, Q)
    plants = {
        "b_intra": lambda o: o["b_intra"][:, :, [1, 0, 2, 3]],                    # heads
        "b_in": lambda o: np.concatenate([o["b_in"][:, 1:], o["b_in"][:, -1:]], 1),  # chunk + 1
        "by_intra": lambda o: o["by_intra"][::-1],                               # batch rows
        "logcum": lambda o: np.concatenate([np.zeros_like(o["logcum"][..., :1]),
                                            o["logcum"][..., :-1]], -1),        # exclusive
        "by_inter": lambda o: o["by_inter"][:, :, [0, 1, 3, 2]],                  # heads
    }
    for name, plant in plants.items():
        bad = dict(o)
        bad[name] = np.ascontiguousarray(plant(o))
        assert name in _intermediate_mismatches(bad, prob, Q), name
    # a transposed state (P = 3, N = 5 read as N x P) cannot even keep its shape
    t = o["b_intra"].reshape(2, -1, 4, 5, 3).swapaxes(-1, -2)
    assert not np.array_equal(t, o["b_intra"])
    bad = dict(o, b_intra=np.ascontiguousarray(t))
    assert "b_intra" in _intermediate_mismatches(bad, prob, Q)


# ------------------------------------------------------- P3: a == 1 is a prefix sum

def test_a_equal_one_is_prefix_sum():
    rng = np.random.default_rng(11)
    x, dt, A, B, C, D, init = _random_problem(rng, 2, 33, 3, 4, 5, 1)
    A = np.zeros_like(A)
    y, fin = oracle.seq(x, dt, A, B, C, D, init)
    outer = x[:, :, :, :, None] * B[:, :, 0, None, None, :]          # [b,L,H,P,N]
    S = init[:, None] + np.cumsum(outer, axis=1)
    ref = np.einsum("blhpn,bln->blhp", S, C[:, :, 0]) + D[None, None, :, None] * x
    assert _rel(y, ref) < 1e-12
    assert _rel(fin, S[:, -1]) < 1e-12
    o = oracle.chunked(x, dt, A, B, C, D, init, 8)
    assert _rel(o["y"], ref) < 1e-12


# ------------------------------------------- P4: a == 0 keeps only the current token

def test_a_equal_zero_keeps_current_token():
    rng = np.random.default_rng(12)
    x, dt, A, B, C, D, init = _random_problem(rng, 2, 19, 3, 4, 5, 1, dt_range=(1e-3, 0.1))
    A = np.full_like(A, -1e6)                 # exp(dt * A) underflows to exactly 0
    y, fin = oracle.seq(x, dt, A, B, C, D, init)
    cb = np.sum(C[:, :, 0] * B[:, :, 0], axis=-1)                     # [b,L]
    ref = cb[:, :, None, None] * x + D[None, None, :, None] * x
    assert _rel(y, ref) < 1e-15
    last = x[:, -1, :, :, None] * B[:, -1, 0, None, None, :]
    assert _rel(fin, last) < 1e-15
    o = oracle.chunked(x, dt, A, B, C, D, init, 4)
    assert _rel(o["y"], ref) < 1e-15


# ------------------------------------------------- P5: textbook scalar IIR filter

@pytest.mark.parametrize("a", [0.0, 0.3, 0.9, 0.999])
def test_scalar_matches_iir_filter(a):
    rng = np.random.default_rng(int(a * 1000))
    L = 200
    xs = rng.standard_normal(L)
    Bs, Cs = 0.7, -1.3
    x, dt, A, B, C, D = _scalar_problem(xs, a if a > 0 else 0.5, Bs, Cs, 0.25)
    if a == 0.0:
        A = np.array([-1e6])
    h = scipy.signal.lfilter([1.0], [1.0, -a], xs * Bs)
    ref = Cs * h + 0.25 * xs
    y, fin = oracle.seq(x, dt, A, B, C, D)
    assert _rel(y.ravel(), ref) < 1e-12
    assert abs(fin.item() - h[-1]) <= 1e-12 * max(1.0, abs(h[-1]))
    o = oracle.chunked(x, dt, A, B, C, D, None, 64)
    assert _rel(o["y"].ravel(), ref) < 1e-12


def test_scalar_closed_form_geometric():
    a, h0, L = 0.8, 1.7, 50
    x, dt, A, B, C, D = _scalar_problem([1.0] * L, a)
    y, _ = oracle.seq(x, dt, A, B, C, D, np.full((1, 1, 1, 1), h0))
    t = np.arange(L)
    ref = a ** (t + 1) * h0 + (1 - a ** (t + 1)) / (1 - a)
    assert _rel(y.ravel(), ref) < 1e-12


# ------------------------------------------------------------- P6: composition

def test_split_sequence_composes():
    rng = np.random.default_rng(21)
    x, dt, A, B, C, D, init = _random_problem(rng, 2, 40, 2, 3, 4, 1)
    y, fin = oracle.seq(x, dt, A, B, C, D, init)
    for L1 in (1, 13, 39):
        y1, f1 = oracle.seq(x[:, :L1], dt[:, :L1], A, B[:, :L1], C[:, :L1], D, init)
        y2, f2 = oracle.seq(x[:, L1:], dt[:, L1:], A, B[:, L1:], C[:, L1:], D, f1)
        assert _rel(np.concatenate([y1, y2], axis=1), y) < 1e-12
        assert _rel(f2, fin) < 1e-12


@pytest.mark.parametrize("store_bf16", [False, True])
def test_vertical_stack_equals_horizontal(store_bf16):
    rng = np.random.default_rng(31)
    layers, L = 4, 24
    x0, dt, _, B, C, _, _ = _random_problem(rng, 2, L, 3, 4, 5, 1, h0=False)
    A = -np.exp(rng.uniform(0, math.log(16), size=(layers, 3)))
    D = rng.uniform(0, 1, size=(layers, 3))
    init = rng.standard_normal((layers, 2, 3, 4, 5)) * 0.2
    ref, fref = oracle.stack_horizontal(x0, dt, A, B, C, D, init, store_bf16=store_bf16)
    for V in (1, 5, 8, 24, 30):
        out, fin = oracle.stack_vertical(x0, dt, A, B, C, D, V, init, store_bf16=store_bf16)
        # The same per-token arithmetic in the same order: equal to the last bit.
        assert np.array_equal(out, ref), V
        assert np.array_equal(fin, fref), V


def test_stack_single_layer_is_the_layer():
    rng = np.random.default_rng(41)
    x, dt, A, B, C, D, init = _random_problem(rng, 1, 17, 2, 3, 4, 1)
    out, fin = oracle.stack_horizontal(x, dt, A[None], B, C, D[None], init[None],
                                       residual=False, store_bf16=False)
    y, f = oracle.seq(x, dt, A, B, C, D, init)
    assert np.array_equal(out, y) and np.array_equal(fin[0], f)


def test_stack_state_mixups_are_detected():
    """Swapping two layers' states, or shifting a segment, changes the output: the
    equality checks above have the power to see state-management mistakes."""
    rng = np.random.default_rng(51)
    layers, L = 3, 16
    x0, dt, _, B, C, _, _ = _random_problem(rng, 1, L, 2, 3, 4, 1, h0=False)
    A = -np.exp(rng.uniform(0, math.log(16), size=(layers, 2)))
    D = rng.uniform(0, 1, size=(layers, 2))
    init = rng.standard_normal((layers, 1, 2, 3, 4))
    ref, _ = oracle.stack_horizontal(x0, dt, A, B, C, D, init, store_bf16=False)
    swapped = init[[1, 0, 2]]
    bad, _ = oracle.stack_vertical(x0, dt, A, B, C, D, 4, swapped, store_bf16=False)
    assert _rel(bad, ref) > 1e-3
    shifted = np.concatenate([x0[:, 1:], x0[:, :1]], axis=1)
    bad2, _ = oracle.stack_vertical(shifted, dt, A, B, C, D, 4, init, store_bf16=False)
    assert _rel(bad2, ref) > 1e-3


# ------------------------------------------------------ P7: linearity and causality

def test_linearity_and_causality():
    rng = np.random.default_rng(61)
    x1, dt, A, B, C, D, _ = _random_problem(rng, 1, 30, 2, 3, 4, 1, h0=False)
    x2 = rng.standard_normal(x1.shape)
    ya, _ = oracle.seq(x1, dt, A, B, C, D)
    yb, _ = oracle.seq(x2, dt, A, B, C, D)
    yc, _ = oracle.seq(2.5 * x1 - 0.75 * x2, dt, A, B, C, D)
    assert _rel(yc, 2.5 * ya - 0.75 * yb) < 1e-12
    for s in (0, 11, 29):
        xp = x1.copy()
        xp[:, s] += 1.0
        yp, _ = oracle.seq(xp, dt, A, B, C, D)
        assert np.array_equal(yp[:, :s], ya[:, :s])
        assert not np.array_equal(yp[:, s:], ya[:, s:])


# ------------------------------------------------------------ bfloat16 rounding

def test_round_bf16_matches_torch_cast():
    """For a value exact in float32, one rounding to bfloat16 from float64 must equal
    torch's float32 -> bfloat16 round-to-nearest-even."""
    rng = np.random.default_rng(71)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(2000) * 1e-39).astype(np.float32),    # subnormals
            (rng.standard_normal(2000) * 1e37).astype(np.float32)]
    # exact ties: bf16 value plus half an ulp, both parities
    base = torch.randn(4000).to(torch.bfloat16).float().numpy()
    half_ulp = np.ldexp(np.ones_like(base), np.frexp(base)[1] - 9)
    vals.append((base + half_ulp).astype(np.float32))
    vals.append(np.array([0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38, 3.4e38,
                          1.1754943508222875e-38, 9.18354961579912e-41], dtype=np.float32))
    v = np.concatenate(vals)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_decode_is_exact():
    t = torch.randn(1000).to(torch.bfloat16)
    assert np.array_equal(oracle.to_f64(t), t.float().numpy().astype(np.float64))
    f = torch.randn(1000)
    assert np.array_equal(oracle.to_f64(f), f.numpy().astype(np.float64))


# ------------------------------------------------ planted mistakes are caught (CPU)

def test_pins_catch_planted_mistakes():
    """Alternative oracles with a plausible mistake each (written here, on the CPU) fail
    the brute-force pin, which shows the pin is sensitive to them."""
    rng = np.random.default_rng(81)
    prob = _random_problem(rng, 1, 12, 2, 3, 4, 1)
    yb, _ = brute.closed_form(*prob)
    x, dt, A, B, C, D, init = prob

    def run(variant):
        y = np.zeros_like(x)
        for h in range(2):
            S = init[0, h].copy()
            for t in range(12):
                a = math.exp(dt[0, t, h] * A[h])
                if variant == "decay_after_input":
                    S = a * (S + np.outer(x[0, t, h], B[0, t, 0]))
                elif variant == "transposed_state":
                    S = a * S + np.outer(B[0, t, 0], x[0, t, h]).T.reshape(S.shape)[::-1]
                else:
                    S = a * S + np.outer(x[0, t, h], B[0, t, 0])
                y[0, t, h] = S @ C[0, t, 0] + (0.0 if variant == "no_skip" else D[h] * x[0, t, h])
        return y

    assert _rel(run("correct"), yb) < 1e-12
    for v in ("decay_after_input", "transposed_state", "no_skip"):
        assert _rel(run(v), yb) > 1e-6, v


def test_chunked_pin_catches_planted_decomposition_mistakes():
    """A Python copy of the decomposition with one plausible mistake planted at a time
    (exclusive diag(L), the wrong chunk's decay product, b(c) in place of b(c-1)) fails
    the chunked == sequential pin, while the unplanted copy passes it."""
    rng = np.random.default_rng(91)
    x, dt, A, B, C, D, init = _random_problem(rng, 1, 14, 1, 2, 3, 1)
    y_ref, _ = oracle.seq(x, dt, A, B, C, D, init)
    Q, L = 4, 14

    def run(mistake):
        a = np.exp(dt[0, :, 0] * A[0])
        y = np.zeros(x.shape)
        chunks = [(t0, min(t0 + Q, L)) for t0 in range(0, L, Q)]
        b_intra, by_intra = [], np.zeros((L, x.shape[3]))
        for t0, t1 in chunks:
            S = np.zeros(init.shape[2:])
            for t in range(t0, t1):
                S = a[t] * S + np.outer(x[0, t, 0], B[0, t, 0])
                by_intra[t] = S @ C[0, t, 0]
            b_intra.append(S)
        b_prev, b_in = init[0, 0].copy(), []
        for c, (t0, t1) in enumerate(chunks):
            lo, hi = (t0, t1) if mistake != "wrong_chunk_product" else (max(t0 - Q, 0), t0)
            nxt = b_intra[c] + np.prod(a[lo:hi]) * b_prev
            b_in.append(nxt if mistake == "b_c_not_b_cm1" else b_prev)
            b_prev = nxt
        for c, (t0, t1) in enumerate(chunks):
            for t in range(t0, t1):
                Li = np.prod(a[t0:t + 1]) if mistake != "exclusive_diagL" else np.prod(a[t0:t])
                y[0, t, 0] = by_intra[t] + Li * (b_in[c] @ C[0, t, 0]) + D[0] * x[0, t, 0]
        return y

    assert _rel(run("none"), y_ref) < 1e-12
    for m in ("exclusive_diagL", "wrong_chunk_product", "b_c_not_b_cm1"):
        assert _rel(run(m), y_ref) > 1e-6, m
