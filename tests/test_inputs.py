"""The seeded input generators: shapes, dtypes, determinism and value ranges (CPU)."""
import math

import numpy as np
import torch

from chunked_linear_recurrence_amd import inputs, WORKLOADS


def test_layer_inputs_shapes_dtypes_and_determinism():
    w = WORKLOADS["mamba2_130m_layer_b2_L2048"]
    a, b = inputs.make(w), inputs.make(w)
    assert a["x"].shape == (2, 2048, 24, 64) and a["x"].dtype == torch.bfloat16
    assert a["dt"].shape == (2, 2048, 24) and a["B"].shape == (2, 2048, 1, 128)
    assert a["A"].dtype == torch.float32 and a["D"].shape == (24,)
    assert a["init_state"] is None
    for k in ("x", "dt", "A", "B", "C", "D"):
        assert torch.equal(a[k], b[k]), k
    c = inputs.make(w, seed=1)
    assert not torch.equal(a["x"], c["x"])


def test_value_ranges():
    w = WORKLOADS["tiny_fp32_L256"]
    d = inputs.make(w)
    dt, A, D = d["dt"].numpy(), d["A"].numpy(), d["D"].numpy()
    assert dt.min() >= 1e-3 and dt.max() <= 0.1
    # softplus(N(-2, 0.5)) exceeds 0.1 about 2/3 of the time: many values sit on the clamp
    assert 0.4 < np.mean(dt == np.float32(0.1)) < 0.9
    assert (A <= -1.0).all() and (A >= -16.0).all()
    assert (D >= 0).all() and (D < 1).all()
    assert abs(d["B"].numpy().std() * math.sqrt(16) - 1) < 0.1


def test_random_init_state_and_narrow_dt():
    d = inputs.make_layer(2, 64, 3, 8, 16, 1, "bf16", seed=0, init="normal", init_std=0.1)
    assert d["init_state"].shape == (2, 3, 8, 16) and d["init_state"].dtype == torch.float32
    assert 0.08 < d["init_state"].std().item() < 0.12
    d2 = inputs.make_layer(1, 4096, 2, 8, 16, 1, "bf16", dt_min=1e-3, dt_max=1e-2)
    dt = d2["dt"].float().numpy()
    assert dt.min() >= 1e-3 - 1e-6 and dt.max() <= 1e-2 + 1e-5
    d3 = inputs.make_layer(1, 4096, 2, 8, 16, 1, "f32", dt_min=1e-3, dt_max=1e-2,
                           dt_dist="loguniform")
    lg = np.log10(d3["dt"].numpy())
    assert lg.min() >= -3 - 1e-6 and lg.max() <= -2 + 1e-6 and 0.2 < lg.std() < 0.4


def test_stack_inputs():
    d = inputs.make_stack(1, 128, 4, 8, 16, 1, layers=3, dtype="bf16")
    assert d["x0"].shape == (1, 128, 4, 8) and d["A"].shape == (3, 4) and d["D"].shape == (3, 4)
    assert not torch.equal(d["A"][0], d["A"][1])
