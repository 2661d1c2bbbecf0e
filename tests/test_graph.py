"""The entry points allocate nothing and never synchronise, so a caller can capture them
in a HIP graph (torch.cuda.CUDAGraph).  Each graph is replayed several times with eager
work and synchronisations in between, and every replay must equal the eager result bit
for bit (the kernels are deterministic)."""
import pytest
import torch

from chunked_linear_recurrence_amd import inputs, ssd

from helpers import to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_layer_call_in_a_graph():
    d = inputs.make_layer(2, 3 * 256 + 40, 4, 64, 128, 1, "bf16", seed=3, init="normal", init_std=0.3)
    g = to_dev(d, DEV)
    dims = ssd.dims_of(g["x"], g["B"])
    ws = ssd.alloc_workspace(ssd.workspace_bytes(dims, 256), DEV)
    y = torch.empty_like(g["x"])
    fin = torch.empty(2, 4, 64, 128, device=DEV)

    def call():
        ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], 256, y=y, final_state=fin,
                workspace=ws)
    call()
    torch.cuda.synchronize()
    y_ref, fin_ref = y.clone(), fin.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for k in range(3):
        y.fill_(float(k + 7))                      # eager work between replays
        fin.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(fin, fin_ref), k


def test_decode_steps_in_a_graph():
    T, b, H, P, N = 8, 3, 6, 64, 128
    d = inputs.make_layer(b, T, H, P, N, 2, "bf16", seed=5, init="normal", init_std=0.5)
    g = to_dev(d, DEV)
    toks = [(g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["B"][:, t].contiguous(),
             g["C"][:, t].contiguous()) for t in range(T)]
    ys = [torch.empty_like(toks[0][0]) for _ in range(T)]
    state = g["init_state"].clone()

    def steps():
        for t in range(T):
            x, dt, B, C = toks[t]
            ssd.step(x, dt, g["A"], B, C, g["D"], state, y=ys[t])
    steps()
    torch.cuda.synchronize()
    y_ref = [y.clone() for y in ys]
    s_ref = state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        state.copy_(g["init_state"])
        steps()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    for k in range(3):
        state.copy_(g["init_state"])               # eager work: reset the carried state
        for y in ys:
            y.fill_(float(k))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, s_ref), k
        for t in range(T):
            assert torch.equal(ys[t], y_ref[t]), (k, t)
