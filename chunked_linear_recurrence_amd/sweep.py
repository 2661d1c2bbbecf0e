"""Chunk length Q and vertical segment length V on one GPU: the tuning study of
[分块推理 §4.1-§4.3] of the page "分块推理：解锁循环模型并行计算，实现长序列高效处理",
rerun on this hardware with synthetic layers.

    python -m chunked_linear_recurrence_amd.sweep [--quick]

prints markdown tables:
  Q   tokens/s of one layer at the 128K-token shape for chunk_Q in {32, 64, 128, 256},
      with each kernel's time (its stage run on its own) and the launches per step;
  V   layer-tokens/s and memory of a 24-layer stack (batch 1, 32768 tokens; and batch 4,
      8192 tokens) for V from Q up to 8192, in both schedules of ssd_chunk_scan_segmented,
      next to the horizontal order; with the page's rule of thumb (stop doubling V once
      the gain is under 5%) applied to the wavefront schedule.
Memory is torch's peak allocation above what the inputs hold: the library allocates
nothing itself, so this is the workspace and activation buffers each schedule needs.
Every number is a HIP-event time on the current stream after an untimed settle phase.
"""
import argparse
import sys

import torch

from . import inputs, ssd, WORKLOADS


def _time(fn, reps, settle=5):
    for _ in range(settle):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def q_sweep(dev, reps):
    w = WORKLOADS["long_context_b1_L131072_h48"]
    d = inputs.make(w)
    g = {k: (v.to(dev) if v is not None else None) for k, v in d.items()}
    rows = []
    for Q in (32, 64, 128, 256):
        dims = ssd.dims_of(g["x"], g["B"])
        if not ssd.shape_supported(dims.dtype, Q, w.headdim, w.dstate):
            rows.append((Q, None, None, None))
            continue
        ws = ssd.alloc_workspace(ssd.workspace_bytes(dims, Q), dev)
        y = torch.empty_like(g["x"])
        fin = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, device=dev)

        def f(first=1, last=ssd.NSTAGES):
            ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], None, Q, y=y, final_state=fin, workspace=ws,
                    first_stage=first, last_stage=last)
        ms = _time(f, reps, settle=30)
        stages = [_time(lambda k=k: f(k, k), reps, settle=3) for k in range(1, ssd.NSTAGES + 1)]
        rows.append((Q, ms, ws.numel(), stages))
        del ws
    return w, rows


def v_sweep(dev, batch, seqlen, reps, Vs):
    base = WORKLOADS["vertical_stack_24x_L32768_V2048"]
    d = inputs.make_stack(batch, seqlen, base.nheads, base.headdim, base.dstate, base.ngroups, base.layers,
                          base.dtype, seed=0)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    nl = base.layers
    dims = ssd.dims_of(g["x0"], g["B"])
    states = torch.zeros(nl, batch, base.nheads, base.headdim, base.dstate, device=dev)
    y = torch.empty_like(g["x0"])
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()

    def measure(fn):
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        ms = _time(fn, reps)
        return ms, torch.cuda.max_memory_allocated() - base_mem

    def hor():
        states.zero_()
        ssd.horizontal(g["x0"], g["dt"], g["A"], g["B"], g["C"], g["D"], states, base.chunk)
    h_ms, h_mem = measure(hor)
    rows = []
    for V in Vs:
        if V > seqlen:
            continue
        r = {"V": V}
        for wf in (True, False):
            ws = ssd.alloc_workspace(ssd.segmented_workspace_bytes(dims, base.chunk, V, nl, wf), dev)

            def seg():
                states.zero_()
                ssd.segmented(g["x0"], g["dt"], g["A"], g["B"], g["C"], g["D"], states, V, base.chunk, y=y,
                              wavefront=wf, workspace=ws)
            ms, mem = measure(seg)
            r["wf" if wf else "one"] = (ms, mem)
            del ws
        rows.append(r)
    return (batch, seqlen, nl, base.chunk), (h_ms, h_mem), rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true", help="fewer repetitions")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    reps = 3 if args.quick else 10
    ssd.lib()

    w, rows = q_sweep(dev, reps)
    print("## Chunk length Q: one layer, %s (batch %d, L %d, H %d, P %d, N %d, %s)\n"
          % (w.name, w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.dtype))
    print("| Q | chunks | ms per layer | M tokens/s | workspace MB | chunk_cumsum us | chunk_state us | "
          "state_pass us | chunk_scan us |")
    print("|---|---|---|---|---|---|---|---|---|")
    for Q, ms, wsb, stages in rows:
        if ms is None:
            print("| %d | | not compiled | | | | | | |" % Q)
        else:
            print("| %d | %d | %.3f | %.1f | %.0f | %s |" % (
                Q, -(-w.seqlen // Q), ms, w.tokens / ms / 1e3, wsb / 1e6,
                " | ".join("%.1f" % (t * 1e3) for t in stages)))
    print("\nEvery Q runs the same 4 launches per layer; smaller Q means more chunks, so more "
          "per-chunk state traffic (it scales with 1/Q) and a longer serial state pass.", flush=True)

    for batch, seqlen in ((1, 32768), (4, 8192)):
        Vs = [256 * 2 ** k for k in range(6)]              # Q .. 8192
        (b, L, nl, Q), (h_ms, h_mem), vrows = v_sweep(dev, batch, seqlen, reps, Vs)
        lt = nl * b * L
        print("## Segment length V: %d-layer stack, batch %d, L %d, H 24, P 64, N 128, Q %d, bf16\n"
              % (nl, b, L, Q))
        print("Horizontal order (one full-sequence call per layer): %.3f ms, %.1f M layer-tokens/s, "
              "%.0f MB above the inputs.\n" % (h_ms, lt / h_ms / 1e3, h_mem / 1e6))
        print("| V | wavefront ms | wavefront M layer-tok/s | wavefront MB | one-at-a-time ms | "
              "one-at-a-time M layer-tok/s | one-at-a-time MB |")
        print("|---|---|---|---|---|---|---|")
        for r in vrows:
            (wms, wmem), (oms, omem) = r["wf"], r["one"]
            print("| %d | %.3f | %.1f | %.0f | %.3f | %.1f | %.0f |"
                  % (r["V"], wms, lt / wms / 1e3, wmem / 1e6, oms, lt / oms / 1e3, omem / 1e6))
        # the page's rule: keep doubling V while the wavefront throughput rises by >= 5%
        best = vrows[0]
        for r in vrows[1:]:
            if best["wf"][0] / r["wf"][0] >= 1.05:
                best = r
            else:
                break
        best = best["V"]
        print("\nRule of [分块推理 §4.3] (double V while throughput rises by at least 5%%): V = %d.\n" % best,
              flush=True)


if __name__ == "__main__":
    main()
