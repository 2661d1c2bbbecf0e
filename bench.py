"""Throughput of the chunked SSD scan on one MI355X, as one JSON line.

A step is one ssd_chunk_scan_fwd call (all four kernels: chunk_cumsum, chunk_state,
state_pass, chunk_scan) over the whole batch of the 128K-token workload
(long_context_b1_L131072_h48: batch 1, L 131072, H 48, P 64, N 128, Q 256, bf16), with
every input already resident in HBM.  Untimed: steps repeated for --settle-ms (clock
ramp-up), then W warm-up steps; then exactly K timed steps between two device
synchronisations.

Besides the headline tokens/s the line carries:
  roofline      the dominant kernel's achieved HBM rate (algorithmic bytes per launch /
                its mean duration, from HIP events around each launch on the stream it
                runs on, inside full steps) against the 8 TB/s peak;
  kernels       the same figures for all four kernels, plus matrix-core rates;
  end_to_end    the method's bytes / step time against peak HBM bandwidth, with the
                bytes per stored per-chunk state element (state_bytes) and the same rate
                on the compulsory bytes alone;
  workloads     one step of the smaller bf16 workloads (cache evicted before each);
  scan_form     the chunk outputs computed by the associative-scan kernel instead of the
                matrix-core one (same layer), for comparison;
  decode        the decode step (ssd_step) at the same layer shape, batch 1 and 8;
  stack         the 24-layer vertical stack (segmented entry point, wavefront and one
                step at a time, and the horizontal order), a secondary figure;
  cpu_baseline  the fp64 CPU oracle timed on this host's cores on the same inputs.

Algorithmic bytes count every input a kernel reads once and every output it writes once,
in the dtype the library stores it in (activations and the per-chunk states b_intra and
b_in in the activation dtype; decay sums, the per-token decay arrays, init and final states
float32).  The end-to-end figure uses the method's own bytes instead (the compulsory I/O
plus the per-chunk state exchange), which leave out the library's decay intermediates.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix cores, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed: repeat the step for this long before the warm-up steps, so the "
                         "timed steps start at steady clocks (the per-step time falls by about 20%% over "
                         "the first ~20 ms of load); 0 disables")
    ap.add_argument("--workload", default=None, help="workload name (default: the 128K-token layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the secondary timing of the 24-layer vertical stack")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the secondary timing of the decode step")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the secondary timing of the smaller bf16 workloads")
    ap.add_argument("--no-scan-form", action="store_true",
                    help="skip the secondary timing of the associative-scan form of the chunk outputs")
    ap.add_argument("--kernel-steps", type=int, default=0, help="launches per kernel for per-kernel timing "
                    "(default: --steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--stack-only", action="store_true",
                    help="time only the 24-layer vertical stack in the wavefront schedule and print its "
                         "object (for kernel traces of that schedule); not the benchmark line")
    return ap.parse_args()


def alg_bytes(w):
    """Bytes each kernel must move once per launch (every input it reads and every output
    it writes, once, in the dtype the library stores it); the method's bytes: the
    compulsory activations and states plus the per-chunk state exchange (b_intra and b_in
    each written and read once, in the activation dtype); and the compulsory bytes alone
    (x, y, dt, B, C, and the initial and final states)."""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    e = w.act_bytes
    nc = w.nchunks
    cum_e = 8 if w.dtype == "f32" else 4
    x = b * L * H * P * e
    y = x
    dt = b * L * H * e
    bc = b * L * G * N * e                      # one of B or C
    cum = b * H * nc * Q * cum_e                # dA_cum
    dec = b * H * nc * Q * 4                    # one per-token decay array (block end or chunk end)
    ctot = b * H * nc * cum_e                   # chunk totals
    states = b * nc * H * P * N
    init = final = b * H * P * N * 4
    k = {
        "chunk_cumsum": dt + cum + 2 * dec + ctot,
        "chunk_state": x + bc + dec + states * e,
        "state_pass": 2 * states * e + ctot + final + (init if w.init != "zero" else 0),
        "chunk_scan": x + 2 * bc + cum + dec + states * e + y,
    }
    compulsory = x + y + dt + 2 * bc + (init if w.init != "zero" else 0) + final
    method = compulsory + 4 * states * e
    return k, method, compulsory


def alg_flops(w):
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = w.nchunks
    per_chunk_state = H * 2 * Q * N * P
    per_chunk_scan = H * (Q * (Q + 1) * P + 2 * Q * N * P)
    per_chunk_cb = G * Q * (Q + 1) * N          # causal C.B^T, once per chunk and group
    return {"chunk_state": b * nc * per_chunk_state, "chunk_scan": b * nc * (per_chunk_scan + per_chunk_cb)}


def kernel_sources_sha256():
    """sha256 over the HIP sources of the library (file names and contents, sorted)."""
    import hashlib
    csrc = os.path.join(ROOT, "chunked_linear_recurrence_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary (scaled by its copy calibration), or None when there is none for this workload
    or the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != kernel_sources_sha256() or kernel not in t.get("kernels", {}):
        return None
    return t["kernels"][kernel]["bytes"]


def stack_timing(torch, dev, reps=5, schedules=("wavefront", "one_at_a_time", "horizontal")):
    """The 24-layer vertical stack (32768 tokens, V = 2048): the segmented entry point in
    the wavefront schedule and one step at a time, and the horizontal order (one
    ssd_chunk_scan_fwd per layer) for reference; HIP events around `reps` whole stacks."""
    from chunked_linear_recurrence_amd import inputs, ssd, WORKLOADS
    w = WORKLOADS["vertical_stack_24x_L32768_V2048"]
    d = inputs.make(w)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    stream = torch.cuda.current_stream()
    dims = ssd.dims_of(g["x0"], g["B"])
    y = torch.empty_like(g["x0"])
    states = torch.zeros(w.layers, w.batch, w.nheads, w.headdim, w.dstate, device=dev)
    ws = {wf: ssd.alloc_workspace(ssd.segmented_workspace_bytes(dims, w.chunk, w.segment, w.layers, wf), dev)
          for wf in (True, False)}

    def seg(wf):
        states.zero_()
        ssd.segmented(g["x0"], g["dt"], g["A"], g["B"], g["C"], g["D"], states, w.segment, w.chunk, y=y,
                      wavefront=wf, workspace=ws[wf], stream=stream)

    def hor():
        states.zero_()
        ssd.horizontal(g["x0"], g["dt"], g["A"], g["B"], g["C"], g["D"], states, w.chunk, stream=stream)

    out = {"workload": w.name, "layers": w.layers, "tokens": w.tokens, "V": w.segment}
    for name, f in (("wavefront", lambda: seg(True)), ("one_at_a_time", lambda: seg(False)),
                    ("horizontal", hor)):
        if name not in schedules:
            continue
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out["ms_" + name] = round(ms, 3)
        out["layer_tokens_per_s_" + name] = round(w.layers * w.tokens / (ms * 1e-3), 1)
    return out


def decode_timing(torch, dev, steps=200):
    """ssd_step at the 128K-token layer's shape (H 48, P 64, N 128, bf16) at batch 1 and 8:
    HIP events around `steps` consecutive steps on the same state.  A step must read and
    write the fp32 state once (its HBM roofline); the rest of its traffic is a few KB."""
    from chunked_linear_recurrence_amd import inputs, ssd
    out = []
    for b in (1, 8):
        d = inputs.make_layer(b, steps, 48, 64, 128, 1, "bf16", seed=b, init="normal", init_std=0.5,
                              dt_max=1e-2)
        g = {k: v.to(dev) for k, v in d.items()}
        toks = [(g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["B"][:, t].contiguous(),
                 g["C"][:, t].contiguous()) for t in range(steps)]
        state = g["init_state"].clone()
        y = torch.empty_like(toks[0][0])
        stream = torch.cuda.current_stream()
        for t in range(10):
            ssd.step(*toks[t][:2], g["A"], *toks[t][2:], g["D"], state, y=y, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(steps):
            x, dt, B, C = toks[t]
            ssd.step(x, dt, g["A"], B, C, g["D"], state, y=y, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        # the same steps captured once in a HIP graph and replayed (launch cost amortised)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for t in range(steps):
                x, dt, B, C = toks[t]
                ssd.step(x, dt, g["A"], B, C, g["D"], state, y=y)
        stream.wait_stream(side)
        with torch.cuda.graph(graph):
            for t in range(steps):
                x, dt, B, C = toks[t]
                ssd.step(x, dt, g["A"], B, C, g["D"], state, y=y)
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) / steps * 1e3
        sbytes = 2 * state.numel() * 4
        out.append({"batch": b, "nheads": 48, "headdim": 64, "dstate": 128, "us_per_step": round(us, 2),
                    "us_per_step_graph": round(us_graph, 2),
                    "tokens_per_s": round(b / (us * 1e-6), 1), "state_bytes_per_step": sbytes,
                    "state_GB_s": round(sbytes / (us * 1e-6) / 1e9, 1)})
    return out


def workload_timing(torch, dev, reps=10):
    """One step of each smaller bf16 workload (the Mamba-2-130M layer, the batch-8
    throughput layer).  Their data fits the 256 MB last-level cache, so a 1 GiB buffer is
    written before every timed step (outside the HIP events around it): the step then
    reads its inputs from HBM, as the large workload does."""
    from chunked_linear_recurrence_amd import inputs, ssd, WORKLOADS
    evict = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("mamba2_130m_layer_b2_L2048", "throughput_b8_L4096_h32"):
        w = WORKLOADS[name]
        d = inputs.make(w)
        g = {k: (v.to(dev) if v is not None else None) for k, v in d.items()}
        dims = ssd.dims_of(g["x"], g["B"])
        ws = ssd.alloc_workspace(ssd.workspace_bytes(dims, w.chunk), dev)
        y = torch.empty_like(g["x"])
        fin = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, device=dev)

        def step():
            ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], w.chunk, y=y,
                    final_state=fin, workspace=ws, stream=stream)
        for _ in range(5):
            step()
        times = []
        for _ in range(reps):
            evict.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        out[name] = {"ms_per_step_median": round(ms, 4), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1)}
    del evict
    return out


def cpu_baseline(d, w):
    """The fp64 oracle (plain C, one thread per (batch, head) pair) on this host."""
    import numpy as np
    import oracle
    x, dt, A, B, C, D = (oracle.to_f64(d[k]) for k in ("x", "dt", "A", "B", "C", "D"))
    init = None if d.get("init_state") is None else oracle.to_f64(d["init_state"])
    threads = min(oracle.default_threads(), w.batch * w.nheads)
    times = []
    for _ in range(3):                         # the whole workload takes a few seconds: median of 3
        t0 = time.perf_counter()
        oracle.seq(x, dt, A, B, C, D, init, nthreads=threads)
        times.append(time.perf_counter() - t0)
    dt_s = sorted(times)[1]
    del x
    return {"value": w.tokens / dt_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt_s, 3),
            "sample": "the whole workload (%d x %d tokens, %d heads), fp64 sequential recurrence, "
                      "one thread per (batch, head) pair; median of 3 runs" % (w.batch, w.seqlen, w.nheads)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this library is a single-GPU kernel set; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from chunked_linear_recurrence_amd import inputs, ssd, WORKLOADS, BENCH_WORKLOAD

    if args.stack_only:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        ssd.lib()
        print(json.dumps({"stack": stack_timing(torch, dev, schedules=("wavefront",))}), flush=True)
        return

    w = WORKLOADS[args.workload or BENCH_WORKLOAD]
    if w.layers > 1:
        print("bench.py times single-layer workloads", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ssd.lib()
    print("[bench] generating %s" % w.name, file=sys.stderr, flush=True)
    d = inputs.make(w)
    g = {k: (v.to(dev) if v is not None else None) for k, v in d.items()}
    dims = ssd.dims_of(g["x"], g["B"])
    ws = ssd.alloc_workspace(ssd.workspace_bytes(dims, w.chunk), dev)
    y = torch.empty_like(g["x"])
    fin = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(first=1, last=ssd.NSTAGES):
        ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], w.chunk, y=y,
                final_state=fin, workspace=ws, stream=stream, first_stage=first, last_stage=last)

    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = w.tokens / (ms_step * 1e-3)

    # per-kernel durations: full steps again, the four stages launched one by one in order
    # on the same stream with a HIP event between consecutive kernels, so each kernel is
    # timed where it runs inside a step (after its producer, before its consumer).
    names = ["chunk_cumsum", "chunk_state", "state_pass", "chunk_scan"]
    kb, method_bytes, compulsory_bytes = alg_bytes(w)
    kf = alg_flops(w)
    ksteps = args.kernel_steps or args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(ksteps)]
    for row in evs:
        row[0].record(stream)
        for stage in range(1, len(names) + 1):
            step(stage, stage)
            row[stage].record(stream)
    torch.cuda.synchronize()
    kernels = {}
    for k, name in enumerate(names):
        us = sum(row[k].elapsed_time(row[k + 1]) for row in evs) / ksteps * 1e3
        gbs = kb[name] / (us * 1e-6) / 1e9
        rec = {"us": round(us, 2), "alg_bytes": kb[name], "GB_s": round(gbs, 1),
               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if name in kf:
            tf = kf[name] / (us * 1e-6) / 1e12
            rec.update({"alg_flops": kf[name], "TFLOP_s": round(tf, 2),
                        "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        kernels[name] = rec
    staged_ms = sum(row[0].elapsed_time(row[-1]) for row in evs) / ksteps
    torch.cuda.synchronize()
    dom = max(names, key=lambda n: kernels[n]["us"])
    roof = {"kernel": dom, "bound": "hbm", "achieved": kernels[dom]["GB_s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kernels[dom]["hbm_frac"], "traffic": measured_traffic(w.name, dom),
            "alg_bytes_per_launch": kb[dom], "mean_launch_us": kernels[dom]["us"]}
    e2e_gbs = method_bytes / (ms_step * 1e-3) / 1e9
    comp_gbs = compulsory_bytes / (ms_step * 1e-3) / 1e9

    out = {
        "metric": "SSD chunked-scan tokens/s per GPU; % of bf16 MFMA peak and % of HBM BW",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups, "chunk": w.chunk},
        "roofline": roof,
        "end_to_end": {"method_bytes": method_bytes, "state_bytes": w.act_bytes,
                       "GB_s": round(e2e_gbs, 1), "hbm_frac": round(e2e_gbs / HBM_PEAK_GBS, 4),
                       "compulsory_bytes": compulsory_bytes,
                       "compulsory_GB_s": round(comp_gbs, 1),
                       "compulsory_hbm_frac": round(comp_gbs / HBM_PEAK_GBS, 4)},
        "kernels": kernels,
        "ms_per_step_staged": round(staged_ms, 4),
        "wall_s_timed": round(wall, 4),
    }
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
    if not args.no_workloads:
        print("[bench] smaller workloads", file=sys.stderr, flush=True)
        out["workloads"] = workload_timing(torch, dev)
    if not args.no_scan_form:
        print("[bench] scan form", file=sys.stderr, flush=True)
        sf = {"workload": w.name, "stage": "chunk outputs (stage 4)"}
        for name, scan_form in (("matrix_core", False), ("scan_form", True)):
            step()
            torch.cuda.synchronize()
            reps = 3 if scan_form else 10
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                ssd.fwd(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["init_state"], w.chunk, y=y,
                        final_state=fin, workspace=ws, stream=stream, first_stage=ssd.NSTAGES,
                        last_stage=ssd.NSTAGES, scan_form=scan_form)
            e1.record(stream)
            torch.cuda.synchronize()
            sf["us_" + name] = round(e0.elapsed_time(e1) / reps * 1e3, 1)
        sf["ratio"] = round(sf["us_scan_form"] / sf["us_matrix_core"], 1)
        out["scan_form"] = sf
    if not args.no_decode:
        print("[bench] decode step", file=sys.stderr, flush=True)
        out["decode"] = decode_timing(torch, dev)
    if not args.no_stack:
        print("[bench] vertical stack", file=sys.stderr, flush=True)
        out["stack"] = stack_timing(torch, dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
