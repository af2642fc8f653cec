"""Benchmark: forward + backward training step of the leaky-tanh recurrence at
the FlyGPT launch shape (N=5,000 nodes, E=524,324 edges, B=32, T=64 input
steps x 2 microsteps, fp32) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-graph] [--no-cpu]

One step = ck_recurrence_forward + ck_recurrence_backward over the whole
window on one HIP stream; inputs, graph and buffers are resident in HBM
before timing starts (graph construction and input generation are excluded).
By default the step's launches are captured once into a HIP graph (through
torch.cuda.CUDAGraph on the stream the library launches on) and the graph is
replayed; --no-graph launches them directly.
Prints one JSON line with:
  value        edge-visits/s = S * E * B / t_step  (S = T * M microsteps)
  ms_per_step  mean time of one step over the K timed steps (HIP events);
               ms_per_step_median / ms_per_step_min from an event pair
               around each of the K steps
  roofline     the dominant kernel's algorithmic bytes per launch / its mean
               launch duration (HIP events around each launch, recorded by the
               library's measurement hook on the stream the kernels run on)
               against the MI355X HBM peak of 8 TB/s
               (achieved); with the committed rocprofv3 counter summary of
               that kernel, also its measured HBM bytes per launch (traffic)
               over the same duration (measured_GBps, measured_frac)
  cpu_baseline the CPU oracle's rate on the same workload (host cores), the
               host CPU model, and one-thread oracle times of whole
               forward+backward windows of the tiny, edge-case and FlyGPT
               workloads
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "ms per fwd+bwd step & edge-visits/s, N=5k E=524k B=32 T×M=64×2; HBM GB/s"


def algorithmic_bytes(N, E, n_in, B, T, M):
    """Byte yardstick of the method's kernel structure: each pass reads its
    operands once and writes its results once (gathers beyond the first read
    of a row count as cache hits).  Returns per-microstep forward and backward
    bytes and the per-step total."""
    NB = N * B
    fwd = 8 * E + 4 * (N + 1) + 12 * N + 4 * n_in * B + 12 * NB
    k1 = 16 * NB + 24 * N + 8 * n_in * B               # elementwise + leak/bias reductions
    k2 = 8 * E + 4 * (N + 1) + 4 * N + 12 * NB         # transposed product
    k3 = 12 * E + 4 * (N + 1) + 8 * NB                 # edge dot product (gv read-modify-write)
    bwd = k1 + k2 + k3
    once = 8 * T * NB + 36 * E + 16 * NB               # out/G, value permutations + scatter, state0
    S = T * M
    return fwd, bwd, S * (fwd + bwd) + once


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "flygpt_traffic.md")
LIF_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "lif_traffic.md")
CSRC = os.path.join(ROOT, "sparse_graph_recurrent_amd", "csrc")


def kernel_source(kernel: str) -> str:
    if kernel.startswith("blk_"):
        return os.path.join(CSRC, "blocked.hip")
    if kernel.startswith("lif_"):
        return os.path.join(CSRC, "lif.hip")
    return os.path.join(CSRC, "resident.hip" if kernel.startswith("res_") else "recurrence.hip")


def measured_traffic(kernel: str, profile: str = TRAFFIC_PROFILE):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    import hashlib
    try:
        with open(profile) as f:
            text = f.read()
        with open(kernel_source(kernel), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get(f"{kernel}_source_sha256", fields.get("source_sha256")) != digest:
        return None
    v = fields.get(f"{kernel}_bytes_per_launch")
    return int(v) if v else None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def one_thread_times():
    """Seconds of one whole forward+backward window of the oracle on one
    thread, for the tiny, edge-case and FlyGPT workloads."""
    import oracle
    import synthetic
    res = {}
    for name in ("tiny", "edge_cases", "flygpt"):
        w = synthetic.make(name)
        t0 = time.perf_counter()
        oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                   w.drives, w.state0, w.microsteps, grad_out=w.grad_out, nthreads=1)
        res[name] = round(time.perf_counter() - t0, 4)
    return res


def cpu_baseline(w, budget_s: float = 12.0):
    """The CPU oracle (fp64, OpenMP over all host cores) on the same workload:
    whole forward+backward windows, repeated until at least budget_s seconds
    of CPU work have been timed (a bounded sample of the benchmark)."""
    import oracle
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    S, E, B = w.T * w.microsteps, w.num_edges, w.B
    runs, total = 0, 0.0
    while runs == 0 or (total < budget_s and runs < 200):
        t0 = time.perf_counter()
        oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                   w.drives, w.state0, w.microsteps, grad_out=w.grad_out, nthreads=threads)
        total += time.perf_counter() - t0
        runs += 1
    per = total / runs
    return {"value": S * E * B / per, "unit": "edge-visits/s", "cores": threads, "kind": "oracle",
            "sample": f"{runs} full forward+backward window(s) of the benchmark workload "
                      f"(all {B} batch columns, {S} microsteps), fp64, {per:.2f} s each, "
                      f"{total:.1f} s in all",
            "ms_per_step": 1e3 * per, "cpu_model": cpu_model(),
            "one_thread_s_per_window": one_thread_times()}


# The active LIF run: threshold 40, reset 0, decay_shifts [2], refractory 2
# (the soup-connectome page's standard parameters with a threshold low enough
# for sustained activity), initial potentials uniform in [0, 60), delays 1..4.
LIF_RUN = dict(T=16, threshold=40, reset=0, refractory_steps=2, decay_shifts=[2])


def lif_bench(args, torch, sgr, synthetic, np):
    """One LIF forward = T timesteps on the synthetic whole-connectome graph.
    value = edge-visits/s = E * T / t_forward (the forward packs the synapses
    every call; ms_per_prepared_run times ck_lif_run alone on synapses packed
    once by ck_lif_prepare); roofline of the per-step gather
    kernel against HBM: algorithmic bytes per launch, over its mean launch
    time = on the LDS-lookup path 8 E (the 8-byte record of every CSR position,
    its row inside) + 8 N (the 64-bit accumulators written) + the R = 4 bit
    rows of ceil(N / 32) words the delays reach; on the byte-lookup path 12 E
    (record and 4-byte destination) + 8 N + one byte row of N."""
    w = synthetic.make_lif("connectome", max_delay=4, v0_range=(0, 60))
    N, E, T = w.num_nodes, w.src.size, LIF_RUN["T"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g = sgr.SparseGraph(dev(w.src), dev(w.dst), N, dev(w.input_nodes))
    imp, dl, v0 = dev(w.impulses), dev(w.delays), dev(w.v0)
    kw = {k: v for k, v in LIF_RUN.items() if k != "T"}
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    import ctypes
    wb = ctypes.c_size_t()
    sgr.lib().ck_lif_workspace_size(g.handle, ctypes.byref(wb))
    ws = torch.empty(wb.value, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        sgr.lif_forward(g, imp, dl, v0, T, workspace=ws, **kw)
    times = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        spikes, _ = sgr.lif_forward(g, imp, dl, v0, T, workspace=ws, **kw)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sum(times) / len(times)
    # runs on synapses prepared once (ck_lif_prepare outside the timed region)
    sgr.lif_prepare(g, imp, dl, workspace=ws)
    for _ in range(args.warmup):
        sgr.lif_run(g, ws, v0, T, **kw)
    run_times = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sgr.lif_run(g, ws, v0, T, **kw)
        e1.record()
        torch.cuda.synchronize()
        run_times.append(e0.elapsed_time(e1))
    ms_run = sum(run_times) / len(run_times)
    sgr.profile_collect_lif()
    sgr.profile_enable(True)
    for _ in range(args.steps):
        sgr.lif_forward(g, imp, dl, v0, T, workspace=ws, **kw)
    sgr.profile_enable(False)
    prof = sgr.profile_collect_lif()
    gather_us = 1e3 * prof["gather_ms"] / max(1, prof["gather_launches"])
    update_us = 1e3 * prof["update_ms"] / max(1, prof["update_launches"])
    maxd = int(w.delays.max())
    row_words = ((N + 31) // 32 + 3) // 4 * 4
    lds_path = maxd <= 16 and maxd * row_words * 4 <= 128 * 1024 and os.environ.get("CK_LIF_LDS") != "0"
    per_launch = (8 * E + 8 * N + maxd * row_words * 4) if lds_path else (12 * E + 9 * N)
    ach = per_launch / (gather_us * 1e-6) / 1e9
    gname = "lif_gather_lds" if lds_path else "lif_gather"
    tr = measured_traffic(gname, LIF_TRAFFIC_PROFILE)
    m = None if tr is None else tr / (gather_us * 1e-6) / 1e9
    res = {"metric": "LIF forward: ms per timestep & edge-visits/s, synthetic whole-connectome "
                     "graph N=211,577 E=24,678,466; HBM GB/s",
           "value": E * T / (ms * 1e-3), "unit": "edge-visits/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_forward": ms,
           "ms_per_timestep": ms / T, "ms_per_forward_min": min(times),
           "ms_per_prepared_run": ms_run, "ms_per_prepared_run_min": min(run_times),
           "prepared_run_edge_visits_per_s": E * T / (ms_run * 1e-3),
           "higher_is_better": True, "vs_baseline": None, "dtype": "int32/int16",
           "data": "synthetic",
           "config": {"workload": f"lif connectome: N={N} E={E} T={T} delays 1..4 "
                                  f"threshold {kw['threshold']} decay_shifts {kw['decay_shifts']} "
                                  f"refractory {kw['refractory_steps']}",
                      "spikes_per_step": spikes.sum(dim=1).tolist()},
           "kernels": {"gather_launch_us": gather_us, "update_launch_us": update_us,
                       "gather_launches_per_forward": prof["gather_launches"] // args.steps,
                       "update_launches_per_forward": prof["update_launches"] // args.steps},
           "roofline": {"bound": "hbm", "kernel": gname, "achieved": ach,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                        "traffic": tr, "measured_GBps": m,
                        "measured_frac": None if m is None else m / HBM_PEAK_GBS}}
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        oracle.lif_run(w.src, w.dst, N, w.impulses, w.delays, w.v0, T, **kw)
        sec = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": E * T / sec, "unit": "edge-visits/s", "cores": 1,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"one whole {T}-step run of the same workload, "
                                         f"{sec:.2f} s (the LIF oracle is single-threaded)"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step directly instead of replaying a captured HIP graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--workload", default="flygpt")
    ap.add_argument("--lif", action="store_true",
                    help="measure the fixed-point LIF forward instead (active run on the "
                         "synthetic whole-connectome graph, 16 timesteps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's plain device copy of MIB MiB three times (the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--read-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's sum over MIB MiB three times (a kernel that "
                         "reads MIB MiB and writes almost nothing)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the recurrence would "
              f"shard over the batch across GPUs, which is not implemented here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_graph_recurrent_amd as sgr
    import synthetic

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}), flush=True)
        return
    if args.read_calibration:
        n = args.read_calibration * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        for _ in range(3):
            t = x.sum()
        torch.cuda.synchronize()
        print(json.dumps({"read_calibration_bytes": n * 4, "sum": float(t)}), flush=True)
        return
    if args.lif:
        print(json.dumps(lif_bench(args, torch, sgr, synthetic, np)), flush=True)
        return
    w = synthetic.make(args.workload)
    N, E, n_in, B, T, M = w.num_nodes, w.num_edges, w.n_in, w.B, w.T, w.microsteps
    S = T * M
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    graph = sgr.SparseGraph(dev(w.src), dev(w.dst), N, dev(w.input_nodes))
    ev, lk, bs, dr, st, G = (dev(x) for x in (w.edge_values, w.leak, w.bias, w.drives, w.state0,
                                               w.grad_out))
    sb, wb = sgr.recurrence_sizes(graph, T, B, M)
    path = sgr.recurrence_path(graph, B)
    out = torch.empty((T, B, N), dtype=torch.float32, device="cuda")
    saved = torch.empty(sb, dtype=torch.uint8, device="cuda")
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    f = dict(dtype=torch.float32, device="cuda")
    grads = {"g_edge_values": torch.empty(E, **f), "g_leak": torch.empty(N, **f),
             "g_bias": torch.empty(N, **f), "g_drives": torch.empty((T, n_in, B), **f),
             "g_state0": torch.empty((B, N), **f)}

    def step():
        sgr.recurrence_forward(graph, ev, lk, bs, dr, st, M, out=out, saved=saved, workspace=ws)
        sgr.recurrence_backward(graph, ev, lk, st, M, saved, G, workspace=ws, grads=grads)

    run = step
    use_graph = not args.no_graph
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            step()
        run = cg.replay

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # the same K steps again, each between its own event pair
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for k in range(args.steps):
        run()
        marks[k + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])

    # per-launch kernel durations: HIP events around every per-microstep launch
    sgr.profile_collect()
    sgr.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sgr.profile_enable(False)
    prof = sgr.profile_collect()
    fwd_us = 1e3 * prof["fwd_ms"] / max(prof["fwd_launches"], 1)
    bwd_us = 1e3 * prof["bwd_ms"] / max(prof["bwd_launches"], 1)
    fwd_n = prof["fwd_launches"] // args.steps
    bwd_n = prof["bwd_launches"] // args.steps

    fwd_b, bwd_b, Q = algorithmic_bytes(N, E, n_in, B, T, M)
    # a step's S microsteps of forward (backward) bytes are spread over its
    # forward (backward) launches: S + 1 per-microstep backward launches (the
    # first has no edge pass), one resident launch per direction, or for the
    # blocked kernels the part and epilogue launches of each microstep
    # together (2 S forward, 2 S + 1 backward); the "blocked" path pairs the
    # blocked forward with the per-microstep backward
    names = {"resident": ("res_fwd", "res_bwd"), "blocked": ("blk_fwd", "bwd_step"),
             "blocked_both": ("blk_fwd", "blk_bwd")}.get(path, ("fwd_step", "bwd_step"))
    per_kernel = {}
    # the resident forward also writes the outputs [T][B][N] itself
    fwd_launch_b = fwd_b * S / fwd_n + (4 * T * N * B if path == "resident" else 0)
    for kname, per_b, us in ((names[0], fwd_launch_b, fwd_us),
                             (names[1], bwd_b * S / bwd_n, bwd_us)):
        a = per_b / (us * 1e-6) / 1e9
        tr = measured_traffic(kname)
        m = None if tr is None else tr / (us * 1e-6) / 1e9
        per_kernel[kname] = {"achieved": a, "frac": a / HBM_PEAK_GBS, "launch_us": us,
                             "algorithmic_bytes_per_launch": per_b, "traffic": tr,
                             "measured_GBps": m,
                             "measured_frac": None if m is None else m / HBM_PEAK_GBS}
    # the dominant kernel is the one with the larger share of the step's time
    name = list(per_kernel)[1] if prof["bwd_ms"] >= prof["fwd_ms"] else list(per_kernel)[0]
    achieved = per_kernel[name]["achieved"]
    visits = S * E * B
    res = {
        "metric": METRIC,
        "value": visits / (ms * 1e-3),
        "unit": "edge-visits/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "ms_per_step_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: N={N} E={E} n_in={n_in} B={B} T={T} "
                               f"microsteps={M} (seed {w.seed})",
                   "parallelism": "single GPU", "hip_graph": use_graph},
        "yardstick_GBps": Q / (ms * 1e-3) / 1e9,
        "yardstick_frac_of_hbm_peak": Q / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels": {"path": path, "fwd_launch_us": fwd_us, "bwd_launch_us": bwd_us,
                    "fwd_launches_per_step": fwd_n, "bwd_launches_per_step": bwd_n},
        "roofline": {"bound": "hbm", "kernel": name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": per_kernel[name]["traffic"],
                     "measured_GBps": per_kernel[name]["measured_GBps"],
                     "measured_frac": per_kernel[name]["measured_frac"]},
        "roofline_by_kernel": per_kernel,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
