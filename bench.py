#!/usr/bin/env python3
"""Benchmark of the ZeRO-DP owned-partition step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

A step is one pass of the whole hot path over one batch of gradients:
zero_adam_step, i.e. the fused reduce + unscale/flag/sum-of-squares + Adam +
fp16 emit kernel and the small commit kernel after it (which also re-emits
the all-gather window of a skipped step).  Inputs are resident in HBM
before timing starts.  Prints one JSON line with the whole-step throughput
(owned elements per second, K steps back to back between device
synchronisations), the step's achieved HBM bandwidth against the 8 TB/s
peak (algorithmic bytes (2*Nd + 26) per owned element over the average
device time of the step's two kernels, from HIP events around K
back-to-back steps on the launch stream), and the oracle's rate on a
bounded sample of the same workload on one host core (and, as
cpu_baseline.all_cores, on every core the process may use, up to 16).
The reported workload is the 60B-parameter shard at Nd = 400 (S =
150,000,128 owned elements, 120 GB of slices), the largest that fits one
GPU; with the plain fused step the other four workloads are timed too and
reported under config.other_workloads, and a skipped step (an inf
gradient, the window re-emitted) is timed apart under config.skipped_step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "owned-shard elements updated/sec + achieved HBM GB/s vs peak, 1 MI355X"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c5",
                    help="c1..c5; c5 (the 60B-parameter shard at Nd = 400, the largest workload that fits "
                         "one GPU) is the reported one")
    ap.add_argument("--others", default="c1,c2,c3,c4",
                    help="plain fused step only: also time these workloads (fewer steps) and report them "
                         "under config.other_workloads ('' = none)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="gradient sets cycled through (0 = enough to exceed 1 GB of slices)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--max-grad-norm", type=float, default=0.0,
                    help="> 0: time the two-pass clipped step instead of the fused step")
    ap.add_argument("--dynamic-scale", type=int, default=0,
                    help="> 0: dynamic loss scaling with this growth interval")
    ap.add_argument("--bucket-elems", type=int, default=0,
                    help="> 0: bucketed step, the window ingested in buckets of this many elements")
    ap.add_argument("--buckets-per-call", type=int, default=1,
                    help="bucketed step: pass this many consecutive arrived buckets to one "
                         "zero_adam_step_buckets call (1: zero_adam_step_bucket per bucket)")
    ap.add_argument("--arrival", action="store_true",
                    help="bucketed step: copy each bucket into one of two constant-size receive "
                         "buffers on a side stream (the simulated reduce-scatter arrival), "
                         "overlapped with the previous bucket's step")
    ap.add_argument("--graph", action="store_true",
                    help="also time the same steps replayed from a HIP graph (reported as config.graph_step_us)")
    ap.add_argument("--gather-layers", action="store_true",
                    help="time the Pos+g+p on-demand gather of every layer (GPT-2 shaped workloads) "
                         "instead of the step")
    ap.add_argument("--layers-per-call", type=int, default=1,
                    help="with --gather-layers: gather this many consecutive layers per zero_gather_layers "
                         "call (one layer buffer each)")
    ap.add_argument("--sweep-nd", action="store_true",
                    help="time the fused step, its stream-mix and its slice reads on one window per Nd "
                         "(1 to 400, about 4 GB of algorithmic traffic per step) instead of a workload")
    ap.add_argument("--gather-streams", type=int, default=1, choices=(1, 2, 3, 4),
                    help="with --gather-layers: N > 1 rotates the layers over N streams (layer buffer "
                         "k %% N on stream k %% N), so one layer's gather overlaps the next ones' launches")
    a = ap.parse_args()
    if a.bucket_elems < 0 or a.bucket_elems % 8 or (a.bucket_elems and a.max_grad_norm > 0):
        ap.error("--bucket-elems must be a multiple of 8, and cannot be combined with clipping")
    if a.arrival and not a.bucket_elems:
        ap.error("--arrival needs --bucket-elems")
    if a.buckets_per_call < 1 or (a.buckets_per_call > 1 and (a.arrival or not a.bucket_elems)):
        ap.error("--buckets-per-call > 1 needs --bucket-elems and buckets read in place (no --arrival)")
    if a.layers_per_call < 1:
        ap.error("--layers-per-call must be >= 1")
    return a


def kernel_fingerprint():
    """Hash of the device source and its build flags; a counter summary in
    profiles/ applies to the kernel only while this matches."""
    import hashlib
    from zero_partitioned_mixed_buffer_amd import build_lib
    h = hashlib.sha256()
    for f in ("zero_dp_kernels.hip", "zero_dp_internal.h"):
        with open(os.path.join(build_lib.CSRC, f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(build_lib.HIP_FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per fused step (all of its fused launches) from the committed
    rocprofv3 counter summaries, or None if absent or stale.  A summary of
    one workload gives traffic_bytes_per_launch; a summary of several gives
    traffic_bytes_per_step_<workload> for each."""
    import glob
    import re
    fp = kernel_fingerprint()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "fused_step_*pmc*.md"))):
        text = open(path).read()
        m_fp = re.search(r"kernel_fingerprint:\s*([0-9a-f]+)", text)
        if not m_fp or m_fp.group(1) != fp:
            continue
        m_tr = re.search(rf"traffic_bytes_per_step_{workload}:\s*([0-9]+)", text)
        if m_tr is None and os.path.basename(path).startswith(f"fused_step_{workload}_"):
            m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
        if m_tr:
            return int(m_tr.group(1))
    return None


def attainable_copy(torch, dev, B, reps=5):
    """Attainable streaming bandwidth on this GPU: the library's own copy
    kernel (zero_gather_params over one 4 GiB window) moving 4 GiB into
    another 4 GiB buffer; GB/s of read + write."""
    n = 1 << 31  # fp16 elements
    src = torch.empty(n, dtype=torch.float16, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    B.gather_params([src], n, 0, n, dst, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        B.gather_params([src], n, 0, n, dst, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": 4 * n / (ms * 1e-3) / 1e9, "bytes_moved": 4 * n, "kernel": "copy_f16_kernel",
            "note": "4 GiB read + 4 GiB written per copy, mean of 5 back-to-back copies"}


def attainable_triad(torch, dev, B, reps=5):
    """STREAM's triad a = b + q*c through the library's calibration kernel
    over 2^30 fp32 elements per array (4 GiB each): GB/s of 8 bytes read
    and 4 written per element."""
    n = 1 << 30
    b = torch.ones(n, dtype=torch.float32, device=dev)
    c = torch.ones(n, dtype=torch.float32, device=dev)
    a = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    B.calib_triad(a, b, c, 3.0, n, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        B.calib_triad(a, b, c, 3.0, n, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    torch.cuda.empty_cache()
    return {"triad_gbs": 12 * n / (ms * 1e-3) / 1e9, "triad_bytes": 12 * n,
            "triad_kernel": "triad_kernel (3 x 4 GiB fp32, mean of 5 back-to-back launches)"}


def calibration_copy(torch, dev):
    """A plain device copy of known size (256 MiB -> 256 MiB) for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a profiled run; not timed."""
    a = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def cpu_baseline(w, n_sample, budget_s, max_grad_norm=0.0, scale_interval=0):
    """The oracle, as it stands, on a bounded sample of the workload's window
    (the clipped or dynamically scaled step when the timed step is; a
    bucketed step computes what the whole-window step computes)."""
    import numpy as np
    import oracle
    from workloads import gen
    master = gen.host_params(w.seed, w.psi, 0, n_sample, w.param_sigma)
    sh = oracle.OwnedShard(master, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                           weight_decay=w.weight_decay, max_grad_norm=max_grad_norm,
                           scale_interval=scale_interval, loss_scale=w.loss_scale)
    grads = [gen.host_grad_slices(w.seed, s, 0, w.nd, n_sample, 0, w.psi, w.grad_sigma, w.loss_scale,
                                  w.dist) for s in (1, 2)]
    steps = 0
    t0 = time.perf_counter()
    while True:
        sh.step(grads[steps % 2], w.loss_scale)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    rate = n_sample * steps / el
    return {"value": rate, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} oracle steps over a {n_sample}-element window of workload {w.key} "
                      f"(Nd={w.nd}, numpy float64, one thread"
                      f"{', clipped' if max_grad_norm > 0 else ''}"
                      f"{', dynamic loss scale' if scale_interval > 0 else ''}), {el:.1f} s",
            "gbs": rate * (2 * w.nd + 26) / 1e9}


def _oracle_share(job):
    """One host core's share of the all-cores oracle figure: its own chunk of
    the workload's parameters and gradients, stepped by the oracle for
    about budget_s.  Returns (elements stepped, seconds)."""
    import oracle
    from workloads import configs, gen
    key, k, n_sample, budget_s, max_grad_norm, scale_interval = job
    w = configs.ALL[key]
    lo = (k * n_sample) % max(1, w.psi - n_sample)
    master = gen.host_params(w.seed, w.psi, lo, lo + n_sample, w.param_sigma)
    sh = oracle.OwnedShard(master, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                           weight_decay=w.weight_decay, max_grad_norm=max_grad_norm,
                           scale_interval=scale_interval, loss_scale=w.loss_scale)
    grads = [gen.host_grad_slices(w.seed, s, 0, w.nd, n_sample, lo, w.psi, w.grad_sigma, w.loss_scale,
                                  w.dist) for s in (1, 2)]
    steps = 0
    t0 = time.perf_counter()
    while True:
        sh.step(grads[steps % 2], w.loss_scale)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return n_sample * steps, el


def cpu_baseline_all_cores(w, n_sample, budget_s, max_grad_norm=0.0, scale_interval=0):
    """The same oracle on every host core this process may use (at most 16):
    one process per core, each stepping its own chunk of the window at the
    same time (elements are independent).  Uses fork, and runs before this
    process loads the HIP library, so no child is made from a process that
    has touched the GPU."""
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(16, affinity))
    jobs = [(w.key, k, n_sample, budget_s, max_grad_norm, scale_interval) for k in range(cores)]
    with mp.get_context("fork").Pool(cores) as pool:
        res = pool.map(_oracle_share, jobs, chunksize=1)
    rate = sum(e / t for e, t in res)
    return {"value": rate, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "affinity_cores": affinity, "core_cap": 16,
            "sample": f"{cores} processes (one per core this process may use, {affinity}, capped at 16), "
                      f"each stepping its own {n_sample}-element chunk of workload {w.key} "
                      f"for {budget_s:.0f} s (numpy float64, one thread each)",
            "gbs": rate * (2 * w.nd + (34 if max_grad_norm > 0 else 26)) / 1e9}


def cpu_baseline_gather(w, windows, part, ranges, budget_s):
    """oracle.gather, as it stands, over every layer of the workload from
    host copies of one set of the windows, repeated for about budget_s."""
    import oracle
    passes = 0
    t0 = time.perf_counter()
    while True:
        for lo, hi in ranges:
            oracle.gather(windows, part, lo, hi)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": w.psi * passes / el, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} oracle gather passes over every layer of workload {w.key} "
                      f"({len(ranges)} layers, Psi = {w.psi}, numpy, one thread), {el:.1f} s"}


def bench_gather(args):
    """Pos+g+p: gather every layer of a GPT-2 shaped list (one forward's
    worth of on-demand gathers, Psi elements) from the Nd owners' windows
    into constant-size layer buffers used in turn, one per stream and at
    least two (a layer buffer is released by reusing it that many layers
    later)."""
    import torch
    from workloads import configs, gen
    from zero_partitioned_mixed_buffer_amd import binding as B
    w = configs.ALL[args.workload]
    if len(w.numels) < 16:
        log(f"--gather-layers needs a GPT-2 shaped workload (c2 or c3), not {w.key}")
        sys.exit(2)
    plan, _ = B.plan_partitions(list(w.numels), w.nd, 256)
    part = plan["part"]
    n_layer = (len(w.numels) - 4) // 12
    ranges = configs.layer_ranges(w.numels, configs.gpt2_layers(n_layer))
    dev = torch.device("cuda", 0)
    # enough copies of the windows that one pass reads more than 1.5 GB of
    # windows no earlier pass left in the MALL
    copies = max(1, min(8, -(-int(1.5e9) // (2 * plan["padded"]))))
    sets = []
    for c in range(copies):
        ws = []
        for r in range(w.nd):
            t = torch.empty(part, dtype=torch.float32, device=dev)
            gen.device_fill_params(t, w.seed + 97 * c + r, w.param_sigma, max(0, min(part, w.psi - r * part)))
            ws.append(t.to(torch.float16))
            del t
        sets.append(ws)
    biggest = max(hi - lo for lo, hi in ranges)
    K = args.layers_per_call
    calls = [ranges[c:c + K] for c in range(0, len(ranges), K)]  # the layers gathered together
    nbuf = max(2, args.gather_streams)
    # one layer buffer per layer of a call, for each of nbuf calls in turn
    bufs = [[torch.empty(biggest, dtype=torch.float16, device=dev) for _ in range(K)] for _ in range(nbuf)]
    stream = torch.cuda.current_stream()
    # layer buffer b is only ever written on streams[b], so reuse is ordered
    if args.gather_streams > 1:
        streams = [stream] + [torch.cuda.Stream() for _ in range(nbuf - 1)]  # default priority
    else:
        streams = [stream] * nbuf
    log(f"gather: {w.key}, {len(ranges)} layers (largest {biggest} elements), Nd={w.nd} windows of {part}, "
        f"{copies} window set(s), {args.gather_streams} stream(s)")

    def one_pass(i):
        ws = sets[i % copies]
        for k, group in enumerate(calls):
            if K == 1:
                lo, hi = group[0]
                B.gather_params(ws, part, lo, hi, bufs[k % nbuf][0], streams[k % nbuf])
            else:
                B.gather_layers(ws, part, group, [b[:hi - lo] for b, (lo, hi) in zip(bufs[k % nbuf], group)],
                                streams[k % nbuf])

    for i in range(args.warmup):
        one_pass(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    side = [st for st in streams[1:] if st is not stream]
    for st in side:
        st.wait_event(e0)
    for i in range(args.steps):
        one_pass(args.warmup + i)
    for st in side:
        done = torch.cuda.Event()
        done.record(st)
        stream.wait_event(done)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    pieces = sum(1 + (hi - 1) // part - lo // part for lo, hi in ranges if hi > lo)
    launches = sum(-(-sum(1 + (hi - 1) // part - lo // part for lo, hi in group if hi > lo) // 16)
                   for group in calls)
    gbs = 4 * w.psi / (ms * 1e-3) / 1e9
    log(f"gather pass: {ms * 1e3:.1f} us ({launches} launches, {pieces} window pieces), {gbs:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_gather(w, [t.cpu().numpy() for t in sets[0]], part, ranges, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.3e} elements/s on 1 core")
    out = {
        "metric": "parameter elements gathered/sec (Pos+g+p on-demand layer gather), 1 MI355X",
        "value": w.psi / (ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "wall_ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": f"{w.key}: every layer of {w.title}", "layers": len(ranges),
                   "largest_layer": biggest, "nd": w.nd, "window": part, "launches_per_pass": launches,
                   "window_pieces_per_pass": pieces, "streams": args.gather_streams,
                   "layers_per_call": K,
                   "window_sets_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes_per_pass": 4 * w.psi,
                     "kernel": "copy_f16_kernel" + (f" ({K} layers per zero_gather_layers call)" if K > 1 else ""),
                     "kernel_fingerprint": kernel_fingerprint()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


SWEEP_ND = (1, 2, 4, 8, 12, 16, 20, 24, 32, 48, 64, 100, 200, 400)


def bench_sweep_nd(args):
    """The fused step across Nd: for each Nd one window of about 4 GB of
    algorithmic traffic per step ((2 Nd + 26) bytes per element, Adam), two
    shards stepped in turn, then the same window's stream-mix and
    slice-read kernels, each timed with HIP events on the launch stream."""
    import torch
    from workloads import gen
    from zero_partitioned_mixed_buffer_amd import OwnedShard, binding as B
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)

    def timed(fn):
        for i in range(max(args.warmup, 1)):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    rows = []
    log("nd window step_us GB/s frac stream_mix_GB/s step/mix slice_read_GB/s read_share")
    for nd in SWEEP_ND:
        n = int(4e9 / (2 * nd + 26)) // 1024 * 1024
        sl = torch.empty((nd, n), dtype=torch.float16, device=dev)
        gen.device_fill_grads(sl, 7, 1, 1e-3, 1024.0, "normal", n)
        shards = [OwnedShard(torch.randn(n, device=dev) * 0.02, **hp) for _ in range(2)]
        ag = torch.zeros(n, dtype=torch.float16, device=dev)
        src = B.grad_src(sl, n, 0, n, nd, 1024.0)

        def step(i):
            sh = shards[i % 2]
            B.adam_step(src, sh.state, sh.hp, ag, 0, sh.workspace, stream)

        t = timed(step)
        sh = shards[0]
        cur = sh.control()["cur"]
        ins = [sh.master[cur], sh.exp_avg[cur], sh.exp_avg_sq[cur]]
        outs = [sh.master[cur ^ 1], sh.exp_avg[cur ^ 1], sh.exp_avg_sq[cur ^ 1]]
        tm = timed(lambda i: B.calib_stream_mix(src, ins, outs, ag, stream))
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        tr = timed(lambda i: B.calib_slice_read(src, sink, stream))
        by = (2 * nd + 26) * n
        row = {"nd": nd, "window": n, "step_us": t, "gbs": by / t / 1e3, "frac": by / t / 1e3 / PEAK_HBM_GBS,
               "stream_mix_gbs": by / tm / 1e3, "step_over_mix": tm / t,
               "slice_read_gbs": 2 * nd * n / tr / 1e3, "slice_read_share": tr / t}
        rows.append(row)
        log(f"{nd} {n} {t:.1f} {row['gbs']:.0f} {row['frac']:.3f} {row['stream_mix_gbs']:.0f} "
            f"{row['step_over_mix']:.3f} {row['slice_read_gbs']:.0f} {row['slice_read_share']:.3f}")
        del sl, shards, ag, src, ins, outs, sh
        torch.cuda.empty_cache()
    lo = min(rows, key=lambda r: r["frac"])
    out = {
        "metric": "fused step HBM rate across Nd, lowest fraction of 8 TB/s",
        "value": lo["frac"], "unit": "fraction of 8 TB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": lo["step_us"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "one window per Nd at about 4 GB of algorithmic traffic per step", "rows": rows},
        "kernel_fingerprint": kernel_fingerprint(),
    }
    print(json.dumps(out), flush=True)


def host_cpu():
    """The host CPU's model name (as lscpu prints it, from /proc/cpuinfo),
    the cores this process may run on, and the cores the host has."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "affinity_cores": len(os.sched_getaffinity(0)), "host_cores": os.cpu_count()}


STAGES = ("DP", "Pos", "Pos+g", "Pos+g+p")


def memory_model_report(B, w):
    """The library's memory and communication model (zero_memory_model) for
    the workload's Psi and Nd: per-device model-state GB (1e9 bytes) of each
    stage, the reduction against plain data parallelism, and the per-rank
    communication volume in elements (nominal and over a ring)."""
    rows = []
    for st in range(4):
        r = B.memory_model(w.psi, w.nd, st)
        rows.append({"stage": STAGES[st],
                     "params_gb": r["params_bytes"] / 1e9, "grads_gb": r["grads_bytes"] / 1e9,
                     "optim_gb": r["optim_bytes"] / 1e9, "total_gb": r["total_bytes"] / 1e9,
                     "total_gb_1dp": round(r["total_bytes"] / 1e9, 1),
                     "reduction_vs_dp": r["reduction_vs_dp"],
                     "comm_elems": r["comm_elems"], "comm_elems_ring": r["comm_elems_ring"]})
    return {"psi": w.psi, "nd": w.nd, "k_bytes_per_param": 12, "stages": rows}


def log_memory_model(mm):
    log(f"memory model, Psi = {mm['psi']:.4g}, Nd = {mm['nd']}: " + " / ".join(
        f"{r['stage']} {r['total_gb_1dp']:.1f} GB ({r['reduction_vs_dp']:.2f}x)" for r in mm["stages"]))
    log("communication per rank and step: " + " / ".join(
        f"{r['stage']} {r['comm_elems']:.4g} elements" for r in mm["stages"]))


def measure_step(args, w, steps, warmup, graph=False, skip_timing=False):
    """Allocates the workload's inputs and state on the GPU, times `steps`
    whole steps after `warmup` untimed ones, frees everything, and returns
    the measurements.  Nothing but the step's own launches runs on the
    stream in the timed regions."""
    import torch
    from workloads import gen
    from zero_partitioned_mixed_buffer_amd import OwnedShard, binding as B
    owner = w.owners[-1]
    plan, _ = B.plan_partitions(list(w.numels), w.nd, 256)
    S = plan["part"]
    off = owner * S
    valid = max(0, min(S, w.psi - off))  # real (non-padding) elements of the window
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"workload {w.key}: {w.title}; S={S} owner={owner} offset={off} Nd={w.nd}")

    slice_bytes = 2 * w.nd * S
    rot = args.rotate or max(1, min(8, -(-(1 << 30) // max(slice_bytes, 1))))
    gsets = []
    for r in range(rot):
        t = torch.empty((w.nd, S), dtype=torch.float16, device=dev)
        gen.device_fill_grads(t, w.seed, r + 1, w.grad_sigma, w.loss_scale, w.dist, valid)
        gsets.append(t)
    log(f"{rot} gradient set(s) of {slice_bytes / 1e9:.3f} GB filled")

    # Several ranks' owned shards (each with its own ping-pong state and
    # all-gather window) are stepped in turn, so that at least 1.5 GB of
    # other traffic passes between two visits to one shard's state: the
    # 256 MB MALL cannot serve a step the state written by the previous one
    # (between two optimizer steps of real training, forward and backward
    # traffic evicts it too).  Every step still processes one full shard.
    step_bytes = (2 * w.nd + 26) * S
    n_shards = 1 if step_bytes > 2e9 else min(w.nd, max(2, -(-int(1.5e9) // step_bytes)))
    # the all-gather buffer: the full flat fp16 buffer when it is modest,
    # otherwise one window per stepped shard
    full = plan["padded"] * 2 <= (8 << 30)
    ag = torch.zeros(plan["padded"] if full else S * n_shards, dtype=torch.float16, device=dev)
    shards, ag_offs = [], []
    for r in range(n_shards):
        rank = (owner + r) % w.nd
        roff = rank * S
        rvalid = max(0, min(S, w.psi - roff))
        master = torch.empty(S, dtype=torch.float32, device=dev)
        gen.device_fill_params(master, w.seed + roff, w.param_sigma, rvalid)
        shards.append(OwnedShard(master, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                                 weight_decay=w.weight_decay, max_grad_norm=args.max_grad_norm,
                                 scale_interval=args.dynamic_scale, loss_scale=w.loss_scale))
        ag_offs.append(roff if full else r * S)
        shards[r].emit(ag, ag_offs[r])
        del master
    torch.cuda.synchronize()
    log(f"{n_shards} owned shard(s) stepped in turn; all-gather: {'full flat buffer' if full else 'windows'}")

    stream = torch.cuda.current_stream()
    srcs = [B.grad_src(t, S, 0, S, w.nd, w.loss_scale) for t in gsets]

    clipped = args.max_grad_norm > 0
    bucketed = args.bucket_elems > 0
    if bucketed:
        nb_elems = min(args.bucket_elems, S)
        buckets = [(o, min(nb_elems, S - o)) for o in range(0, S, nb_elems)]
        side = torch.cuda.Stream(device=dev)  # default priority
        recv = [torch.empty((w.nd, nb_elems), dtype=torch.float16, device=dev) for _ in range(2)]
        arrived = [torch.cuda.Event() for _ in range(2)]
        consumed = [torch.cuda.Event() for _ in range(2)]
        for ev in consumed:
            ev.record(stream)
        log(f"bucketed: {len(buckets)} buckets of {nb_elems} elements"
            + ("; arrival copies into 2 constant-size receive buffers on a side stream" if args.arrival else
               "; buckets read in place"))
        # the gradient sources of every bucket and call, made once per
        # gradient set outside the timed region (they do not change)
        K = args.buckets_per_call
        call_groups = [buckets[c:c + K] for c in range(0, len(buckets), K)]
        bucket_srcs = [[B.grad_src(gs, S, o, k, w.nd, w.loss_scale) for o, k in buckets] for gs in gsets]
        call_arrays = [[B.bucket_array([(B.grad_src(gs, S, o, k, w.nd, w.loss_scale), o) for o, k in group])
                        for group in call_groups] for gs in gsets]
        recv_srcs = [B.grad_src(r, nb_elems, 0, nb_elems, w.nd, w.loss_scale) for r in recv]

    def launch_bucketed(i, s):
        sh = shards[i % n_shards]
        gs = gsets[i % rot]
        if args.buckets_per_call > 1:
            arrays = call_arrays[i % rot]
            for c, arr in enumerate(arrays):
                phase = (B.BUCKET_FIRST if c == 0 else 0) | (B.BUCKET_LAST if c == len(arrays) - 1 else 0)
                B.adam_step_buckets(arr, sh.state, sh.hp, S, ag, ag_offs[i % n_shards], phase, sh.workspace, s)
            return
        for b, (o, k) in enumerate(buckets):
            phase = (B.BUCKET_FIRST if b == 0 else 0) | (B.BUCKET_LAST if b == len(buckets) - 1 else 0)
            if args.arrival:
                r = b % 2
                side.wait_event(consumed[r])
                with torch.cuda.stream(side):
                    recv[r][:, :k].copy_(gs[:, o:o + k])
                arrived[r].record(side)
                stream.wait_event(arrived[r])
                src = recv_srcs[r]
                if k != nb_elems:
                    src = B.grad_src(recv[r], nb_elems, 0, k, w.nd, w.loss_scale)
            else:
                src = bucket_srcs[i % rot][b]
            B.adam_step_bucket(src, sh.state, sh.hp, o, S, ag, ag_offs[i % n_shards], phase, sh.workspace, s)
            if args.arrival:
                consumed[r].record(stream)

    def launch(i, s=None):
        sh = shards[i % n_shards]
        s = s or stream
        if bucketed:
            launch_bucketed(i, s)
            return
        if clipped:  # two passes; a skipped step leaves the window untouched
            B.adam_step_clipped(srcs[i % rot], sh.state, sh.hp, sh.grad_buf, ag, ag_offs[i % n_shards],
                                sh.workspace, s)
            return
        # the fused kernel and the commit kernel (which also re-emits the
        # window of a skipped step)
        B.adam_step(srcs[i % rot], sh.state, sh.hp, ag, ag_offs[i % n_shards], sh.workspace, s)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back, nothing else on the stream.
    t0 = time.perf_counter()
    for i in range(steps):
        launch(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Device time of the step's kernels: K steps back to back between two
    # HIP events on the launch stream (per-launch event records would add a
    # cache release and a dispatch gap to every launch).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        launch(warmup + steps + i)
    e1.record(stream)
    torch.cuda.synchronize()
    kern_avg = e0.elapsed_time(e1) / steps
    # Distribution: the same launches, each between its own pair of events
    # (the records add a little to every launch, so the mean above is the
    # figure reported; these are its spread).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        launch(warmup + 2 * steps + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    pct = lambda q: per[min(len(per) - 1, int(round(q * (len(per) - 1))))]  # noqa: E731
    ctls = [sh.control() for sh in shards]
    if sum(c["t"] for c in ctls) != warmup + 3 * steps or any(c["skipped"] for c in ctls):
        log(f"unexpected control state after timing: {ctls}")
        sys.exit(1)

    graph_us = None
    if graph and not args.arrival:
        # the same K steps captured once in a HIP graph and replayed: the
        # launches are identical, only the host-side launch cost goes
        base = warmup + 3 * steps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(steps):
                launch(base + j, torch.cuda.current_stream())
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(3):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1e3 / (3 * steps)
        log(f"the same steps from a HIP graph: {graph_us:.1f} us per step")
        del g

    skip = None
    if skip_timing and not (clipped or bucketed or args.dynamic_scale):
        # A step with an inf gradient (slice min(17, Nd-1), window element
        # S/2): the fused pass runs as on any step, then the commit kernel
        # skips it and re-emits the window from the committed master
        # (6 more bytes per element).  Timed apart from the clean steps.
        k, j = min(17, w.nd - 1), S // 2
        sh = shards[0]
        gs = gsets[0]
        keep = gs[k, j].clone()
        gs[k, j] = float("inf")
        t_before = sh.control()["t"]
        reps = 3
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(reps):
            B.adam_step(srcs[0], sh.state, sh.hp, ag, ag_offs[0], sh.workspace, stream)
        s1.record(stream)
        torch.cuda.synchronize()
        c = sh.control()
        gs[k, j] = keep
        if c["t"] != t_before or c["skipped"] != reps or c["overflow"] != 1:
            log(f"the injected step was not skipped: {c}")
            sys.exit(1)
        skip_us = s0.elapsed_time(s1) * 1e3 / reps
        skip = {"step_us": skip_us, "extra_bytes_per_elem": 6,
                "injected": f"+inf at slice {k}, window element {j}",
                "extra_us_vs_clean": skip_us - kern_avg * 1e3}
        log(f"skipped step (inf at slice {k}, element {j}): {skip_us:.1f} us "
            f"({skip_us - kern_avg * 1e3:+.1f} us against a clean step; the re-emit moves 6 B per element)")

    mix = None
    if not (clipped or bucketed):
        # The same buffers through the calibration kernel that moves exactly
        # this step's streams (Nd fp16 slices and 3 fp32 state arrays read,
        # 3 fp32 arrays and the fp16 window written) in the same launch
        # shape with no arithmetic: the rate this memory schedule attains
        # on this GPU.  It writes the non-current state set and the windows,
        # which the next step overwrites anyway.
        ctls = [sh.control() for sh in shards]  # cur after the graph and skip runs

        def mix_launch(i):
            r = i % n_shards
            sh, cur = shards[r], ctls[r]["cur"]
            ins = [sh.master[cur], sh.exp_avg[cur], sh.exp_avg_sq[cur]]
            outs = [sh.master[cur ^ 1], sh.exp_avg[cur ^ 1], sh.exp_avg_sq[cur ^ 1]]
            B.calib_stream_mix(srcs[i % rot], ins, outs, ag[ag_offs[r]:ag_offs[r] + S], stream)

        for i in range(max(1, min(warmup, 3))):
            mix_launch(i)
        torch.cuda.synchronize()
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for i in range(steps):
            mix_launch(i)
        m1.record(stream)
        torch.cuda.synchronize()
        mix_us = m0.elapsed_time(m1) * 1e3 / steps
        mix = {"us": mix_us, "gbs": (2 * w.nd + 26) * S / (mix_us * 1e-6) / 1e9}

        # The slice reads alone (2*Nd bytes per element) in the same visit
        # order and launch pieces, with no state streams and no stores: the
        # rate the step's slice streams attain by themselves.
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for i in range(max(1, min(warmup, 3))):
            B.calib_slice_read(srcs[i % rot], sink, stream)
        torch.cuda.synchronize()
        m0.record(stream)
        for i in range(steps):
            B.calib_slice_read(srcs[i % rot], sink, stream)
        m1.record(stream)
        torch.cuda.synchronize()
        read_us = m0.elapsed_time(m1) * 1e3 / steps
        mix["slice_read_us"] = read_us
        mix["slice_read_gbs"] = 2 * w.nd * S / (read_us * 1e-6) / 1e9

    # algorithmic bytes per owned element: fused 2*Nd + 26; clipped
    # (2*Nd + 4) for the reduce pass + 30 for the update pass
    bytes_elem = 2 * w.nd + (34 if clipped else 26)
    achieved = bytes_elem * S / (kern_avg * 1e-3) / 1e9
    if bucketed and args.buckets_per_call > 1:
        K = args.buckets_per_call
        what = f"bucketed step ({len(buckets)} buckets in {-(-len(buckets) // K)} calls of up to {K} + commit)"
    else:
        what = None
    what = what or (f"bucketed step ({len(buckets)} launches + commit)" if bucketed else
            "clipped step (reduce + update + commit kernels)" if clipped else "fused step (fused + commit kernels)")
    ms_step = wall * 1e3 / steps
    log(f"{w.key} {what}: avg {kern_avg * 1e3:.1f} us over {steps} back-to-back steps; "
        f"step {ms_step * 1e3:.1f} us; {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBS:.3f} of peak)")
    if mix is not None:
        log(f"{w.key} the same streams with no arithmetic (stream-mix kernel): {mix['us']:.1f} us, "
            f"{mix['gbs']:.0f} GB/s; the step runs at {achieved / mix['gbs']:.3f} of it")
        log(f"{w.key} the slice reads alone (slice-read kernel): {mix['slice_read_us']:.1f} us, "
            f"{mix['slice_read_gbs']:.0f} GB/s of slice reads; they take {mix['slice_read_us'] / (kern_avg * 1e3):.3f} "
            f"of the step's time")
    res = {
        "w": w, "S": S, "owner": owner, "rot": rot, "n_shards": n_shards, "full": full,
        "ms_step": ms_step, "kern_avg_ms": kern_avg, "pcts_us": [pct(0.1), pct(0.5), pct(0.9)],
        "bytes_elem": bytes_elem, "achieved_gbs": achieved, "graph_us": graph_us, "skip": skip,
        "what": what, "n_buckets": len(buckets) if bucketed else 0, "mix": mix,
    }
    del gsets, srcs, shards, ag
    if bucketed:
        del recv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the step of one rank runs on one MI355X and no "
              f"collective is part of this path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.gather_layers:
        bench_gather(args)
        return
    if args.sweep_nd:
        bench_sweep_nd(args)
        return

    from workloads import configs

    w = configs.ALL[args.workload]
    cpu_all = None
    if not args.no_cpu_baseline:
        # before torch and the HIP library are loaded: the worker processes are forked, and a fork
        # taken after a library has started threads can inherit a held lock
        n_pool = min(w.psi // w.nd, 1 << 21) if w.nd <= 64 else min(w.psi // w.nd, 1 << 16)
        cpu_all = cpu_baseline_all_cores(w, n_pool, args.cpu_seconds / 2, args.max_grad_norm, args.dynamic_scale)
        log(f"oracle: {cpu_all['value']:.3e} elements/s on {cpu_all['cores']} cores")

    import torch
    from zero_partitioned_mixed_buffer_amd import binding as B
    dev = torch.device("cuda", 0)

    clipped = args.max_grad_norm > 0
    bucketed = args.bucket_elems > 0
    plain = not (clipped or bucketed or args.dynamic_scale or args.arrival)
    mm = memory_model_report(B, w)
    log_memory_model(mm)

    res = measure_step(args, w, args.steps, args.warmup, graph=args.graph, skip_timing=plain)
    S = res["S"]

    others = {}
    if plain and args.others:
        # the other workloads' whole steps, each in its own allocation (the
        # headline's buffers are freed first), reported beside the headline
        for key in [k for k in args.others.split(",") if k and k != w.key]:
            wo = configs.ALL[key]
            r = measure_step(args, wo, max(5, args.steps // 2), min(args.warmup, 3))
            others[key] = {"workload": f"{wo.key}: {wo.title}", "owned_elems": r["S"], "nd": wo.nd,
                           "bytes_per_elem": r["bytes_elem"], "step_us_events": r["kern_avg_ms"] * 1e3,
                           "step_us_host": r["ms_step"] * 1e3, "hbm_gbs": r["achieved_gbs"],
                           "frac_of_peak": r["achieved_gbs"] / PEAK_HBM_GBS,
                           "elements_per_s": r["S"] / (r["ms_step"] * 1e-3),
                           "mix_gbs": r["mix"]["gbs"] if r["mix"] else None,
                           "frac_of_mix": r["achieved_gbs"] / r["mix"]["gbs"] if r["mix"] else None,
                           "slice_read_gbs": r["mix"]["slice_read_gbs"] if r["mix"] else None,
                           "slice_read_share": (r["mix"]["slice_read_us"] / (r["kern_avg_ms"] * 1e3)
                                                if r["mix"] else None)}

    calibration_copy(torch, dev)
    attain = attainable_copy(torch, dev, B)
    attain.update(attainable_triad(torch, dev, B))
    if res["mix"] is not None:
        attain["mix_gbs"] = res["mix"]["gbs"]
        attain["mix_kernel"] = "stream_mix_kernel (this workload's streams, the step's launch shape, no arithmetic)"
        attain["slice_read_gbs"] = res["mix"]["slice_read_gbs"]
        attain["slice_read_us"] = res["mix"]["slice_read_us"]
        attain["slice_read_kernel"] = ("slice_read_kernel (this workload's 2*Nd bytes of slice reads per element "
                                       "alone, the step's visit order and launch pieces)")
    log(f"attainable on this GPU: copy {attain['copy_gbs']:.0f} GB/s, triad {attain['triad_gbs']:.0f} GB/s"
        + (f", this step's stream mix {attain['mix_gbs']:.0f} GB/s" if "mix_gbs" in attain else ""))
    traffic = None if (clipped or bucketed) else measured_traffic(w.key)

    kern_avg = res["kern_avg_ms"]
    ms_step = res["ms_step"]
    bytes_elem = res["bytes_elem"]
    achieved = res["achieved_gbs"]

    cpu = None
    if not args.no_cpu_baseline:
        n_sample = min(S, 1 << 21) if w.nd <= 64 else min(S, 1 << 16)
        cpu = cpu_baseline(w, n_sample, args.cpu_seconds, args.max_grad_norm, args.dynamic_scale)
        log(f"oracle: {cpu['value']:.3e} elements/s on 1 core")
        cpu["host"] = host_cpu()
        cpu["all_cores"] = cpu_all

    out = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": f"{w.key}: {w.title}",
            "nd": w.nd,
            "owner": res["owner"],
            "owned_elems": S,
            "bytes_per_elem": bytes_elem,
            "grad_sets_rotated": res["rot"],
            "shards_rotated": res["n_shards"],
            "allgather": "full flat buffer" if res["full"] else "one window per shard",
            "step_hbm_gbs": bytes_elem * S / (ms_step * 1e-3) / 1e9,
            "max_grad_norm": args.max_grad_norm,
            "dynamic_scale_interval": args.dynamic_scale,
            "bucket_elems": args.bucket_elems,
            "bucket_arrival_copies": bool(args.arrival),
            "buckets_per_call": args.buckets_per_call if bucketed else None,
            "graph_step_us": res["graph_us"],
            "skipped_step": res["skip"],
            "memory_model": mm,
            "other_workloads": others or None,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            # measured HBM bytes per step (rocprofv3 counters, committed summary)
            # over the same average step duration, in GB/s like `achieved`
            "traffic": None if traffic is None else traffic / (kern_avg * 1e-3) / 1e9,
            "timed_unit": ("one step call, timed with HIP events on its stream: every launch of the kernel "
                           "below over the window (a window longer than two launch lengths takes several "
                           "fused launches), then the commit launch; a rocprofv3 summary gives the fused "
                           "kernel per launch, and the launches times their average plus the commit's "
                           "make this step"),
            "traffic_bytes_per_step": traffic,
            "algorithmic_bytes_per_step": bytes_elem * S,
            "kernel": ("reduce_owned_kernel + clipped_update_kernel + commit_kernel" if clipped else
                       (f"fused_runs_kernel, {res['n_buckets']} buckets in calls of {args.buckets_per_call}"
                        " + commit_kernel" if args.buckets_per_call > 1 else
                        f"fused_step_kernel x {res['n_buckets']} buckets + commit_kernel") if bucketed else
                       "fused_step_kernel + commit_kernel"),
            "step_avg_us": kern_avg * 1e3,
            "step_us_p10_p50_p90_events": res["pcts_us"],
            "attainable": attain,
            "frac_of_attainable": achieved / attain["copy_gbs"],
            "frac_of_mix": achieved / attain["mix_gbs"] if "mix_gbs" in attain else None,
            # the share of the step's time that its slice reads alone take
            "slice_read_share": (attain["slice_read_us"] / (kern_avg * 1e3) if "slice_read_us" in attain
                                 else None),
            "kernel_fingerprint": kernel_fingerprint(),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
