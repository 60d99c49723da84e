#!/usr/bin/env python3
"""Decode-step benchmark of the sparse attention hot path on one GPU.

The timed step is one decode step of one layer of the bit-plane index at a
1,048,576-token context: 8 KV heads x 4 query heads (GQA), d = 128, a read
plan of B = 56 plane bits per KV head, k = 512 selected rows per KV head:

    fathom_plan -> fathom_scan (+ 64-token block and 512-token group maxima)
                -> topk_select_block_max_split -> gather_attend

All inputs are seeded synthetic data (synth.fathom_case(3)) resident in HBM
before timing starts.  Eight copies of the plane index and of the K/V cache
rotate between steps, so the 256 MB last-level cache can serve neither the
index nor the selected K/V rows from one step to the next (a real decode
step reads each layer's index and rows once).  The timed steps carry no
events between their two bracketing ones.

Output: one JSON line.  `value` is keys scored per second over the whole
step (n * G / step time).  `roofline` prices the dominant kernel (the fused
fathom_plan_scan) against HBM: algorithmic bytes per launch (plane-prefix
bits, one scale/offset word per active channel per 64-token block, the fp32
score write) over its launch time, taken as the mean of back-to-back launches
over the rotating copies between two HIP events on the stream they run on
(what a kernel trace of the step reports as its average duration).
`roofline_valu` prices the same launches against the vector ALU (one
weighted accumulate per plane bit per token).  `cpu_baseline` is the CPU
oracle (fp64 NumPy) timed on the host on the same 1M-token workload, one KV
head at a time on one thread; `cpu_baseline_all_cores` splits the heads'
token ranges over every host CPU.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--no-extras]
                    [--variant hamming|minmax|oasis]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode-step µs & keys scored/s at 1M ctx; % of HBM/VALU roofline"
HBM_PEAK_GBS = 8000.0                          # MI355X HBM3E
VALU_PEAK_OPS = 256 * 64 * 2.4e9               # 256 CUs x 64 lanes x 2.4 GHz, one op per lane-cycle
N_COPIES = 8                                   # rotating copies of the plane index (4.6 GB)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fathom_scan_n1M_G8_B56.traffic.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "decode_step_n1M_G8_B56.kernel_trace.txt")
SCAN_SOURCE = os.path.join(ROOT, "sparse_top_decode_query_amd", "csrc", "scan.hip")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--budget", type=int, default=56, help="plane bits per KV head")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the plan variants, the host-resident index and configs 4/5")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 512 MiB device copies (for counter calibration)")
    ap.add_argument("--variant", choices=("hamming", "minmax", "oasis"),
                    help="run only the config 4 (hamming) step, the config 5 (minmax) step or the "
                         "resident-pool step on the config 5 layer, for kernel traces; prints one "
                         "JSON line about that step")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pct(xs, p):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


def scan_traffic(depth_rows_key):
    """HBM bytes per fathom_scan launch from the committed counter summary,
    if it was taken on the current scan source with the same plan."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        with open(SCAN_SOURCE, "rb") as f:
            src = hashlib.sha256(f.read()).hexdigest()
        if kv.get("scan_source_sha256") != src or kv.get("plan_sha256") != depth_rows_key:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def trace_average(path, kernel):
    """Average duration (us) of one kernel in a committed kernel-trace summary."""
    try:
        with open(path) as f:
            for line in f:
                if kernel in line:
                    return float(line.split()[-5])
    except (OSError, ValueError, IndexError):
        pass
    return None


def cpu_model():
    """The host CPU's model name and logical CPU count (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        outp = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in outp.splitlines():
            if line.startswith("Model name:"):
                return f"{line.split(':', 1)[1].strip()}, {os.cpu_count()} logical CPUs"
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return f"{line.split(':', 1)[1].strip()}, {os.cpu_count()} logical CPUs"
    except OSError:
        pass
    return f"unknown, {os.cpu_count()} logical CPUs"


# ------------------------------------------------------------------ CPU oracle
def cpu_baseline(budget, k, min_seconds=10.0, max_passes=50):
    """The CPU oracle's plan + scan + top-k + attention on the same 1M-token
    layer, one KV head at a time; the index is built once, untimed, and
    passes over all KV heads repeat until at least `min_seconds` of timed
    work."""
    import synth
    from oracle import attend as o_attend
    from oracle import fathom as o_fathom
    from oracle import select as o_select
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except ImportError:                                        # pragma: no cover
        limiter = None
    c = synth.CONFIGS[3]
    G, Hgrp = c["G"], c["Hgrp"]
    heads = []
    for g in range(G):
        case = synth.fathom_case(3, heads=[g])
        planes, meta = o_fathom.ingest(case["K"])
        heads.append((case["n"], planes, meta, case["q"][g * Hgrp:(g + 1) * Hgrp],
                      case["var"][g:g + 1], case["K"], case["V"]))
    log("cpu oracle: index built for every KV head")
    timed, keys, passes = 0.0, 0, 0
    stage = {"plan": 0.0, "scan": 0.0, "topk": 0.0, "attend": 0.0}
    while timed < min_seconds and passes < max_passes:
        for n, planes, meta, q, var, K, V in heads:
            t0 = time.perf_counter()
            depth, qbar = o_fathom.plan_heads(q, var, Hgrp, budget=budget)
            t1 = time.perf_counter()
            s = o_fathom.scan_heads(planes, meta, depth, qbar, n)
            t2 = time.perf_counter()
            idx = o_select.topk(s[0], k)
            t3 = time.perf_counter()
            o_attend.attend(q[None], K[None], V[None], idx[None, None])
            t4 = time.perf_counter()
            for name, dt in zip(stage, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
                stage[name] += dt
            timed += t4 - t0
            keys += n
        passes += 1
        log(f"cpu oracle: pass {passes}: {timed:.1f} s timed so far")
    if limiter is not None:
        limiter.unregister()
    single = {
        "value": keys / timed, "unit": "keys/s", "cores": 1, "kind": "oracle",
        "sample": (f"{passes} passes over all {G} KV heads at n=1048576 (4 query heads each, "
                   f"B={budget}, k={k}): plan+scan+top-k+attention per head, fp64 NumPy, one thread; "
                   f"index build untimed; host has {os.cpu_count()} logical CPUs"),
        "seconds": round(timed, 2),
        "stage_ms_per_head": {name: round(v / (passes * G) * 1e3, 2) for name, v in stage.items()},
    }

    # the same work spread over every host CPU: each KV head's token range is
    # cut into 64-token-aligned chunks that score independently (blocks are
    # independent), the chunks run on a thread pool (NumPy releases the
    # interpreter lock in its array loops), then each head's top-k and
    # attention run; wall clock per pass
    import concurrent.futures as cf
    import numpy as np

    workers = os.cpu_count() or 1
    chunks = max(1, -(-workers // G))

    def scan_chunk(arg):
        h, c0, c1 = arg
        n, planes, meta, q, var, K, V = heads[h]
        depth, qbar = o_fathom.plan_heads(q, var, Hgrp, budget=budget)
        return o_fathom.scan(planes[0][:, :, c0 // 32:c1 // 32], meta[0][:, c0 // 64:c1 // 64],
                             depth[0], qbar[0], c1 - c0)

    def finish_head(arg):
        h, s = arg
        n, planes, meta, q, var, K, V = heads[h]
        idx = o_select.topk(s, k)
        o_attend.attend(q[None], K[None], V[None], idx[None, None])
        return n

    wall, keys_p, passes_p = 0.0, 0, 0
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        while wall < min_seconds / 2 and passes_p < max_passes:
            t0 = time.perf_counter()
            tasks = []
            for h, (n, *_rest) in enumerate(heads):
                step = -(-n // (chunks * 64)) * 64
                tasks += [(h, c0, min(n, c0 + step)) for c0 in range(0, n, step)]
            parts = list(ex.map(scan_chunk, tasks))
            rows = {}
            for (h, c0, c1), sc in zip(tasks, parts):
                rows.setdefault(h, []).append(sc)
            keys_p += sum(ex.map(finish_head, [(h, np.concatenate(v)) for h, v in rows.items()]))
            wall += time.perf_counter() - t0
            passes_p += 1
    log(f"cpu oracle, {workers} threads: {passes_p} passes in {wall:.1f} s")
    parallel = {
        "value": keys_p / wall, "unit": "keys/s", "cores": workers, "kind": "oracle",
        "sample": (f"{passes_p} passes over all {G} KV heads as above; each head's scan split into "
                   f"{chunks} token ranges, {G * chunks} scan tasks on {workers} threads, then top-k "
                   f"and attention per head; wall clock"),
        "seconds": round(wall, 2),
        "cpu": cpu_model(),
    }
    single["cpu"] = parallel["cpu"]
    return single, parallel


# ------------------------------------------------------------------ GPU
def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the decode step shards by KV head with no "
              "exchange, so the per-GPU figure is the N=1 line (run without --gpus).",
              file=sys.stderr)
        sys.exit(2)
    if args.variant:
        run_variant(args)
        return

    import numpy as np
    import torch

    import synth
    from sparse_top_decode_query_amd import bytemodel, lib

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    lib.load()                                   # raises if the HIP library is not built
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    c = synth.CONFIGS[3]
    G, Hgrp, n, k, B = c["G"], c["Hgrp"], c["n"], c["k"], args.budget
    t0 = time.time()
    case = synth.fathom_case(3)
    log(f"generated the 1M-token layer in {time.time() - t0:.1f} s")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    K, V = to_dev(case["K"]), to_dev(case["V"])
    q, var = to_dev(case["q"]), to_dev(case["var"])
    index = lib.fathom_ingest(K)
    P = [index.planes] + [index.planes.clone() for _ in range(N_COPIES - 1)]
    M = [index.meta] + [index.meta.clone() for _ in range(N_COPIES - 1)]
    KC = [K.view(1, G, n, 128)] + [K.view(1, G, n, 128).clone() for _ in range(N_COPIES - 1)]
    VC = [V.view(1, G, n, 128)] + [V.view(1, G, n, 128).clone() for _ in range(N_COPIES - 1)]
    depth, qbar = lib.fathom_plan(q, var, B)
    scores = torch.empty(G, n, device=dev)
    bmax = torch.empty(G, n // 64, device=dev)
    gmax = torch.empty(G, lib.n_groups(n), device=dev)
    idx = torch.empty(G, k, dtype=torch.int32, device=dev)
    out = torch.empty(1, G * Hgrp, 128, device=dev)
    ws = lib.attend_workspace(1, G * Hgrp, G, False, k, 1, dev)
    ws_bm = lib.topk_bm_split_workspace(G, n, dev)
    q3, K4, V4, idx3 = q.view(1, G * Hgrp, 128), KC[0], VC[0], idx.view(1, G, k)
    torch.cuda.synchronize()

    def plan_scan(i):
        # plan + scan in one launch (each scan workgroup derives its head's plan)
        lib.fathom_plan_scan(index, q, var, B, n, planes=P[i % N_COPIES], meta=M[i % N_COPIES],
                             scores=scores, block_max=bmax, write_plan=False, group_max=gmax)

    def step(i, ev=None):
        # ev (4 events) brackets every stage: used only by the stage breakdown
        if ev:
            ev[0].record()
        plan_scan(i)
        if ev:
            ev[1].record()
        lib.topk_select_block_max_split(scores, bmax, k, idx=idx, ws=ws_bm, group_max=gmax)
        if ev:
            ev[2].record()
        lib.gather_attend(q3, KC[i % N_COPIES], VC[i % N_COPIES], idx3, out=out, ws=ws)
        if ev:
            ev[3].record()

    # warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, captured into one HIP graph (a decode
    # loop replays its captured step; a Python call per kernel costs about
    # as much host time as the step's GPU time) and replayed once between two
    # events, after one untimed replay.  The replayed step is checked against
    # the same step run eagerly.
    Ksteps = args.steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(Ksteps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    out_graph, idx_graph = out.clone(), idx.clone()
    step(Ksteps - 1)
    torch.cuda.synchronize()
    if not (torch.equal(out_graph, out) and torch.equal(idx_graph, idx)):
        raise SystemExit("graph replay of the decode step differs from the eager step")
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e_start.record()
    graph.replay()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e_start.elapsed_time(e_end) / Ksteps
    del graph
    # the same K steps launched eagerly from Python, one call per kernel (context)
    t_host = time.perf_counter()
    e_start.record()
    for i in range(Ksteps):
        step(i)
    t_enqueue = time.perf_counter() - t_host
    e_end.record()
    torch.cuda.synchronize()
    ms_per_step_eager = e_start.elapsed_time(e_end) / Ksteps
    step_us = []
    for a in range(max(1, Ksteps // 10)):
        step_us.append(timeit_graph(torch, lambda i: step(a * 10 + i), reps=10, warm=0))

    # the dominant launch alone, back to back over the rotating copies (the
    # figure a kernel trace averages); and its fixed cost: the same launch with
    # an empty plan (budget 0) over one 64-token block per KV head, i.e.
    # dispatch, the plan and the drain, with nothing to stream
    scan_launch_us = timeit_graph(torch, plan_scan, reps=64, warm=5, replays=7)
    sc_small = torch.empty(G, 64, device=dev)
    bm_small = torch.empty(G, 1, device=dev)
    gm_small = torch.empty(G, 1, device=dev)
    scan_fixed_us = timeit_graph(torch, lambda i: lib.fathom_plan_scan(
        index, q, var, 0, 64, scores=sc_small, block_max=bm_small, write_plan=False, group_max=gm_small),
        reps=64, warm=5)
    del sc_small, bm_small, gm_small

    # stage breakdown in a separate pass with every stage bracketed (context:
    # the extra events lengthen these steps)
    K2 = min(Ksteps, 50)
    evs2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K2)]
    for i in range(K2):
        step(i, evs2[i])
    torch.cuda.synchronize()
    stage_us = {name: statistics.mean(e[a].elapsed_time(e[a + 1]) * 1e3 for e in evs2)
                for a, name in enumerate(("plan_scan", "topk", "attend"))}

    # roofline of the scan from the actual plan
    d_rows = depth.cpu().numpy()
    plan_key = hashlib.sha256(d_rows.tobytes()).hexdigest()
    scan_bytes = bytemodel.plane_scan_bytes(n, d_rows)
    scan_ops = bytemodel.plane_scan_bit_ops(n, d_rows)
    scan_s = scan_launch_us * 1e-6
    t_hbm = scan_bytes / (HBM_PEAK_GBS * 1e9)
    t_valu = scan_ops / VALU_PEAK_OPS
    achieved_gbs = scan_bytes / scan_s / 1e9
    roofline = {
        "bound": "hbm" if t_hbm >= t_valu else "alu",
        "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "traffic": scan_traffic(plan_key),
        "kernel": "fathom_plan_scan", "bytes_per_launch": scan_bytes,
        "launch_us": round(scan_launch_us, 2),
        "launch_timing": "mean of 64 back-to-back launches (a replayed HIP graph) over the 8 rotating index copies, median of 7 replays",
        "trace_avg_us": trace_average(TRACE_FILE, "fathom_scan_kernel<1, false>"),
        "floor_us": round(max(t_hbm, t_valu) * 1e6, 2),
        "frac_of_binding_floor": round(max(t_hbm, t_valu) / scan_s, 4),
        "fixed_cost_us": round(scan_fixed_us, 2),
        "fixed_cost": "the same launch with budget 0 over 64 tokens per KV head (dispatch, plan, drain)",
        "frac_excluding_fixed_cost": round(scan_bytes / ((scan_launch_us - scan_fixed_us) * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
    }
    # the published peak is the roofline's; beside it, what plain streaming
    # kernels reach on this machine
    hbm_meas = hbm_microbench(torch, dev)
    roofline["measured_hbm"] = hbm_meas
    # the scan reads and writes (76 MB read, 34 MB of scores written at
    # B = 56), a mix closest to a copy's
    roofline["frac_of_measured_copy"] = round(achieved_gbs / hbm_meas["copy_GBps"], 4)
    roofline_valu = {
        "bound": "alu", "achieved": round(scan_ops / scan_s / 1e12, 3),
        "peak": round(VALU_PEAK_OPS / 1e12, 1), "unit": "Tops/s (plane-bit accumulates)",
        "frac": round(scan_ops / scan_s / VALU_PEAK_OPS, 4), "ops_per_launch": scan_ops,
    }
    # the plain scan (plan read from a fathom_plan launch) as context
    plain_us = timeit_graph(torch, lambda i: lib.fathom_scan(index, depth, qbar, n, planes=P[i % N_COPIES],
                                                             meta=M[i % N_COPIES], scores=scores,
                                                             block_max=bmax, group_max=gmax),
                            reps=64, warm=5, replays=7)
    plan_us = timeit_graph(torch, lambda i: lib.fathom_plan(q, var, B, depth=depth, qbar=qbar), reps=64, warm=5,
                           replays=7)
    roofline_plain = {"kernel": "fathom_scan (plan read)", "launch_us": round(plain_us, 2),
                      "frac": round(scan_bytes / (plain_us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
                      "fathom_plan_launch_us": round(plan_us, 2)}
    plan_bits = int(d_rows.sum())
    active = int((d_rows > 0).sum())
    log(f"step {ms_per_step * 1e3:.1f} us; stages {stage_us}; scan {scan_launch_us:.2f} us "
        f"({achieved_gbs:.0f} GB/s), fixed {scan_fixed_us:.2f} us")

    extras = {}
    if not args.no_extras:
        extras = run_extras(torch, np, lib, bytemodel, synth, dev, case, K4, V4, q, var, q3, index,
                            P, M, n, G, Hgrp, k, args.no_cpu)
    if args.copy_calibration:
        extras["copy_calibration_bytes"] = copy_calibration(torch, dev)

    cpu = cpu_all = None
    if not args.no_cpu:
        cpu, cpu_all = cpu_baseline(B, k)

    keys = n * G
    result = {
        "metric": METRIC,
        "value": keys / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": Ksteps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"bit-plane decode step, 1 layer: {G} KV heads x {Hgrp} query heads, d=128, "
                         f"n={n} tokens, read plan B={B} plane bits/KV head, k={k}, index in HBM"),
            "n": n, "kv_heads": G, "q_heads": G * Hgrp, "budget_bits": B, "k": k,
            "plan_bits_total": plan_bits, "active_channels_total": active,
            "plan_sha256": plan_key,
        },
        "roofline": roofline,
        "roofline_valu": roofline_valu,
        "roofline_plain_scan": roofline_plain,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "step_us": {"mean": round(ms_per_step * 1e3, 2), "p10": round(pct(step_us, 10), 2),
                    "p50": round(pct(step_us, 50), 2), "p90": round(pct(step_us, 90), 2),
                    "timing": "one replay of the K steps captured in a HIP graph; p10/p50/p90 over "
                              "replays of 10-step graphs"},
        "step_us_eager": {"mean": round(ms_per_step_eager * 1e3, 2),
                          "host_enqueue_us_per_step": round(t_enqueue / Ksteps * 1e6, 2),
                          "timing": "the same K steps launched from Python one kernel at a time"},
        "stage_us": {k_: round(v, 2) for k_, v in stage_us.items()},
        "keys_scored_per_s_scan": keys / scan_s,
        "host_wall_s_timed_region": round(wall, 4),
        "extras": extras,
    }
    print(json.dumps(result), flush=True)


def timeit(torch, fn, reps=30, warm=3, cover=None):
    """Mean GPU time per call between two events.  For calls shorter than
    their host-side launch cost, ``cover`` (a callable) first queues a long
    GPU operation, so that every timed call is already queued when the first
    one starts and the events measure the calls back to back."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if cover is not None:
        cover()
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def timeit_graph(torch, fn, reps=30, warm=3, replays=1):
    """Mean GPU time per call of `reps` calls captured into one HIP graph and
    replayed between two events (the median over `replays` replays).  A
    replay launches every captured kernel from the device-side graph, so
    calls shorter than their host-side launch cost (a Python call through
    ctypes) are timed back to back, as a decode loop replaying a captured
    step runs them.  The calls must allocate nothing and must not
    synchronise."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()                                   # untimed first replay
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return statistics.median(times)


def run_extras(torch, np, lib, bytemodel, synth, dev, case, K4, V4, q, var, q3, index, P, M, n, G,
               Hgrp, k, no_cpu=False):
    """Context numbers: other read plans, the offloaded-index step, configs 1, 2, 4 and 5."""
    ex = {}
    c = synth.CONFIGS[3]
    scores = torch.empty(G, n, device=dev)
    bmax = torch.empty(G, n // 64, device=dev)
    for B in list(c["budgets"]) + [None]:
        if B is None:
            depth, qbar = lib.fathom_plan(q, var, 0, uniform_channels=c["uniform_channels"])
            name = f"uniform_{c['uniform_channels']}x4"
        else:
            depth, qbar = lib.fathom_plan(q, var, B)
            name = f"B{B}"
        us = timeit_graph(torch, lambda i: lib.fathom_scan(index, depth, qbar, n, planes=P[i % len(P)],
                                                           meta=M[i % len(M)], scores=scores, block_max=bmax))
        d_rows = depth.cpu().numpy()
        nbytes = bytemodel.plane_scan_bytes(n, d_rows)
        ex[f"scan_{name}"] = {"us": round(us, 2), "bytes": nbytes,
                              "hbm_frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
                              "valu_frac": round(bytemodel.plane_scan_bit_ops(n, d_rows) / (us * 1e-6) / VALU_PEAK_OPS, 4)}
        log(f"extras: scan {name} {us:.1f} us")
    ws_t = lib.topk_workspace(G, n, k, lib.SDQ_KEY_F32_MAX, dev)
    idx = torch.empty(G, k, dtype=torch.int32, device=dev)
    ex["topk_select_generic_us"] = round(timeit_graph(torch, lambda i: lib.topk_select(scores, k, idx=idx, ws=ws_t)), 2)

    # offloaded index (the config's second mode): the planes and metadata sit
    # in pinned host memory; each step plans, gathers the plan's active
    # prefixes into an HBM staging copy on a side stream (ordered by events),
    # then scans the staged copy, selects and attends
    ex["offload_step"] = offload_steps(torch, lib, bytemodel, dev, index, q, var, q3, K4, V4, n, G,
                                       Hgrp, k, c)
    torch.cuda.empty_cache()

    # host-resident K/V rows: attention reads the k selected rows of every KV
    # head in place over the host link (this step's own top-k output)
    lib.topk_select_block_max(scores, bmax, k, idx=idx)
    Kh = torch.empty(K4.shape, dtype=K4.dtype, pin_memory=True)
    Vh = torch.empty(V4.shape, dtype=V4.dtype, pin_memory=True)
    Kh.copy_(K4)
    Vh.copy_(V4)
    out = torch.empty(1, G * Hgrp, 128, device=dev)
    ws_a = lib.attend_workspace(1, G * Hgrp, G, False, k, 1, dev)
    torch.cuda.synchronize()
    idx3 = idx.view(1, G, k)
    us = timeit_graph(torch, lambda i: lib.gather_attend_host_kv(q3, Kh, Vh, idx3, out=out, ws=ws_a), reps=10, warm=2)
    us_dev = timeit_graph(torch, lambda i: lib.gather_attend(q3, K4, V4, idx3, out=out, ws=ws_a), reps=10, warm=2)
    moved = bytemodel.attend_bytes(k, G)
    ex["offload_attend_k512"] = {"us": round(us, 1), "bytes": moved, "GB_per_s": round(moved / (us * 1e-6) / 1e9, 1),
                                 "device_resident_us": round(us_dev, 1)}
    log(f"extras: host K/V attention {us:.0f} us")
    del Kh, Vh

    # decode-time appends into this layer's cache (rows of n tokens): the new
    # tokens' blocks are quantised again; appending keys already there
    # rewrites the same words, so the index stays as it was
    # (one append is a few microseconds of GPU work, less than its host-side
    # launch cost, so the calls are timed as a replayed graph)
    for m in (1, 64):
        us = timeit_graph(torch, lambda i: lib.fathom_append(K4[0], n - m, m, index), reps=30, warm=5)
        ex[f"fathom_append_{m}tok_us"] = round(us, 2)
    bmin_a = torch.empty(G, n // 16, 128, dtype=torch.int16, device=dev)
    bmax_a = torch.empty_like(bmin_a)
    us = timeit_graph(torch, lambda i: lib.minmax_append(K4[0], n - 1, 1, bmin_a, bmax_a, 16), reps=30, warm=5)
    ex["minmax_append_1tok_us"] = round(us, 2)
    del bmin_a, bmax_a
    log(f"extras: append {ex['fathom_append_1tok_us']} us (1 token), {ex['fathom_append_64tok_us']} us (64)")

    # a whole step at a ragged length (the open block's last 27 slots empty),
    # the last 64 positions kept as the local window
    n_r = n - 27
    sc_r = torch.empty(G, n, device=dev)
    bm_r = torch.empty(G, n // 64, device=dev)
    gm_r = torch.empty(G, lib.n_groups(n), device=dev)
    idx_r = torch.empty(G, k + 64, dtype=torch.int32, device=dev)
    ws_r = lib.attend_workspace(1, G * Hgrp, G, False, k + 64, 1, dev)
    ws_bm = lib.topk_bm_split_workspace(G, n, dev)
    out_r = torch.empty_like(q3)

    def ragged(i):
        lib.fathom_plan_scan(index, q, var, 56, n_r, planes=P[i % len(P)], meta=M[i % len(M)],
                             scores=sc_r, block_max=bm_r, write_plan=False, group_max=gm_r)
        lib.topk_select_block_max_split(sc_r, bm_r, k, n_local=64, idx=idx_r, ws=ws_bm, group_max=gm_r)
        lib.gather_attend(q3, K4, V4, idx_r.view(1, G, -1), out=out_r, ws=ws_r, n=n_r)
    ex["decode_step_ragged_us"] = round(timeit_graph(torch, ragged), 2)
    log(f"extras: ragged step {ex['decode_step_ragged_us']} us")
    del sc_r, bm_r, gm_r, idx_r, ws_r, out_r, ws_bm

    # read-plan quality on this layer: sparse vs dense attention error, needle and
    # exact top-k recall, scan bytes per plan
    from sparse_top_decode_query_amd import quality
    t0 = time.time()
    ex["quality_1M"] = quality.evaluate(K4[0], V4[0], q, var, index, case["needle_pos"], k)
    log(f"extras: plan quality in {time.time() - t0:.1f} s")
    torch.cuda.empty_cache()
    # the 32k-token layer whose lifted keys separate the plans: a sweep of budgets
    # and uniform plans and the equal-error bits against the uniform 136-bit plan
    t0 = time.time()
    qa = quality.run(2, layer="aligned", sweep=True)
    keep = ("plan_bits", "scan_bytes", "mass_mean", "rel_err_mean", "exact_topk_recall", "needle_recall")
    ex["quality_aligned_32k"] = {
        "equal_error": qa["equal_error"], "exact_topk": qa["exact_topk"],
        "plans": {name: {f: row[f] for f in keep} for name, row in qa["plans"].items()}}
    log(f"extras: aligned-layer sweep in {time.time() - t0:.1f} s")
    torch.cuda.empty_cache()

    us_step, us_scan, info = variant_hamming(torch, np, lib, bytemodel, synth, dev, timeit_graph)
    if not no_cpu:
        info["cpu_baseline"] = cpu_baseline_hamming(synth)
    ex["hamming_cfg4"] = info
    log(f"extras: hamming step {us_step:.1f} us")
    torch.cuda.empty_cache()
    us_step, us_scan, info = variant_minmax(torch, np, lib, bytemodel, synth, dev, timeit_graph)
    if not no_cpu:
        info["cpu_baseline"] = cpu_baseline_minmax(synth)
    ex["minmax_cfg5"] = info
    log(f"extras: minmax step {us_step:.1f} us")
    torch.cuda.empty_cache()
    for cfg in (1, 2):
        ex[f"fathom_cfg{cfg}"] = fathom_small_step(torch, np, lib, bytemodel, synth, dev, cfg)
        log(f"extras: config {cfg} step {ex[f'fathom_cfg{cfg}']['step_us']} us")
    ex["oasis_cfg5"] = variant_oasis(torch, np, lib, synth, dev)
    log(f"extras: resident-pool step {ex['oasis_cfg5']['step_us']:.1f} us")
    return ex


def offload_steps(torch, lib, bytemodel, dev, index, q, var, q3, K4, V4, n, G, Hgrp, k, c, reps=6):
    """The offloaded-index step for every read plan of the config: plan ->
    fathom_gather (pinned host -> HBM staging, side stream) -> fathom_scan of
    the staged copy (+ block maxima) -> block-max top-k -> gather attention.
    The gather is the PCIe-bound stage; this time includes the host link and
    is never the headline value."""
    planes_h = torch.empty(index.planes.shape, dtype=index.planes.dtype, pin_memory=True)
    meta_h = torch.empty(index.meta.shape, dtype=index.meta.dtype, pin_memory=True)
    planes_h.copy_(index.planes)
    meta_h.copy_(index.meta)
    stage_p, stage_m = torch.zeros_like(index.planes), torch.zeros_like(index.meta)
    scores = torch.empty(G, n, device=dev)
    bm = torch.empty(G, n // 64, device=dev)
    idx = torch.empty(G, k, dtype=torch.int32, device=dev)
    out = torch.empty_like(q3)
    ws = lib.attend_workspace(1, G * Hgrp, G, False, k, 1, dev)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    res = {}
    plans = [(f"B{B}", B, None) for B in c["budgets"]] + [(f"uniform_{c['uniform_channels']}x4", 0, c["uniform_channels"])]
    for name, B, u in plans:
        depth = torch.empty(G, 128, dtype=torch.uint8, device=dev)
        qbar = torch.empty(G, 128, device=dev)

        def step(i):
            lib.fathom_plan(q, var, B, depth=depth, qbar=qbar, uniform_channels=u)
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
            lib.fathom_gather(planes_h, meta_h, depth, stage_p, stage_m, stream=side)
            ev2 = torch.cuda.Event()
            ev2.record(side)
            main.wait_event(ev2)
            lib.fathom_scan(index, depth, qbar, n, planes=stage_p, meta=stage_m, scores=scores, block_max=bm)
            lib.topk_select_block_max(scores, bm, k, idx=idx)
            lib.gather_attend(q3, K4, V4, idx.view(1, G, k), out=out, ws=ws)
        us = timeit(torch, step, reps=reps, warm=1)
        us_gather = timeit(torch, lambda i: lib.fathom_gather(planes_h, meta_h, depth, stage_p, stage_m),
                           reps=reps, warm=1)
        moved = bytemodel.plane_scan_read_bytes(n, depth.cpu().numpy())
        res[name] = {"step_us": round(us, 1), "gather_us": round(us_gather, 1), "link_bytes": moved,
                     "gather_GB_per_s": round(moved / (us_gather * 1e-6) / 1e9, 1)}
        log(f"extras: offloaded-index step {name}: {us:.0f} us (gather {us_gather:.0f} us)")
    uni = res[f"uniform_{c['uniform_channels']}x4"]["step_us"]
    res["uniform_over_B56_step_time"] = round(uni / res["B56"]["step_us"], 3)
    res["pages_context"] = ("A100, index and KV rows in host memory: 56-bit plan 1.67x faster than "
                            "a 136-bit scan at 1M tokens (Fathom summary, results)")
    del planes_h, meta_h, stage_p, stage_m
    return res


def fathom_small_step(torch, np, lib, bytemodel, synth, dev, cfg):
    """The bit-plane decode step at config 1 (1 KV head, 4096 tokens, B=48,
    k=64) or config 2 (8 KV heads x 4 query heads, 32768 tokens, B=56, k=512):
    fused plan + scan, top-k, gather attention.  Both take the generic top-k:
    the block-max forms need k well below the row's block count, and at 4096
    and 32768 tokens k is 1/64 of the row or more."""
    cc = synth.fathom_case(cfg)
    G, Hgrp, n, k, B = cc["G"], cc["Hgrp"], cc["n"], cc["k"], cc["budget"]
    K = torch.from_numpy(cc["K"].view(np.int16)).to(dev)
    V = torch.from_numpy(cc["V"].view(np.int16)).to(dev)
    q = torch.from_numpy(cc["q"]).to(dev)
    var = torch.from_numpy(cc["var"]).to(dev)
    index = lib.fathom_ingest(K)
    scores = torch.empty(G, n, device=dev)
    bm = torch.empty(G, n // 64, device=dev)
    idx = torch.empty(G, k, dtype=torch.int32, device=dev)
    q3 = q.view(1, G * Hgrp, 128)
    out = torch.empty_like(q3)
    ws = lib.attend_workspace(1, G * Hgrp, G, False, k, 1, dev)
    ws_t = lib.topk_workspace(G, n, k, lib.SDQ_KEY_F32_MAX, dev)
    K4, V4 = K.view(1, G, n, 128), V.view(1, G, n, 128)
    use_bm = n >= 65536                          # never at configs 1 and 2

    def step(i):
        lib.fathom_plan_scan(index, q, var, B, n, scores=scores, block_max=bm, write_plan=False)
        if use_bm:
            lib.topk_select_block_max(scores, bm, k, idx=idx)
        else:
            lib.topk_select(scores, k, idx=idx, ws=ws_t)
        lib.gather_attend(q3, K4, V4, idx.view(1, G, k), out=out, ws=ws)
    us = timeit_graph(torch, step, reps=50, warm=5)
    us_scan = timeit_graph(torch, lambda i: lib.fathom_plan_scan(index, q, var, B, n, scores=scores, block_max=bm,
                                                                 write_plan=False), reps=50, warm=5)
    d_rows = lib.fathom_plan(q, var, B)[0].cpu().numpy()
    nbytes = bytemodel.plane_scan_bytes(n, d_rows)
    return {"step_us": round(us, 2), "keys_scored_per_s_step": n * G / (us * 1e-6),
            "plan_scan_us": round(us_scan, 2), "scan_bytes": nbytes,
            "scan_hbm_frac": round(nbytes / (us_scan * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "shape": f"G={G} x H_grp={Hgrp}, n={n}, B={B}, k={k}"}


def cpu_baseline_hamming(synth, heads=8):
    """The CPU oracle's Hamming step (distances, top-512 + 128 sink + 128
    local, attention per query head) on `heads` of the 32 query heads of
    config 4, one thread."""
    from oracle import attend as o_attend
    from oracle import hamming as o_hamming
    from oracle import select as o_select
    h = synth.hamming_case(4)
    t0 = time.perf_counter()
    for hh in range(heads):
        d = o_hamming.distances(h["sigs"][hh], h["qsig"][hh])
        idx = o_select.topk(d, h["m"], False, h["sink"], h["local"])
        o_attend.attend(h["q"][None, hh:hh + 1], h["K"][None, hh // 4:hh // 4 + 1],
                        h["V"][None, hh // 4:hh // 4 + 1], idx[None, None], per_query_head=True)
    dt = time.perf_counter() - t0
    return {"value": h["n"] * heads / dt, "unit": "keys/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of 32 query heads at n={h['n']}: distances, top-k with windows, attention; one thread",
            "seconds": round(dt, 2)}


def cpu_baseline_minmax(synth, rows=8):
    """The CPU oracle's block-summary step (block scores, top 128 + local
    block, attention over 16-row blocks) on `rows` of the 512 (request, KV
    head) rows of config 5, one thread; the summaries are built untimed."""
    from oracle import attend as o_attend
    from oracle import quest as o_quest
    from oracle import select as o_select
    mm = synth.minmax_case(5, R=1)
    n, G, Hg = mm["n"], mm["G"], mm["Hgrp"]
    rows = min(rows, G)
    summ = [o_quest.summaries(mm["K"][0, g], 16) for g in range(rows)]
    t0 = time.perf_counter()
    for g in range(rows):
        mn, mx = summ[g]
        S = o_quest.block_scores(mn, mx, mm["q"][0, g * Hg:(g + 1) * Hg])
        idx = o_select.topk(S, mm["top_blocks"], True, 0, 1)
        o_attend.attend(mm["q"][:, g * Hg:(g + 1) * Hg], mm["K"][:, g:g + 1], mm["V"][:, g:g + 1],
                        idx[None, None], block_tokens=16)
    dt = time.perf_counter() - t0
    return {"value": n * rows / dt, "unit": "keys/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of 512 (request, KV head) rows at n={n}: block scores, top-k, attention; one thread",
            "seconds": round(dt, 2)}


def variant_oasis(torch, np, lib, synth, dev, steps=10, cap=16, drift=0.25):
    """Resident-pool decode on the batched min/max layer (64 requests x 8 KV
    heads, 16384 tokens in 16-token blocks): the full K/V stays in pinned host
    memory, the GPU holds the summaries and a pool of 129 blocks per KV head.
    Each step: block scan under the draft query (the query plus a seeded
    N(0, drift^2) perturbation) -> top 128 + the local block -> selection
    against the pool (at most `cap` fetches per KV head) -> fetch over the host
    link -> the normal and draft queries attend over the pool in one call."""
    mm = synth.minmax_case(5)
    R, Gm, nm, Hg, kb = mm["R"], mm["G"], mm["n"], mm["Hgrp"], mm["top_blocks"]
    rows, nbk, S = R * Gm, nm // 16, kb + 1
    Kh = torch.from_numpy(mm["K"].reshape(rows, nm, 128).view(np.int16)).pin_memory()
    Vh = torch.from_numpy(mm["V"].reshape(rows, nm, 128).view(np.int16)).pin_memory()
    bmin, bmax = lib.minmax_summarize(Kh.to(dev), 16)
    q = torch.from_numpy(mm["q"]).to(dev)
    g = np.random.default_rng(synth.seed_of(5) + 1)
    drafts = [q + drift * torch.from_numpy(g.standard_normal(mm["q"].shape, dtype=np.float32)).to(dev)
              for _ in range(steps + 1)]
    # the projection hands attention the normal and draft rows already stacked
    stacked = [lib.stacked_layout(q, dq, Gm) for dq in drafts]
    out_s = torch.empty(R, 2 * Gm * Hg, 128, device=dev)
    pool = lib.BlockPool(rows, S, dev)
    Kp = torch.zeros(rows, S * 16, 128, dtype=torch.int16, device=dev)
    Vp = torch.zeros_like(Kp)
    sc = torch.empty(rows, nbk, device=dev)
    pred = torch.empty(rows, S, dtype=torch.int32, device=dev)
    ws_t = lib.topk_workspace(rows, nbk, kb, lib.SDQ_KEY_F32_MAX, dev)
    ws_a = lib.attend_workspace(R, 2 * Gm * Hg, Gm, False, S, 16, dev)
    # fill the pool from the first draft without a cap (not timed)
    lib.minmax_block_scan(bmin, bmax, drafts[0].reshape(-1, 128), scores=sc)
    lib.topk_select(sc, kb, 0, 1, idx=pred, ws=ws_t)
    ps, pb, nf, slots = lib.oasis_select(pred, sc, pool, 0, S)
    lib.oasis_fetch(Kh, Vh, ps, pb, Kp, Vp, 16)
    torch.cuda.synchronize()
    ps, pb = torch.empty(rows, cap, dtype=torch.int32, device=dev), torch.empty(rows, cap, dtype=torch.int32, device=dev)
    names = ("scan", "topk", "select", "fetch", "attend")
    acc = {k_: 0.0 for k_ in names}
    fetched = hits = misses = 0
    for t in range(1, steps + 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        held = pool.resident.cpu().numpy()
        ev[0].record()
        lib.minmax_block_scan(bmin, bmax, drafts[t].reshape(-1, 128), scores=sc)
        ev[1].record()
        lib.topk_select(sc, kb, 0, 1, idx=pred, ws=ws_t)
        ev[2].record()
        lib.oasis_select(pred, sc, pool, t, cap, plan_slot=ps, plan_block=pb, n_fetch=nf, slots=slots)
        ev[3].record()
        lib.oasis_fetch(Kh, Vh, ps, pb, Kp, Vp, 16)
        ev[4].record()
        lib.attend_stacked(stacked[t], Kp.view(R, Gm, S * 16, 128), Vp.view(R, Gm, S * 16, 128),
                           slots.view(R, Gm, S), 16, out=out_s, ws=ws_a)
        ev[5].record()
        torch.cuda.synchronize()
        for i, k_ in enumerate(names):
            acc[k_] += ev[i].elapsed_time(ev[i + 1]) * 1e3
        fetched += int(nf.sum())
        P = pred.cpu().numpy()
        for r in range(rows):                     # the step's hits and misses, off the clock
            h = len(np.intersect1d(P[r], held[r]))
            hits += h
            misses += S - h
    stage = {k_: round(v / steps, 2) for k_, v in acc.items()}
    per_step = fetched / steps
    return {"step_us": round(sum(stage.values()), 2), "stage_us": stage, "cap_per_kv_head": cap,
            "blocks_fetched_per_step": per_step, "fetch_bytes_per_step": int(per_step * 16 * 256 * 2),
            "pool_hit_rate": round(hits / (hits + misses), 4),
            "misses_left_unfetched_per_step": (misses - fetched) / steps, "drift_sigma": drift,
            "steps": steps}


def setup_hamming(torch, np, lib, synth, dev):
    """Config 4: Hamming signatures -> top-512 + 128 sink + 128 local -> attention
    per query head.  Sixteen copies of the signatures (268 MB) and four of
    K/V rotate between steps, so the last-level cache serves neither.
    Returns (step, parts, h) with parts the individual calls."""
    h = synth.hamming_case(4)
    sig0 = torch.from_numpy(h["sigs"].view(np.int32)).to(dev)
    sigs = [sig0] + [sig0.clone() for _ in range(15)]
    qsig = torch.from_numpy(h["qsig"].view(np.int32)).to(dev)
    K0 = torch.from_numpy(h["K"].view(np.int16)).to(dev)[None]
    V0 = torch.from_numpy(h["V"].view(np.int16)).to(dev)[None]
    Ks = [K0] + [K0.clone() for _ in range(3)]
    Vs = [V0] + [V0.clone() for _ in range(3)]
    qh = torch.from_numpy(h["q"]).to(dev)[None]
    dist = torch.empty(h["H"], h["n"], dtype=torch.uint8, device=dev)
    m_tot = h["m"] + h["sink"] + h["local"]
    idx_h = torch.empty(h["H"], m_tot, dtype=torch.int32, device=dev)
    out_h = torch.empty(1, h["H"], 128, device=dev)
    ws_h = lib.topk_workspace(h["H"], h["n"], h["m"], lib.SDQ_KEY_U8_MIN, dev)
    ws_a = lib.attend_workspace(1, h["H"], h["Hkv"], True, m_tot, 1, dev)

    def scan_topk(i):
        lib.hamming_scan_topk(sigs[i % 16], qsig, h["m"], h["sink"], h["local"], dist=dist, idx=idx_h, ws=ws_h)

    def attend(i):
        lib.gather_attend(qh, Ks[i % 4], Vs[i % 4], idx_h[None], per_query_head=True, out=out_h, ws=ws_a)

    def step(i):
        scan_topk(i)
        attend(i)

    def step_separate(i):
        lib.hamming_scan(sigs[i % 16], qsig, dist=dist)
        lib.topk_select(dist, h["m"], h["sink"], h["local"], idx=idx_h, ws=ws_h)
        attend(i)

    def scan(i):
        lib.hamming_scan(sigs[i % 16], qsig, dist=dist)
    step.separate = step_separate
    return step, {"scan": scan, "scan_topk": scan_topk, "attend": attend}, h


def variant_hamming(torch, np, lib, bytemodel, synth, dev, timeit):
    step, parts, h = setup_hamming(torch, np, lib, synth, dev)
    us_step = timeit(torch, step)
    us_sep = timeit(torch, step.separate)
    us = {name: timeit(torch, fn, reps=40) for name, fn in parts.items()}
    hb = bytemodel.hamming_scan_bytes(h["n"], h["H"])
    m_tot = h["m"] + h["sink"] + h["local"]
    ab = bytemodel.attend_bytes(m_tot, h["H"])
    info = {"step_us": round(us_step, 2), "step_separate_calls_us": round(us_sep, 2),
            "scan_us": round(us["scan"], 2), "scan_topk_us": round(us["scan_topk"], 2),
            "attend_us": round(us["attend"], 2),
            "keys_scored_per_s_step": h["n"] * h["H"] / (us_step * 1e-6),
            "scan_hbm_frac": round(hb / (us["scan"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "scan_topk_hbm_frac": round(hb / (us["scan_topk"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "attend_bytes": ab,
            "attend_hbm_frac": round(ab / (us["attend"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "launch_timing": "back-to-back calls (a replayed HIP graph) over 16 signature copies and 4 K/V copies"}
    return us_step, us["scan"], info


def setup_minmax(torch, np, lib, synth, dev):
    """Config 5: min/max block summaries, 64 requests -> top 128 blocks + the
    local block -> attention over 16-row blocks.  Two copies of the summaries
    (512 MiB) rotate; attention reads 541 MB per step, more than the
    last-level cache holds.  Returns (step, parts, mm)."""
    mm = synth.minmax_case(5)
    R, Gm, nm = mm["R"], mm["G"], mm["n"]
    Km = torch.from_numpy(mm["K"].reshape(R * Gm, nm, 128).view(np.int16)).to(dev)
    Vm = torch.from_numpy(mm["V"].view(np.int16)).to(dev)
    qm = torch.from_numpy(mm["q"]).to(dev)
    summ = [lib.minmax_summarize(Km, 16)]
    summ.append((summ[0][0].clone(), summ[0][1].clone()))
    nbk = nm // 16
    S = torch.empty(R * Gm, nbk, device=dev)
    kb = mm["top_blocks"]
    idx_m = torch.empty(R * Gm, kb + 1, dtype=torch.int32, device=dev)
    out_m = torch.empty(R, Gm * mm["Hgrp"], 128, device=dev)
    ws_m = lib.topk_workspace(R * Gm, nbk, kb, lib.SDQ_KEY_F32_MAX, dev)
    ws_am = lib.attend_workspace(R, Gm * mm["Hgrp"], Gm, False, kb + 1, 16, dev)
    qflat = qm.reshape(-1, 128)
    Kmv = Km.view(R, Gm, nm, 128)

    def scan(i):
        lib.minmax_block_scan(summ[i % 2][0], summ[i % 2][1], qflat, scores=S)

    def topk(i):
        lib.topk_select(S, kb, 0, 1, idx=idx_m, ws=ws_m)

    def attend(i):
        lib.gather_attend(qm, Kmv, Vm, idx_m.view(R, Gm, -1), block_tokens=16, out=out_m, ws=ws_am)

    def step(i):
        scan(i)
        topk(i)
        attend(i)
    return step, {"scan": scan, "topk": topk, "attend": attend}, mm


def variant_minmax(torch, np, lib, bytemodel, synth, dev, timeit):
    step, parts, mm = setup_minmax(torch, np, lib, synth, dev)
    R, Gm, nm, kb = mm["R"], mm["G"], mm["n"], mm["top_blocks"]
    nbk = nm // 16
    us_step = timeit(torch, step, reps=20)
    us = {name: timeit(torch, fn, reps=20) for name, fn in parts.items()}
    mb = bytemodel.minmax_scan_bytes(nbk, R * Gm)
    ab = bytemodel.attend_bytes((kb + 1) * 16, R * Gm)
    info = {"step_us": round(us_step, 2), "scan_us": round(us["scan"], 2),
            "topk_us": round(us["topk"], 2), "attend_us": round(us["attend"], 2),
            "keys_scored_per_s_step": nm * R * Gm / (us_step * 1e-6),
            "scan_hbm_frac": round(mb / (us["scan"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "attend_bytes": ab,
            "attend_hbm_frac": round(ab / (us["attend"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "launch_timing": "back-to-back calls (a replayed HIP graph) over 2 summary copies"}
    return us_step, us["scan"], info


def hbm_microbench(torch, dev, nbytes=1 << 30, reps=10):
    """HBM rates of plain streaming kernels on this machine: a full reduction
    (read), a device copy (read + write) and a fill (write) over 1 GiB
    buffers, two of each alternating (2 GiB, far past the 256 MB last-level
    cache), launched back to back between two events.  The roofline's peak stays the
    published 8 TB/s; these say how much of it a kernel can reach here."""
    n = nbytes // 4
    a = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(2)]
    b = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2)]
    out = torch.empty((), dtype=torch.float32, device=dev)

    def eager(fn):
        # each call is hundreds of microseconds of GPU work, far above its
        # host-side launch cost, so eager launches run back to back (a
        # reduction is not captured into a graph here: it may record memsets)
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    read = eager(lambda i: torch.sum(a[i % 2], dim=0, out=out))
    copy = eager(lambda i: b[i % 2].copy_(a[i % 2]))
    write = eager(lambda i: b[i % 2].zero_())
    del a, b
    return {"read_GBps": round(nbytes / (read * 1e-6) / 1e9, 1),
            "copy_GBps": round(2 * nbytes / (copy * 1e-6) / 1e9, 1),
            "write_GBps": round(nbytes / (write * 1e-6) / 1e9, 1),
            "bytes": nbytes, "kernels": "torch sum (read), copy_ (read + write), zero_ (write)"}


def copy_calibration(torch, dev):
    """A plain elementwise copy of known size (multiply by one: 512 MiB read,
    512 MiB written), for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return src.numel() * 4


def same_size_reference(torch, dev, reps=20):
    """Plain streaming kernels of the Hamming scan's size, for its kernel
    trace: a device copy moving 21 MB (10.5 MB read, 10.5 MB written; the
    distance kernel moves 16.8 MB of signatures read and 4.2 MB of distances
    written) and a 16.8 MB read with a row sum.  Their durations are what a kernel of this size takes once
    launch, ramp and drain are counted."""
    src = torch.ones(2_621_440, dtype=torch.float32, device=dev)      # 10.5 MB each way
    dst = torch.empty_like(src)
    sig = torch.ones(32, 131072, dtype=torch.int32, device=dev)
    out = torch.empty(32, dtype=torch.int64, device=dev)
    for _ in range(reps):
        dst.copy_(src)
        torch.sum(sig, dim=1, out=out)
    torch.cuda.synchronize()
    return {"copy_bytes": src.numel() * 4 * 2, "read_bytes": sig.numel() * 4, "reps": reps}


def run_variant(args):
    """--variant hamming|minmax|oasis: only that step, W warm-up + K steps (the
    resident-pool step fills its pool first, untimed, and times K steps), for
    kernel traces of the variant kernels; prints one JSON line about it."""
    import numpy as np
    import torch
    import synth
    from sparse_top_decode_query_amd import lib
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    lib.load()
    dev = torch.device("cuda:0")
    if args.variant == "oasis":
        info = variant_oasis(torch, np, lib, synth, dev, steps=args.steps)
        print(json.dumps({"variant": "oasis", **info}), flush=True)
        return
    setup = setup_hamming if args.variant == "hamming" else setup_minmax
    step, _, _ = setup(torch, np, lib, synth, dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    line = {"variant": args.variant, "steps": args.steps,
            "us_per_step": round(e0.elapsed_time(e1) / args.steps * 1e3, 2)}
    if args.copy_calibration:
        line["copy_calibration_bytes"] = copy_calibration(torch, dev)
        if args.variant == "hamming":
            line["same_size_reference"] = same_size_reference(torch, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
