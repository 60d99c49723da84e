#!/usr/bin/env python3
"""Decode-step benchmark of the sparse attention hot path on one GPU.

The timed step is one decode step of one layer of the bit-plane index at a
1,048,576-token context: 8 KV heads x 4 query heads (GQA), d = 128, a read
plan of B = 56 plane bits per KV head, k = 512 selected rows per KV head:

    fathom_plan -> fathom_scan (+ 64-token block maxima)
                -> topk_select_block_max -> gather_attend

All inputs are seeded synthetic data (synth.fathom_case(3)) resident in HBM
before timing starts.  Eight copies of the plane index rotate between steps
so the 256 MB last-level cache cannot serve the index from one step to the
next (a real decode step reads each layer's index once).

Output: one JSON line.  `value` is keys scored per second over the whole
step (n * G / step time).  `roofline` prices the dominant kernel
(fathom_scan) against HBM: algorithmic bytes per launch (plane-prefix bits,
one scale/offset word per active channel per 64-token block, the fp32 score
write) over its average launch time, measured with HIP events on the stream
the kernels run on.  `roofline_valu` prices the same launches against the
vector ALU (one weighted accumulate per plane bit per token).
`cpu_baseline` is the CPU oracle (fp64 NumPy) timed on the host on the same
1M-token workload, one KV head at a time on one thread;
`cpu_baseline_all_cores` runs the heads on one thread each.

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

    # the same calls with the KV heads in parallel, one thread each (NumPy
    # releases the interpreter lock in its array loops); wall clock per pass
    import concurrent.futures as cf

    def one_head(h):
        n, planes, meta, q, var, K, V = h
        depth, qbar = o_fathom.plan_heads(q, var, Hgrp, budget=budget)
        s = o_fathom.scan_heads(planes, meta, depth, qbar, n)
        idx = o_select.topk(s[0], k)
        o_attend.attend(q[None], K[None], V[None], idx[None, None])
        return n

    workers = min(G, os.cpu_count() or 1)
    wall, keys_p, passes_p = 0.0, 0, 0
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        while wall < min_seconds / 2 and passes_p < max_passes:
            t0 = time.perf_counter()
            keys_p += sum(ex.map(one_head, heads))
            wall += time.perf_counter() - t0
            passes_p += 1
    log(f"cpu oracle, {workers} threads: {passes_p} passes in {wall:.1f} s")
    parallel = {
        "value": keys_p / wall, "unit": "keys/s", "cores": workers, "kind": "oracle",
        "sample": (f"{passes_p} passes over all {G} KV heads as above, the heads on {workers} threads "
                   f"at once (BLAS at its default thread count); wall clock"),
        "seconds": round(wall, 2),
    }
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
    depth, qbar = lib.fathom_plan(q, var, B)
    scores = torch.empty(G, n, device=dev)
    bmax = torch.empty(G, n // 64, device=dev)
    idx = torch.empty(G, k, dtype=torch.int32, device=dev)
    out = torch.empty(1, G * Hgrp, 128, device=dev)
    ws = lib.attend_workspace(1, G * Hgrp, G, False, k, 1, dev)
    q3, K4, V4, idx3 = q.view(1, G * Hgrp, 128), K.view(1, G, n, 128), V.view(1, G, n, 128), idx.view(1, G, k)
    torch.cuda.synchronize()

    def step(i, ev=None):
        # plan + scan in one launch (each scan workgroup derives its head's plan);
        # ev brackets the plan + scan launch, and with 4 entries every stage
        if ev:
            ev[0].record()
        lib.fathom_plan_scan(index, q, var, B, n, planes=P[i % N_COPIES], meta=M[i % N_COPIES],
                             scores=scores, block_max=bmax, write_plan=False)
        if ev:
            ev[1].record()
        lib.topk_select_block_max(scores, bmax, k, idx=idx)
        if ev and len(ev) > 2:
            ev[2].record()
        lib.gather_attend(q3, K4, V4, idx3, out=out, ws=ws)
        if ev and len(ev) > 2:
            ev[3].record()

    # warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps.  A recorded event costs several microseconds of
    # GPU time on this stack, so the dominant launch (plan + scan) is
    # bracketed by events on its stream in every SAMPLE-th step only (its
    # average duration feeds the roofline), and the per-step spread is taken
    # over groups of SAMPLE steps, from one bracketed step to the next.
    Ksteps = args.steps
    SAMPLE = 10
    sampled = list(range(0, Ksteps, SAMPLE))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e_start.record()
    for i in range(Ksteps):
        step(i, evs.get(i))
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = e_start.elapsed_time(e_end) / Ksteps
    step_us = []
    for a, i in enumerate(sampled):
        nxt = evs[sampled[a + 1]][0] if a + 1 < len(sampled) else e_end
        steps_in = (sampled[a + 1] if a + 1 < len(sampled) else Ksteps) - i
        step_us.append(evs[i][0].elapsed_time(nxt) * 1e3 / steps_in)
    scan_launch_us = statistics.mean(evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in sampled)

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
        "floor_us": round(max(t_hbm, t_valu) * 1e6, 2),
        "frac_of_binding_floor": round(max(t_hbm, t_valu) / scan_s, 4),
    }
    roofline_valu = {
        "bound": "alu", "achieved": round(scan_ops / scan_s / 1e12, 3),
        "peak": round(VALU_PEAK_OPS / 1e12, 1), "unit": "Tops/s (plane-bit accumulates)",
        "frac": round(scan_ops / scan_s / VALU_PEAK_OPS, 4), "ops_per_launch": scan_ops,
    }
    plan_bits = int(d_rows.sum())
    active = int((d_rows > 0).sum())
    log(f"step {ms_per_step * 1e3:.1f} us; stages {stage_us}; scan {achieved_gbs:.0f} GB/s")

    extras = {}
    if not args.no_extras:
        extras = run_extras(torch, np, lib, bytemodel, synth, dev, case, K4, V4, q, var, q3, index,
                            P, M, n, G, Hgrp, k)
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
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "step_us": {"mean": round(ms_per_step * 1e3, 2), "p10": round(pct(step_us, 10), 2),
                    "p50": round(pct(step_us, 50), 2), "p90": round(pct(step_us, 90), 2)},
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


def run_extras(torch, np, lib, bytemodel, synth, dev, case, K4, V4, q, var, q3, index, P, M, n, G,
               Hgrp, k):
    """Context numbers: other read plans, the host-resident index, configs 4 and 5."""
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
        us = timeit(torch, lambda i: lib.fathom_scan(index, depth, qbar, n, planes=P[i % len(P)],
                                                     meta=M[i % len(M)], scores=scores, block_max=bmax))
        d_rows = depth.cpu().numpy()
        nbytes = bytemodel.plane_scan_bytes(n, d_rows)
        ex[f"scan_{name}"] = {"us": round(us, 2), "bytes": nbytes,
                              "hbm_frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
                              "valu_frac": round(bytemodel.plane_scan_bit_ops(n, d_rows) / (us * 1e-6) / VALU_PEAK_OPS, 4)}
        log(f"extras: scan {name} {us:.1f} us")
    ws_t = lib.topk_workspace(G, n, k, lib.SDQ_KEY_F32_MAX, dev)
    idx = torch.empty(G, k, dtype=torch.int32, device=dev)
    ex["topk_select_generic_us"] = round(timeit(torch, lambda i: lib.topk_select(scores, k, idx=idx, ws=ws_t)), 2)

    # host-resident index: gather the active prefixes into HBM, then scan
    depth, qbar = lib.fathom_plan(q, var, 56)
    planes_h = torch.empty(index.planes.shape, dtype=index.planes.dtype, pin_memory=True)
    meta_h = torch.empty(index.meta.shape, dtype=index.meta.dtype, pin_memory=True)
    planes_h.copy_(index.planes)
    meta_h.copy_(index.meta)
    stage_p, stage_m = torch.zeros_like(index.planes), torch.zeros_like(index.meta)
    torch.cuda.synchronize()
    moved = bytemodel.plane_scan_read_bytes(n, depth.cpu().numpy())
    us = timeit(torch, lambda i: lib.fathom_gather(planes_h, meta_h, depth, stage_p, stage_m), reps=5, warm=1)
    ex["offload_gather_B56"] = {"us": round(us, 1), "bytes": moved, "GB_per_s": round(moved / (us * 1e-6) / 1e9, 1)}
    log(f"extras: host gather {us:.0f} us")
    del planes_h, meta_h, stage_p, stage_m

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
    us = timeit(torch, lambda i: lib.gather_attend_host_kv(q3, Kh, Vh, idx3, out=out, ws=ws_a), reps=10, warm=2)
    us_dev = timeit(torch, lambda i: lib.gather_attend(q3, K4, V4, idx3, out=out, ws=ws_a), reps=10, warm=2)
    moved = bytemodel.attend_bytes(k, G)
    ex["offload_attend_k512"] = {"us": round(us, 1), "bytes": moved, "GB_per_s": round(moved / (us * 1e-6) / 1e9, 1),
                                 "device_resident_us": round(us_dev, 1)}
    log(f"extras: host K/V attention {us:.0f} us")
    del Kh, Vh

    # decode-time appends into this layer's cache (rows of n tokens): the new
    # tokens' blocks are quantised again; appending keys already there
    # rewrites the same words, so the index stays as it was
    # (one append is a few microseconds of GPU work but about ten of host-side
    # launch cost, so a 2 GiB multiply is queued ahead of the timed calls)
    big = torch.ones(1 << 29, device=dev)
    cover = lambda: big.mul_(1.0)                                   # noqa: E731
    for m in (1, 64):
        us = timeit(torch, lambda i: lib.fathom_append(K4[0], n - m, m, index), reps=30, warm=5,
                    cover=cover)
        ex[f"fathom_append_{m}tok_us"] = round(us, 2)
    bmin_a = torch.empty(G, n // 16, 128, dtype=torch.int16, device=dev)
    bmax_a = torch.empty_like(bmin_a)
    us = timeit(torch, lambda i: lib.minmax_append(K4[0], n - 1, 1, bmin_a, bmax_a, 16), reps=30,
                warm=5, cover=cover)
    ex["minmax_append_1tok_us"] = round(us, 2)
    del bmin_a, bmax_a, big
    log(f"extras: append {ex['fathom_append_1tok_us']} us (1 token), {ex['fathom_append_64tok_us']} us (64)")

    # a whole step at a ragged length (the open block's last 27 slots empty),
    # the last 64 positions kept as the local window
    n_r = n - 27
    sc_r = torch.empty(G, n, device=dev)
    bm_r = torch.empty(G, n // 64, device=dev)
    idx_r = torch.empty(G, k + 64, dtype=torch.int32, device=dev)
    ws_r = lib.attend_workspace(1, G * Hgrp, G, False, k + 64, 1, dev)
    out_r = torch.empty_like(q3)

    def ragged(i):
        lib.fathom_plan_scan(index, q, var, 56, n_r, planes=P[i % len(P)], meta=M[i % len(M)],
                             scores=sc_r, block_max=bm_r, write_plan=False)
        lib.topk_select_block_max(sc_r, bm_r, k, n_local=64, idx=idx_r)
        lib.gather_attend(q3, K4, V4, idx_r.view(1, G, -1), out=out_r, ws=ws_r, n=n_r)
    ex["decode_step_ragged_us"] = round(timeit(torch, ragged), 2)
    log(f"extras: ragged step {ex['decode_step_ragged_us']} us")
    del sc_r, bm_r, idx_r, ws_r, out_r

    # read-plan quality on this layer: sparse vs dense attention error, needle and
    # exact top-k recall, scan bytes per plan
    from sparse_top_decode_query_amd import quality
    t0 = time.time()
    ex["quality_1M"] = quality.evaluate(K4[0], V4[0], q, var, index, case["needle_pos"], k)
    log(f"extras: plan quality in {time.time() - t0:.1f} s")
    torch.cuda.empty_cache()

    us_step, us_scan, info = variant_hamming(torch, np, lib, bytemodel, synth, dev, timeit)
    ex["hamming_cfg4"] = info
    log(f"extras: hamming step {us_step:.1f} us")
    us_step, us_scan, info = variant_minmax(torch, np, lib, bytemodel, synth, dev, timeit)
    ex["minmax_cfg5"] = info
    log(f"extras: minmax step {us_step:.1f} us")
    ex["oasis_cfg5"] = variant_oasis(torch, np, lib, synth, dev)
    log(f"extras: resident-pool step {ex['oasis_cfg5']['step_us']:.1f} us")
    return ex


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
    per query head.  Returns (step, scan, h)."""
    h = synth.hamming_case(4)
    sigs, qsig = torch.from_numpy(h["sigs"].view(np.int32)).to(dev), torch.from_numpy(h["qsig"].view(np.int32)).to(dev)
    Kh = torch.from_numpy(h["K"].view(np.int16)).to(dev)[None]
    Vh = torch.from_numpy(h["V"].view(np.int16)).to(dev)[None]
    qh = torch.from_numpy(h["q"]).to(dev)[None]
    dist = torch.empty(h["H"], h["n"], dtype=torch.uint8, device=dev)
    m_tot = h["m"] + h["sink"] + h["local"]
    idx_h = torch.empty(h["H"], m_tot, dtype=torch.int32, device=dev)
    out_h = torch.empty(1, h["H"], 128, device=dev)
    ws_h = lib.topk_workspace(h["H"], h["n"], h["m"], lib.SDQ_KEY_U8_MIN, dev)
    ws_a = lib.attend_workspace(1, h["H"], h["Hkv"], True, m_tot, 1, dev)

    def step(i):
        lib.hamming_scan_topk(sigs, qsig, h["m"], h["sink"], h["local"], dist=dist, idx=idx_h, ws=ws_h)
        lib.gather_attend(qh, Kh, Vh, idx_h[None], per_query_head=True, out=out_h, ws=ws_a)

    def step_separate(i):
        lib.hamming_scan(sigs, qsig, dist=dist)
        lib.topk_select(dist, h["m"], h["sink"], h["local"], idx=idx_h, ws=ws_h)
        lib.gather_attend(qh, Kh, Vh, idx_h[None], per_query_head=True, out=out_h, ws=ws_a)

    def scan(i):
        lib.hamming_scan(sigs, qsig, dist=dist)
    step.separate = step_separate
    return step, scan, h


def variant_hamming(torch, np, lib, bytemodel, synth, dev, timeit):
    step, scan, h = setup_hamming(torch, np, lib, synth, dev)
    us_step = timeit(torch, step)
    us_sep = timeit(torch, step.separate)
    us_scan = timeit(torch, scan)
    hb = bytemodel.hamming_scan_bytes(h["n"], h["H"])
    info = {"step_us": round(us_step, 2), "step_separate_calls_us": round(us_sep, 2),
            "scan_us": round(us_scan, 2),
            "keys_scored_per_s_step": h["n"] * h["H"] / (us_step * 1e-6),
            "scan_hbm_frac": round(hb / (us_scan * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)}
    return us_step, us_scan, info


def setup_minmax(torch, np, lib, synth, dev):
    """Config 5: min/max block summaries, 64 requests -> top 128 blocks + the
    local block -> attention over 16-row blocks.  Returns (step, scan, mm)."""
    mm = synth.minmax_case(5)
    R, Gm, nm = mm["R"], mm["G"], mm["n"]
    Km = torch.from_numpy(mm["K"].reshape(R * Gm, nm, 128).view(np.int16)).to(dev)
    Vm = torch.from_numpy(mm["V"].view(np.int16)).to(dev)
    qm = torch.from_numpy(mm["q"]).to(dev)
    bmin, bmax_s = lib.minmax_summarize(Km, 16)
    nbk = nm // 16
    S = torch.empty(R * Gm, nbk, device=dev)
    kb = mm["top_blocks"]
    idx_m = torch.empty(R * Gm, kb + 1, dtype=torch.int32, device=dev)
    out_m = torch.empty(R, Gm * mm["Hgrp"], 128, device=dev)
    ws_m = lib.topk_workspace(R * Gm, nbk, kb, lib.SDQ_KEY_F32_MAX, dev)
    ws_am = lib.attend_workspace(R, Gm * mm["Hgrp"], Gm, False, kb + 1, 16, dev)
    qflat = qm.reshape(-1, 128)
    Kmv = Km.view(R, Gm, nm, 128)

    def step(i):
        lib.minmax_block_scan(bmin, bmax_s, qflat, scores=S)
        lib.topk_select(S, kb, 0, 1, idx=idx_m, ws=ws_m)
        lib.gather_attend(qm, Kmv, Vm, idx_m.view(R, Gm, -1), block_tokens=16, out=out_m, ws=ws_am)

    def scan(i):
        lib.minmax_block_scan(bmin, bmax_s, qflat, scores=S)
    return step, scan, mm


def variant_minmax(torch, np, lib, bytemodel, synth, dev, timeit):
    step, scan, mm = setup_minmax(torch, np, lib, synth, dev)
    R, Gm, nm, kb = mm["R"], mm["G"], mm["n"], mm["top_blocks"]
    nbk = nm // 16
    us_step = timeit(torch, step, reps=20)
    us_scan = timeit(torch, scan, reps=20)
    mb = bytemodel.minmax_scan_bytes(nbk, R * Gm)
    info = {"step_us": round(us_step, 2), "scan_us": round(us_scan, 2),
            "keys_scored_per_s_step": nm * R * Gm / (us_step * 1e-6),
            "scan_hbm_frac": round(mb / (us_scan * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "attend_bytes": bytemodel.attend_bytes((kb + 1) * 16, R * Gm)}
    return us_step, us_scan, info


def copy_calibration(torch, dev):
    """A plain elementwise copy of known size (multiply by one: 512 MiB read,
    512 MiB written), for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return src.numel() * 4


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
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
