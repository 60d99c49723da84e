"""Short text summaries of rocprofv3 result databases.

    python -m sparse_top_decode_query_amd.profsum kernels DB OUT --command CMD
        per-kernel dispatch count and average / min / max / total duration
        from a `--kernel-trace --stats` run.

    python -m sparse_top_decode_query_amd.profsum traffic FETCH_DB WRITE_DB OUT \
            --kernel fathom_scan --copy-bytes N --plan-sha256 H --command-fetch C1 --command-write C2
        HBM bytes per dispatch of one kernel from two counter runs (FETCH_SIZE,
        then WRITE_SIZE, both in KiB per dispatch).  Each counter is scaled by
        what it reads for a plain elementwise copy of N bytes (a float32
        multiply by one, so N bytes read and N written) in the same run.  The
        output also records the SHA-256 of the scan source and of the plan, so
        a consumer can tell when the figures no longer describe the kernel.

    python -m sparse_top_decode_query_amd.profsum counters OUT DB [DB ...] \
            --kernel fathom_scan --command CMD [--command CMD] [--clocks FILE]
        per-dispatch means of the SQ counters of one or more `--pmc` runs, and
        the rocm-smi clock listing of the box if given.

Reads SQLite only; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import os
import sqlite3
import statistics

_PKG = os.path.dirname(os.path.abspath(__file__))
SCAN_SOURCE = os.path.join(_PKG, "csrc", "scan.hip")


def _short(name: str) -> str:
    return name.split("(")[0]


def kernel_rows(db_path):
    db = sqlite3.connect(db_path)
    return db.execute("select name, duration from kernels order by start").fetchall()


def kernels_summary(db_path, command):
    agg = collections.OrderedDict()
    for name, dur in kernel_rows(db_path):
        agg.setdefault(_short(name), []).append(dur)
    total = sum(sum(v) for v in agg.values()) or 1
    lines = [f"# rocprofv3 kernel trace summary", f"command: {command}", "",
             f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s} {'pct':>6s}"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k[:58]:58s} {len(v):6d} {sum(v) / len(v) / 1e3:9.2f} {min(v) / 1e3:9.2f} "
                     f"{max(v) / 1e3:9.2f} {sum(v) / 1e3:10.1f} {100.0 * sum(v) / total:6.2f}")
    return "\n".join(lines) + "\n"


def counter_per_dispatch(db_path, counter, name_filter):
    """Mean over dispatches of one counter (summed over its instances within
    a dispatch) for kernels whose name contains `name_filter`."""
    db = sqlite3.connect(db_path)
    per = collections.defaultdict(float)
    for disp, kname, value in db.execute(
            "select dispatch_id, kernel_name, value from counters_collection where counter_name = ?",
            (counter,)):
        if name_filter in kname:
            per[disp] += float(value)
    if not per:
        raise SystemExit(f"{db_path}: no {counter} rows for kernels matching {name_filter!r}")
    return statistics.mean(per.values()), len(per)


def traffic_summary(fetch_db, write_db, kernel, copy_bytes, plan_sha, cmd_fetch, cmd_write,
                    source=SCAN_SOURCE):
    copy_tag = "MulFunctor"
    f_k, nf = counter_per_dispatch(fetch_db, "FETCH_SIZE", kernel)
    w_k, nw = counter_per_dispatch(write_db, "WRITE_SIZE", kernel)
    f_c, _ = counter_per_dispatch(fetch_db, "FETCH_SIZE", copy_tag)
    w_c, _ = counter_per_dispatch(write_db, "WRITE_SIZE", copy_tag)
    sf = copy_bytes / (f_c * 1024.0)
    sw = copy_bytes / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * sf
    write_b = w_k * 1024.0 * sw
    with open(source, "rb") as f:
        src_sha = hashlib.sha256(f.read()).hexdigest()
    sha_key = "scan_source_sha256" if os.path.abspath(source) == os.path.abspath(SCAN_SOURCE) \
        else f"source_sha256 ({os.path.relpath(source, _PKG)})"
    return "\n".join([
        f"# HBM traffic of {kernel} per dispatch (rocprofv3 --pmc, two runs)",
        f"command_fetch: {cmd_fetch}",
        f"command_write: {cmd_write}",
        f"kernel: {kernel}",
        f"dispatches_fetch: {nf}",
        f"dispatches_write: {nw}",
        f"fetch_kib_per_dispatch: {f_k:.1f}",
        f"write_kib_per_dispatch: {w_k:.1f}",
        f"copy_bytes: {copy_bytes}",
        f"copy_fetch_kib: {f_c:.1f}",
        f"copy_write_kib: {w_c:.1f}",
        f"fetch_scale: {sf:.4f}",
        f"write_scale: {sw:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"{sha_key}: {src_sha}",
        f"plan_sha256: {plan_sha}",
    ]) + "\n"


def counters_summary(dbs, kernel, commands, clocks_file=None):
    """Per-dispatch means (summed over a dispatch's counter instances) of every
    counter in the given `--pmc` result databases, for one kernel."""
    lines = [f"# rocprofv3 counters of {kernel} per dispatch"]
    lines += [f"command: {c}" for c in commands]
    vals = {}
    for db_path in dbs:
        db = sqlite3.connect(db_path)
        names = [r[0] for r in db.execute("select distinct counter_name from counters_collection")]
        for cn in names:
            mean, nd = counter_per_dispatch(db_path, cn, kernel)
            vals[cn] = (mean, nd)
    lines.append(f"kernel: {kernel}")
    for cn in sorted(vals):
        lines.append(f"{cn}: {vals[cn][0]:.6g}  (dispatches {vals[cn][1]})")
    if "SQ_INSTS_VALU" in vals:
        lines.append(f"valu_lane_ops (SQ_INSTS_VALU x 64): {vals['SQ_INSTS_VALU'][0] * 64:.6g}")
    if "SQ_ACTIVE_INST_VALU" in vals and "SQ_BUSY_CYCLES" in vals:
        lines.append("note: counter meanings as listed by `rocprofv3 --list-avail` on the box")
    if clocks_file and os.path.exists(clocks_file):
        lines.append("")
        lines.append("# rocm-smi --showclocks on the same box")
        with open(clocks_file) as f:
            lines += [l.rstrip() for l in f if l.strip() and not set(l.strip()) <= set("=-")]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("kernels")
    a.add_argument("db")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_db")
    b.add_argument("write_db")
    b.add_argument("out")
    b.add_argument("--kernel", default="fathom_scan")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--plan-sha256", default="-", help="sha256 of the plan the scan ran (scan only)")
    b.add_argument("--source", default="scan.hip", help="the kernel's source file under csrc/")
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernel", default="fathom_scan")
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--clocks", default=None, help="rocm-smi --showclocks output to append")
    args = ap.parse_args(argv)
    if args.cmd == "kernels":
        text = kernels_summary(args.db, args.command)
    elif args.cmd == "counters":
        text = counters_summary(args.dbs, args.kernel, args.command, args.clocks)
    else:
        text = traffic_summary(args.fetch_db, args.write_db, args.kernel, args.copy_bytes,
                               args.plan_sha256, args.command_fetch, args.command_write,
                               os.path.join(_PKG, "csrc", args.source))
    with open(args.out, "w") as f:
        f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
