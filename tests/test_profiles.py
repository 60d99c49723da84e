"""The committed rocprofv3 summaries (CPU): they parse, every one names the
command that made it, and every traffic summary was taken on the kernel
source that is in the tree now (its SHA-256 matches), so the figures the
bench and the documentation quote describe the current kernels."""
import glob
import hashlib
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_top_decode_query_amd", "csrc")


def _kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


TRAFFIC = sorted(glob.glob(os.path.join(PROFILES, "*.traffic.txt")))
TRACES = sorted(glob.glob(os.path.join(PROFILES, "*.kernel_trace.txt")))
COUNTERS = sorted(glob.glob(os.path.join(PROFILES, "*.counters.txt")))


def test_there_are_summaries():
    assert TRAFFIC and TRACES and COUNTERS


@pytest.mark.parametrize("path", TRAFFIC, ids=os.path.basename)
def test_traffic_summary_matches_current_source(path):
    kv = _kv(path)
    assert "rocprofv3 --pmc FETCH_SIZE" in kv["command_fetch"] and "bench.py" in kv["command_fetch"]
    assert "rocprofv3 --pmc WRITE_SIZE" in kv["command_write"]
    src_keys = [k for k in kv if "sha256" in k and k != "plan_sha256"]
    assert len(src_keys) == 1, src_keys
    key = src_keys[0]
    src = os.path.join(CSRC, "scan.hip") if key == "scan_source_sha256" else \
        os.path.join(os.path.dirname(CSRC), key.split("(", 1)[1].rstrip(")"))
    assert kv[key] == _sha(src), f"{os.path.basename(path)} was taken on another {os.path.basename(src)}"
    # the copy calibration: FETCH_SIZE counts half the bytes read, WRITE_SIZE all written
    assert abs(float(kv["fetch_scale"]) - 2.0) < 0.01 and abs(float(kv["write_scale"]) - 1.0) < 0.01
    assert float(kv["traffic_bytes_per_launch"]) > 0
    assert int(kv["dispatches_fetch"]) > 0 and int(kv["dispatches_write"]) > 0


@pytest.mark.parametrize("path", TRACES, ids=os.path.basename)
def test_kernel_trace_summary_parses(path):
    with open(path) as f:
        lines = f.read().splitlines()
    assert lines[1].startswith("command: rocprofv3 --kernel-trace --stats") and "bench.py" in lines[1]
    rows = [l for l in lines[4:] if l.strip()]
    assert rows
    for l in rows:
        calls, avg, mn, mx, tot = l.split()[-6:-1]
        assert int(calls) > 0 and 0 < float(mn) <= float(avg) <= float(mx)


@pytest.mark.parametrize("path", COUNTERS, ids=os.path.basename)
def test_counter_summary_parses(path):
    kv = _kv(path)
    assert any(k == "command" for k in kv) or open(path).read().count("command: rocprofv3 --pmc") >= 2
    assert int(float(kv["SQ_WAVES"].split()[0])) > 0
    assert float(kv["SQ_INSTS_VALU"].split()[0]) > 0


def test_bench_reads_the_step_trace():
    import sys
    sys.path.insert(0, ROOT)
    import bench
    us = bench.trace_average(bench.TRACE_FILE, "fathom_scan_kernel<1, false>")
    assert us is not None and 10.0 < us < 100.0
