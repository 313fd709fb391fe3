"""bench.py's host-side pieces, on the CPU: the committed HBM-traffic table it
reads, its source-hash guard, and its refusal of more than one GPU."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ternary_weight_linear_block_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.txt")
sys.path.insert(0, ROOT)


def _rows():
    rows = []
    for ln in open(TRAFFIC):
        if ln.startswith("#") or not ln.strip():
            continue
        rows.append(ln.split())
    return rows


def _sha16(src):
    return hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()[:16]


def test_traffic_table_format():
    rows = _rows()
    assert rows, "no data lines"
    seen = set()
    for r in rows:
        assert len(r) == 5, r
        src, workload, sha, fetch, write = r
        assert os.path.exists(os.path.join(CSRC, src)), src
        assert len(sha) == 16 and int(sha, 16) >= 0
        assert int(fetch) > 0 and int(write) > 0
        assert (src, workload) not in seen
        seen.add((src, workload))
    # the two lines bench.py reports
    assert ("gemm_i8.hip", "prefill_gate_up") in seen
    assert ("gemv.hip", "decode_gate_up_m1") in seen


def test_traffic_for_follows_the_source_hash():
    import bench
    for src, workload, sha, fetch, write in _rows():
        got = bench.traffic_for(src, workload)
        if sha == _sha16(src):
            assert got == float(fetch) + float(write)
        else:
            assert got is None  # counters taken on another version of the kernel
    assert bench.traffic_for("gemm_i8.hip", "no_such_workload") is None


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""
