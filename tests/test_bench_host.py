"""Host-side behaviour of bench.py that needs no GPU: the path is built for
one GPU's expert share, so any other GPU count is refused before torch or
the device is touched; the committed profile records it reads parse."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2
    assert "measures one GPU" in p.stderr
    assert p.stdout == ""


def test_profile_records_parse():
    sys.path.insert(0, ROOT)
    import bench
    for path, tag, field in ((bench.TRACE_FILE, "TRACE ", "avg_launch_us"),
                             (bench.TRAFFIC_FILE, "TRAFFIC ", "fetch_bytes")):
        recs = [json.loads(line[len(tag):]) for line in open(path) if line.startswith(tag)]
        assert len(recs) == 1
        assert len(recs[0]["source_sha256"]) == 64 and recs[0][field] > 0
