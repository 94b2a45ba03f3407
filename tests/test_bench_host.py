"""Host-side checks of bench.py's contract (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr and r.stdout == ""


def test_traffic_records_are_tied_to_the_kernel_sources():
    import bench
    for which, (path, _) in bench.TRAFFIC.items():
        rec = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    rec[k.strip()] = v.strip()
        assert int(rec["traffic_bytes_per_launch"]) == (int(rec["fetch_bytes_per_launch"])
                                                         + int(rec["write_bytes_per_launch"]))
        # the figure is reported only while the sources match the ones it was measured on
        if rec["source_sha256"] == bench.kernel_source_hash(which):
            assert bench.measured_traffic(which) == int(rec["traffic_bytes_per_launch"])
        else:
            assert bench.measured_traffic(which) is None
