"""bench.py's command-line contract and its summary helpers, on the CPU:
more than one GPU is refused with a message and a non-zero status before any
GPU work; the per-replay spread reports nearest-rank order statistics."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one MI355X" in r.stderr
    for line in r.stdout.splitlines():                   # no result line
        if line.strip().startswith("{"):
            assert "value" not in json.loads(line)


def test_spread_order_statistics():
    import bench
    xs = [float(v) for v in range(11, 0, -1)]            # 11 .. 1, unsorted input
    s = bench.spread(xs)
    assert s["latency_us_min_median_max"] == [1.0, 6.0, 11.0]
    assert s["latency_us_p10_median_p90"] == [2.0, 6.0, 10.0]
    assert bench.pct(sorted(xs), 0.0) == 1.0 and bench.pct(sorted(xs), 1.0) == 11.0
    one = bench.spread([3.25])
    assert one["latency_us_min_median_max"] == [3.25, 3.25, 3.25]
