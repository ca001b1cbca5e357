"""Host-side checks of bench.py's contract (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_step_statistics_helper():
    sys.path.insert(0, ROOT)
    import bench
    bench._stats("t", [3.0, 1.0, 2.0, 4.0])
    assert bench.STEP_STATS["t"] == {"median_ms": 2.5, "min_ms": 1.0, "max_ms": 4.0, "first_ms": 3.0,
                                     "last_ms": 4.0}
    bench._stats("u", [5.0, 1.0, 3.0])
    assert bench.STEP_STATS["u"]["median_ms"] == 3.0


def test_recorded_traffic_tracks_the_kernel_source():
    """The committed HBM-traffic record names the source file and its hash; bench.py reports
    the figure only while the hash matches."""
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for name, r in rec.items():
        assert os.path.exists(os.path.join(ROOT, r["source"]))
        got = bench.recorded_traffic(name)
        assert got is None or abs(got - r["bytes_per_launch"]) < 1.0


def test_sampled_steps_counts_the_kernel_timed_steps():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.sampled_steps(20) == 2 and bench.sampled_steps(100) == 10 and bench.sampled_steps(3) == 1


def test_bench_does_not_import_the_tests():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert "tests._util" not in src and "from tests" not in src
