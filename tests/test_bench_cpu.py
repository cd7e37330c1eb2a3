"""bench.py contract checks that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_reports_all_cores_and_one_core():
    """The oracle's CPU rate: all cores and one core, each a median of 3 runs."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    wl = synth.make(synth.specs()["tiny"])
    r = bench.cpu_baseline(wl, wl.spec, 0.3, "MXFP4")
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert r["one_core"]["cores"] == 1 and r["one_core"]["value"] > 0
    assert "median of 3" in r["sample"]
