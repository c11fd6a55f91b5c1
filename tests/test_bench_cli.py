"""bench.py's command-line contract and its CPU baseline (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU only" in r.stderr and not r.stdout


def test_cpu_baseline_reports_the_oracle():
    sys.path.insert(0, ROOT)
    import bench
    out = bench.cpu_baseline(budget_s=0.5)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1 and "query rows" in out["sample"]
    one = out["single_thread"]
    assert one["value"] > 0 and one["unit"] == "TFLOP/s"
