"""CPU checks of the benchmark script's surface: it refuses more than one GPU
with a JSON message, and every measurement helper the default and profiling
runs call is present (importing it touches no GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_helpers_present():
    sys.path.insert(0, ROOT)
    import bench
    for name in ("cpu_baseline", "run_extra", "run_gemm", "run_gemm_raster", "hbm_ceiling", "committed_counters",
                 "kernel_source_hash", "main"):
        assert callable(getattr(bench, name)), name
    assert bench.GEMM_DEFAULT in bench.GEMM_VARIANTS
    assert bench.BYTES_PER_STEP == 268435456
