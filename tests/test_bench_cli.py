"""bench.py's command line without a GPU."""
import subprocess
import sys
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_counts():
    sys.path.insert(0, ROOT)
    import bench
    f, b = bench.counted_flops(2, 32, 8192, 128, True)
    assert f == 4 * 8192 ** 2 * 128 * 64 / 2
    assert b == 2.5 * f
    k = bench.kernel_flops(2, 32, 8192, 128, True)
    assert k["fwd"] == f
    assert k["bwd_dkdv"] + k["bwd_dq"] == 3.5 * f  # 7 products run vs 5 counted
    k64 = bench.kernel_flops(2, 32, 8192, 64, True)
    assert k64["bwd_dkdv"] + k64["bwd_dq"] == 4 * k64["fwd"]  # separate dV and dK kernels at d = 64


def test_cpu_baseline_runs_on_a_small_head():
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    rng = np.random.default_rng(0)
    heads = {n: rng.standard_normal((2, 64, 128)) for n in ("q", "k", "v", "do")}
    cb = bench.cpu_baseline(heads, True)
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
