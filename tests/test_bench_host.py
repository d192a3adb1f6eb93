"""Host-side checks of bench.py: its one-GPU contract and the CPU baseline leg
(the oracle timed on a row sample).  No GPU is touched."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus, "--steps", "1"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bench_cpu_baseline_reports_the_oracle_sample():
    sys.path.insert(0, ROOT)
    import bench
    res = bench.cpu_baseline(1.2)
    json.dumps(res)
    assert {"value", "unit", "cores", "kind", "sample"} <= set(res)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["value"] > 0 and res["cores"] >= 1 and res["cpu_model"]
    assert "K=4096, N=14336" in res["sample"]
    # both halves of the metric, on all threads and on one
    for key in ("gemm_f64_TFLOPs", "gemm_f32_naive_TFLOPs", "quant_GBps", "dequant_GBps",
                "gemm_f64_TFLOPs_1thread", "quant_GBps_1thread", "dequant_GBps_1thread"):
        assert res["parts"][key] > 0, key
