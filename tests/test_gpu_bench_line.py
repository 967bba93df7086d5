"""bench.py's JSON line on the GPU, for the smallest workload in a fresh
process: every field the line promises is there, with sane values, and the
sampled parity is within its bar."""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import announce

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_fields():
    announce("bench line, single 256x128")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                          "single_256x128_fp32", "--steps", "3", "--warmup", "1"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    line = json.loads(out.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "parity", "measured_peaks", "kernels"):
        assert key in line, key
    assert line["unit"] == "ms" and line["value"] > 0 and line["n_gpus"] == 1
    assert (line["steps"], line["warmup"]) == (3, 1) and line["higher_is_better"] is False
    assert line["config"]["workload"] == "single_256x128_fp32"
    roof = line["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert 0 < roof["frac"] < 1 and roof["peak"] > 0
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    par = line["parity"]
    assert par["matrices"] == 1 and 0 < par["max_rel_err_dW"] <= par["bar"]
    peaks = line["measured_peaks"]
    assert peaks["mfma_bf16_tflops"] > 1000 and peaks["copy_gbs"] > 1000
