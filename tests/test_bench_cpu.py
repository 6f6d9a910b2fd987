"""bench.py's JSON line and its one-GPU guard, without a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from backward_implicit_gemm_amd import inputs  # noqa: E402


def _line(name):
    wl = next(w for w in inputs.WORKLOADS if w.name == name)
    per_call = {}
    for i in range(len(wl.layers)):
        per_call.update({f"fwd{i + 1}": 50.0, f"dgrad{i + 1}": 60.0, f"wgrad{i + 1}": 55.0})
    floor = {"kernels_per_step": 6, "us_per_step": 12.0, "us_per_kernel": 2.0}
    return wl, bench.report(wl, 0.2, 0.25, per_call, {}, 0.3, floor, 100, 20, None)


def test_report_carries_the_contract_keys():
    wl, line = _line(bench.DEFAULT_WORKLOAD)
    json.dumps(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "ms_per_step_cold", "launch_floor"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["config"]["workload"] == wl.name
    roof = line["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    # the dominant call is the slowest one; fp32 is priced against fp32 MFMA
    assert roof["kernel_call"] == "dgrad1" and roof["bound"] == "mfma" and roof["peak"] == 157.3
    flops = 2 * 1024 * 128 * 3 * 4 * 59 * 5 * 5
    assert abs(roof["achieved"] - flops / 60e-6 / 1e12) < 1e-2
    assert abs(line["value"] - 3 * flops / 0.2e-3 / 1e12) < 1e-2


def test_report_bf16_is_priced_against_hbm():
    _, line = _line("layer1_bf16_relu_b1024")
    assert line["roofline"]["bound"] == "hbm" and line["roofline"]["unit"] == "GB/s"
    assert line["dtype"] == "bf16"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
