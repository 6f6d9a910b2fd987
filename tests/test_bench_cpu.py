"""bench.py's JSON line and its one-GPU guard, without a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from backward_implicit_gemm_amd import inputs  # noqa: E402


def _measured(wl, hot=None, cold=None):
    per_call = {}
    n = len(wl.layers)
    for i in range(n):
        per_call.update({f"fwd{i + 1}": 50.0, f"bwd{i + 1}": 100.0, f"dgrad{i + 1}": 60.0,
                         f"wgrad{i + 1}": 55.0})
    floor = {"kernels_per_step": 6, "us_per_step": 12.0, "us_per_kernel": 2.0}
    steps = [f"fwd{i + 1}" for i in range(n)] + [f"bwd{i + 1}" for i in reversed(range(n))]
    return {"ms_step": 0.2, "ms_eager": 0.25, "per_call": hot or per_call,
            "per_call_cold": cold or {k: v + 10.0 for k, v in per_call.items()},
            "bias_us": {}, "ms_cold": 0.3, "floor": floor, "step_calls": steps,
            "ms_step_separate": 0.21}


def _line(name, **kw):
    wl = next(w for w in inputs.WORKLOADS if w.name == name)
    return wl, bench.report(wl, _measured(wl), 100, 20, None, **kw)


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
    # the dominant call is the step's slowest, the one-call backward (both
    # passes' flops); fp32 is priced against fp32 MFMA
    assert roof["kernel_call"] == "bwd1" and roof["bound"] == "mfma" and roof["peak"] == 157.3
    assert roof["kernels"] == ["bwd_fused_f32", "wgrad_reduce"]
    flops = 2 * 1024 * 128 * 3 * 4 * 59 * 5 * 5
    assert abs(roof["achieved"] - 2 * flops / 100e-6 / 1e12) < 1e-2
    assert abs(line["value"] - 3 * flops / 0.2e-3 / 1e12) < 1e-2
    # the separate passes are still reported, each against its own work
    assert abs(line["calls"]["wgrad1"]["frac"] - flops / 55e-6 / 1e12 / 157.3) < 1e-4
    assert line["us_per_iter"]["bwd"] == 100.0 and line["ms_per_step_separate_calls"] == 0.21


def test_report_bf16_is_priced_against_hbm_on_cold_times():
    wl, line = _line("layer1_bf16_relu_b1024")
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and line["dtype"] == "bf16"
    # the backward's algorithmic bytes (dy, y as the mask, x, w read; dx, dw
    # written) over its cold 110 us
    L = wl.layers[0]
    nx, nw, ny = L.B * 59 * 165, 128 * 59 * 25, L.B * 128 * 12
    by = 2 * (2 * ny + 2 * nx + 2 * nw)
    assert roof["kernel_call"] == "bwd1" and roof["us_per_launch"] == 110.0
    assert abs(roof["achieved"] - by / 110e-6 / 1e9) < 1e-2
    # d_input alone: dy, y, w, dx
    by_d = 2 * (2 * ny + nw + nx)
    assert abs(line["calls"]["dgrad1"]["frac_hot"] - by_d / 60e-6 / 1e9 / 8000) < 1e-4


def test_report_carries_other_workloads_and_data_independence():
    others = {}
    for w in inputs.WORKLOADS:
        if w.name != bench.DEFAULT_WORKLOAD:
            others[w.name] = bench.workload_summary(w, _measured(w))
    _, line = _line(bench.DEFAULT_WORKLOAD, others=others, data_ind={"x*8": {}})
    json.dumps(line)
    assert set(line["workloads"]) == {w.name for w in inputs.WORKLOADS} - {bench.DEFAULT_WORKLOAD}
    c = line["workloads"]["layer1_bf16_relu_b1024"]["calls"]
    assert set(c) == {"fwd1", "bwd1", "dgrad1", "wgrad1"} and 0 < c["fwd1"]["frac"] < 1
    assert set(line["workloads"]["chain_bf16_b16384"]["calls"]) == {
        "fwd1", "fwd2", "bwd1", "bwd2", "dgrad1", "dgrad2", "wgrad1", "wgrad2"}
    assert "ms_per_step_separate_calls" in line["workloads"]["chain_bf16_b16384"]
    assert "data_independence" in line


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_copy_fractions_are_added_to_hbm_bound_calls():
    others = {w.name: bench.workload_summary(w, _measured(w))
              for w in inputs.WORKLOADS if w.name != bench.DEFAULT_WORKLOAD}
    _, line = _line(bench.DEFAULT_WORKLOAD, others=others)
    copy = {"gbs": 5000.0, "frac_of_peak": 0.625, "bytes_per_copy": 2 << 30, "us_per_copy": 400.0}
    line = bench.add_copy_fractions(line, copy)
    json.dumps(line)
    assert line["hbm_copy"] == copy
    c = line["workloads"]["layer1_bf16_relu_b1024"]["calls"]["fwd1"]
    assert abs(c["frac_copy"] - c["frac"] * 8000.0 / 5000.0) < 1e-3
    # fp32 calls are priced against MFMA and get no copy fraction
    assert "frac_copy" not in line["calls"]["wgrad1"]
    assert "frac_copy" not in line["workloads"]["layer2_fp32_b1024"]["calls"]["fwd1"]


def test_step_call_kernels_follow_the_backward_plan():
    # the launch floor and the roofline's kernel list count what gc_conv_bwd runs
    by = {w.name: w for w in inputs.WORKLOADS}
    assert bench.call_kernels(by["layer1_fp32_relu_b1024"], "bwd1") == ["bwd_fused_f32", "wgrad_reduce"]
    assert bench.call_kernels(by["layer2_bf16_b1024"], "bwd1") == [
        "bwd_prep_bf16", "bwd_fused_bf16", "wgrad_reduce"]
    assert bench.call_kernels(by["layer1_bf16_relu_b1024"], "bwd1") == [
        "bwd_prep_bf16", "dgrad_ig_bf16", "wgrad_ws_bf16", "wgrad_reduce"]
    assert bench.call_kernels(by["layer1_fp32_relu_b1024"], "fwd1") == ["pack_w_fwd_f32", "fwd_ws_f32"]


def test_bf16_calls_carry_their_same_bytes_copy():
    wl = next(w for w in inputs.WORKLOADS if w.name == "layer1_bf16_relu_b1024")
    m = _measured(wl)
    by = bench.call_work(wl)["fwd1"][1]
    m["same_copy"] = {"fwd1": {"us_hot": 4.0, "us_cold": 6.0, "bytes": by}}
    c = bench.workload_summary(wl, m)["calls"]
    cp = c["fwd1"]["same_bytes_copy"]
    json.dumps(c)
    # the copy's bytes over its cold time against 8 TB/s, and the call's cold
    # 60 us against the copy's 6 us
    assert abs(cp["frac"] - by / 6e-6 / 1e9 / 8000) < 1e-4
    assert abs(c["fwd1"]["frac_of_same_bytes_copy"] - 6.0 / 60.0) < 1e-4
    # calls without a copy measurement carry no such keys
    assert "same_bytes_copy" not in c["dgrad1"]


def test_short_calls_get_more_cold_copies():
    # the cold time is a difference of two graph timings divided by the copy
    # count: short calls are given more copies
    assert bench.cold_reps(10.0) == 16 and bench.cold_reps(29.9) == 16
    assert bench.cold_reps(30.0) == 4 and bench.cold_reps(500.0) == 4
