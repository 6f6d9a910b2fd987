"""Benchmark: convolution forward + d_input + wgrad through libgc's C ABI.

One step is one pass of the whole path over one batch -- forward (with the
fused ReLU where the layer has one), d_input and wgrad -- on synthetic seeded
inputs already resident in HBM.  The default workload is the policy
network's layer 1 in fp32 at B=1024 (59->128 channels, 11x15 input, 5x5
kernel, stride 3, ReLU), as benchmarked in "Speedups to gemm_conv_forward and
gemm_conv_backward kernels" (PufferLib pull request #522), which times
forward and backward separately over 50 warmup and 200 timed iterations.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]

Prints one JSON line per workload: throughput in TFLOP/s of algorithmic work
(2*B*OC*OH*OW*IC*KH*KW per pass, three passes per step) over K steps, each
step replayed as one HIP graph between HIP events on the launch stream; the
same K steps issued eagerly (host work included); the step timed cold
(caches flushed by a 640 MB write before each replay); the launch floor (a
graph of as many one-element kernels as a step launches); per-call GPU times
from graphs of back-to-back copies of each call; the backward through
gc_conv_bwd (d_input and wgrad in one call) per call and as a step; a roofline entry for the
dominant call; and the CPU oracle timed on this host on a bounded sample
(default workload only).
"""
import argparse
import hashlib
import glob
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv fwd+bwd µs/iter and TFLOP/s at B=1024 (layer1/layer2, fp32/bf16)"
DEFAULT_WORKLOAD = "layer1_fp32_relu_b1024"

# MI355X published peaks.
PEAK = {"mfma_f32": 157.3, "mfma_bf16": 2500.0, "hbm_gbs": 8000.0}

# Page 1's fast kernels (gemm_fast), unnamed NVIDIA GPU, microseconds per
# iteration for forward and for backward (wgrad + d_input): context only.
PAGE1_US = {
    "layer1_fp32_relu_b1024": (192.4102, 541.7361),
    "layer2_fp32_b1024": (56.8698, 100.2875),
    "layer1_bf16_relu_b1024": (106.4277, 403.5356),
    "layer2_bf16_b1024": (18.4427, 49.1440),
}

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true", help="every workload, one line each")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle leg")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run a device copy of this many MB (fp32 multiply by 1), the "
                         "known-size reference for HBM byte counters")
    return ap.parse_args()


def layer_flops(L):
    return 2.0 * L.B * L.OC * L.OH * L.OW * L.IC * L.KH * L.KW


def layer_bytes(L, esize):
    """Algorithmic bytes: each tensor read once, each output written once."""
    nx = L.B * L.IC * L.H * L.W
    nw = L.OC * L.IC * L.KH * L.KW
    ny = L.B * L.OC * L.OH * L.OW
    fwd = (nx + nw + ny) * esize
    dgrad = (ny + (ny if L.relu else 0) + nw + nx) * esize
    wgrad = (nx + ny + (ny if L.relu else 0) + nw) * esize
    return {"fwd": fwd, "dgrad": dgrad, "wgrad": wgrad}


def source_digest():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "backward_implicit_gemm_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, op):
    """HBM bytes per call from the committed rocprofv3 counter summary (the
    first ```json block of profiles/traffic.md), if it was taken on the
    current kernel sources; else None."""
    try:
        text = open(PROFILE_TRAFFIC).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        t = json.loads(block)
    except (OSError, ValueError, IndexError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    e = t.get("entries", {}).get(f"{workload}/{op}")
    return None if e is None else e.get("bytes_per_launch")


def run_gpu(wl, steps, warmup):
    import torch

    from backward_implicit_gemm_amd import binding as gb
    from backward_implicit_gemm_amd import inputs

    dev = torch.device("cuda:0")
    td = inputs.torch_dtype(wl.dtype)
    t = inputs.workload_inputs(wl)
    layers = wl.layers
    convs = [gb.Conv(L.x_shape, L.w_shape, L.stride, L.relu, td, dev) for L in layers]
    if len(layers) == 1:
        xs = [t["x"].to(dev)]
        ws = [t["w"].to(dev)]
    else:
        xs = [t["x"].to(dev), None]
        ws = [t["w1"].to(dev), t["w2"].to(dev)]
    ys = [torch.empty(L.y_shape, dtype=td, device=dev) for L in layers]
    if len(layers) == 2:
        xs[1] = ys[0]
    dys = [None] * len(layers)
    dys[-1] = t["dy"].to(dev)
    for i in range(len(layers) - 1):
        dys[i] = torch.empty(layers[i].y_shape, dtype=td, device=dev)
    dxs = [torch.empty(L.x_shape, dtype=td, device=dev) if i == 0 else dys[i - 1]
           for i, L in enumerate(layers)]
    dws = [torch.empty(L.w_shape, dtype=td, device=dev) for L in layers]

    # calls of one step, in order: forward through the layers, then backward
    calls = []
    for i, c in enumerate(convs):
        calls.append((f"fwd{i + 1}", lambda c=c, i=i: c.fwd(xs[i], ws[i], ys[i])))
    for i in reversed(range(len(convs))):
        c = convs[i]
        calls.append((f"dgrad{i + 1}", lambda c=c, i=i: c.bwd_data(dys[i], ws[i], ys[i], dxs[i])))
        calls.append((f"wgrad{i + 1}", lambda c=c, i=i: c.bwd_weight(xs[i], dys[i], ys[i], dws[i])))

    def step():
        for _, f in calls:
            f()

    # Eager warmup: plans, LDS attributes and the library's lazy set-up are
    # settled before capture, so the graphs hold kernel launches only.
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()

    # One step as a HIP graph: replaying it issues the step's kernels without
    # the per-call host work (argument checks, ctypes marshalling), which at
    # these sizes is comparable to the kernels themselves.
    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        step()
    for _ in range(warmup):
        step_graph.replay()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step_graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps

    # Cold protocol: before each timed step, write 640 MB (more than the
    # 256 MB MALL and every XCD's L2 together) so the step starts from HBM.
    flush = torch.empty(640 << 20, dtype=torch.uint8, device=dev)
    cold_n = max(3, min(20, steps // 10))
    cold_ms = 0.0
    for _ in range(cold_n):
        flush.fill_(1)
        start.record(stream)
        step_graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        cold_ms += start.elapsed_time(end)
    ms_cold = cold_ms / cold_n
    del flush

    # Launch floor: the same number of kernels as one step, each a one-element
    # add, replayed as a graph; the least time a step of that many dependent
    # launches can take.
    nk = sum(len(CALL_KERNELS[name.rstrip("0123456789")][wl.dtype]) for name, _ in calls)
    tiny = torch.zeros(1, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(nk):
            tiny.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    floor = {"kernels_per_step": nk, "us_per_step": round(start.elapsed_time(end) / steps * 1e3, 3)}
    floor["us_per_kernel"] = round(floor["us_per_step"] / nk, 3)
    del g

    # The same steps issued eagerly through the C ABI, host work included.
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / steps

    # Per call: a graph of REPS back-to-back copies of the call, replayed and
    # timed with HIP events on the launch stream, so each figure is the
    # call's GPU time (its kernels plus the gaps between graph nodes).
    reps = 10
    replays = max(2, min(20, steps // reps))
    per_call = {}
    for name, f in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        per_call[name] = start.elapsed_time(end) / (replays * reps) * 1e3
        del g

    # The whole backward of each layer through gc_conv_bwd (one call for
    # d_input and wgrad; fewer launches where a fused plan exists), per call
    # and as a step with the forward calls.
    fused_calls = [(f"bwd{i + 1}", lambda c=c, i=i: c.bwd(xs[i], ws[i], dys[i], ys[i], dxs[i], dws[i]))
                   for i, c in reversed(list(enumerate(convs)))]
    fused = {"us_per_call": {}}
    for name, f in fused_calls:
        f()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        fused["us_per_call"][name] = round(start.elapsed_time(end) / (replays * reps) * 1e3, 3)
        del g
    fwd_calls = [c for c in calls if c[0].startswith("fwd")]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, f in fwd_calls + fused_calls:
            f()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    fused["ms_per_step"] = round(start.elapsed_time(end) / steps, 5)
    del g

    # The bias entry points (forward with a bias, bias gradient), timed the
    # same way; not part of the step.
    bias_calls = []
    for i, c in enumerate(convs):
        L = layers[i]
        bound = 1.0 / (L.IC * L.KH * L.KW) ** 0.5
        b = inputs.uniform((L.OC,), 900 + i, bound, wl.dtype).to(dev)
        db = torch.empty_like(b)
        yb = torch.empty_like(ys[i])
        bias_calls.append((f"fwd_bias{i + 1}", lambda c=c, i=i, b=b, yb=yb: c.fwd_bias(xs[i], ws[i], b, yb)))
        bias_calls.append((f"bwd_bias{i + 1}", lambda c=c, i=i, db=db: c.bwd_bias(dys[i], ys[i], db)))
    bias_us = {}
    for name, f in bias_calls:
        f()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        bias_us[name] = start.elapsed_time(end) / (replays * reps) * 1e3
        del g
    return ms_step, ms_eager, per_call, bias_us, ms_cold, floor, fused


def cpu_baseline(wl, budget_s):
    """The oracle (fp64, OpenMP) on a bounded sample of the workload's batch."""
    import numpy as np

    from backward_implicit_gemm_amd import inputs
    from oracle import oracle as orc

    L = wl.layers[0]
    x, w, dy = inputs.layer_inputs(L, wl.seeds, wl.dtype)
    f64 = lambda a: a.to(dtype=__import__("torch").float64).numpy()
    X, Wt, DY = f64(x), f64(w), f64(dy)

    def step(nb):
        xs, dys = X[:nb], DY[:nb]
        t0 = time.perf_counter()
        y = orc.conv_fwd(xs, Wt, L.stride, L.relu)
        orc.conv_bwd_data(dys, Wt, y if L.relu else None, xs.shape, L.stride, L.relu)
        orc.conv_bwd_weight(xs, dys, y if L.relu else None, Wt.shape, L.stride, L.relu)
        return time.perf_counter() - t0

    # size the sample from a small probe so the leg takes about budget_s
    probe_b = min(L.B, 16)
    tp = step(probe_b)
    nb = int(min(L.B, max(probe_b, probe_b * (budget_s / 3.0) / max(tp, 1e-6))))
    times = [step(nb) for _ in range(3)]
    t = statistics.median(times)
    flops = 3 * layer_flops(L.with_batch(nb))
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.thread_count(),
        "kind": "oracle",
        "sample": f"{nb} of {L.B} images of {wl.name}, fwd+dgrad+wgrad in fp64, median of 3",
        "ms_per_step_sample": t * 1e3,
    }


# Kernels behind each call, as named in rocprofv3 summaries.
CALL_KERNELS = {
    "fwd": {"f32": ["pack_w_fwd_f32", "fwd_ws_f32"], "bf16": ["pack_w_fwd_bf16", "fwd_ws_bf16"]},
    "dgrad": {"f32": ["dgrad_rf_f32"], "bf16": ["pack_w_dgrad_bf16", "dgrad_ig_bf16"]},
    "wgrad": {"f32": ["wgrad_rf_f32", "wgrad_reduce"],
              "bf16": ["dz_groups_bf16", "wgrad_ws_bf16", "wgrad_reduce"]},
}

def report(wl, ms_step, ms_eager, per_call, bias_us, ms_cold, floor, steps, warmup, cpu, fused=None):
    L0 = wl.layers[0]
    esize = 4 if wl.dtype == "f32" else 2
    flops_step = sum(3 * layer_flops(L) for L in wl.layers)
    # per-call algorithmic work
    work = {}
    for i, L in enumerate(wl.layers):
        b = layer_bytes(L, esize)
        for op in ("fwd", "dgrad", "wgrad"):
            work[f"{op}{i + 1}"] = (layer_flops(L), b[op])
    dom = max(per_call, key=per_call.get)
    fl, by = work[dom]
    us = per_call[dom]
    if wl.dtype == "f32":
        bound, peak, unit, achieved = "mfma", PEAK["mfma_f32"], "TFLOP/s", fl / (us * 1e-6) / 1e12
    else:
        # bf16 at these shapes sits left of the MFMA ridge: HBM-bound
        bound, peak, unit, achieved = "hbm", PEAK["hbm_gbs"], "GB/s", by / (us * 1e-6) / 1e9
    roof = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(wl.name, dom),
            "kernel_call": dom, "kernels": CALL_KERNELS[dom.rstrip("0123456789")][wl.dtype],
            "us_per_launch": round(us, 3)}
    value = flops_step / (ms_step * 1e-3) / 1e12
    fwd_us = sum(v for k, v in per_call.items() if k.startswith("fwd"))
    bwd_us = sum(v for k, v in per_call.items() if not k.startswith("fwd"))
    vs = None
    if wl.name in PAGE1_US:
        page_us = sum(PAGE1_US[wl.name])
        vs = round(page_us / (ms_step * 1e3), 3)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_cold": round(ms_cold, 5),
        "launch_floor": floor,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "global_batch": L0.B,
            "layers": [f"{L.IC}->{L.OC} {L.H}x{L.W} k{L.KH}x{L.KW} s{L.stride}"
                       + (" relu" if L.relu else "") for L in wl.layers],
            "parallelism": "none (one GPU)",
        },
        "us_per_iter": {"fwd": round(fwd_us, 3), "bwd": round(bwd_us, 3),
                        **{k: round(v, 3) for k, v in per_call.items()}},
        "tflops": {"fwd": round(sum(layer_flops(L) for L in wl.layers) / (fwd_us * 1e-6) / 1e12, 3),
                   "bwd": round(sum(2 * layer_flops(L) for L in wl.layers) / (bwd_us * 1e-6) / 1e12, 3)},
        "roofline": roof,
        "bias_us_per_call": {k: round(v, 3) for k, v in bias_us.items()},
        "fused_bwd": fused,
        "cpu_baseline": cpu,
    }
    if vs is not None:
        line["baseline_note"] = ("page 1 gemm_fast fwd+bwd on an unnamed NVIDIA GPU: "
                                 f"{PAGE1_US[wl.name][0]} + {PAGE1_US[wl.name][1]} us; context only")
    return line


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    from backward_implicit_gemm_amd import inputs

    if a.copy_probe_mb > 0:
        import torch
        n = a.copy_probe_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    names = [w.name for w in inputs.WORKLOADS]
    todo = names if a.all else [a.workload]
    for name in todo:
        if name not in names:
            print(f"unknown workload {name}; choose from {names}", file=sys.stderr)
            sys.exit(2)
        wl = inputs.WORKLOADS[names.index(name)]
        ms, ms_eager, per_call, bias_us, ms_cold, floor, fused = run_gpu(wl, a.steps, a.warmup)
        cpu = None
        if not a.no_cpu and name == DEFAULT_WORKLOAD:
            cpu = cpu_baseline(wl, a.cpu_seconds)
        print(json.dumps(report(wl, ms, ms_eager, per_call, bias_us, ms_cold, floor, a.steps, a.warmup,
                                cpu, fused)), flush=True)


if __name__ == "__main__":
    main()
