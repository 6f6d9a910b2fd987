"""Benchmark: convolution forward + d_input + wgrad through libgc's C ABI.

One step is one pass of the whole path over one batch -- forward (with the
fused ReLU where the layer has one), then d_input and wgrad through
gc_conv_bwd, the library's one-call backward (the page's gemm_conv_backward
counterpart) -- on synthetic seeded inputs already resident in HBM.  The default workload is the policy
network's layer 1 in fp32 at B=1024 (59->128 channels, 11x15 input, 5x5
kernel, stride 3, ReLU), as benchmarked in "Speedups to gemm_conv_forward and
gemm_conv_backward kernels" (PufferLib pull request #522), which times
forward and backward separately over 50 warmup and 200 timed iterations.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]

Prints one JSON line: throughput in TFLOP/s of algorithmic work
(2*B*OC*OH*OW*IC*KH*KW per pass, three passes per step) over K steps, each
step replayed as one HIP graph between HIP events on the launch stream; the
same K steps issued eagerly (host work included), all after an untimed
pre-warm of 0.3 s of step replays and the W warmup steps; the step timed cold
(caches flushed by a 640 MB write before each replay); the launch floor (a
graph of as many one-element kernels as a step launches); per-call GPU times,
hot (graphs of back-to-back copies of each call, warmed for 20 ms, at least
ten replays timed) and cold (each call alone
after a cache flush, median of several), for the step's calls and for the
two backward passes as separate calls (gc_conv_bwd_data, gc_conv_bwd_weight),
with the step made of those separate calls beside it; a roofline entry for
the dominant call of the step; and
the CPU oracle timed on this host on a bounded sample.  The same line carries,
under "workloads", every other workload's step and per-call times with each
call's fraction of its binding roofline (bf16: algorithmic bytes over the cold
time against HBM; fp32: flops over the hot time against fp32 MFMA), and under
"data_independence" the layer-1 bf16 calls rerun with x scaled by 1/8 and 8,
and under "hbm_copy" the bandwidth a plain 1 GiB device copy reaches here
(reads + writes), beside which each bf16 call's fraction of the measured
copy rate is given as "frac_copy" (the roofline fractions use the published
8 TB/s); each bf16 call also carries "same_bytes_copy", a plain copy moving
the call's algorithmic bytes timed the same way (hot and cold, with its own
fraction of 8 TB/s), and "frac_of_same_bytes_copy", the copy's cold time over
the call's: what one launch of that size reaches here, beside the call.
--workload NAME (or --all) prints the full line of other workloads.
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

# Seconds of untimed step replays before the warmup steps of each workload,
# and of untimed replays of each per-call graph before it is timed.
PREWARM_S = 0.3
PREWARM_CALL_S = 0.02


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true", help="every workload, one line each")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--headline-only", action="store_true",
                    help="default workload only: skip the other workloads and the "
                         "data-independence leg")
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
    nm = ny if L.relu else 0      # y, read as the ReLU mask
    fwd = (nx + nw + ny) * esize
    dgrad = (ny + nm + nw + nx) * esize
    wgrad = (nx + ny + nm + nw) * esize
    bwd = (ny + nm + nx + nw + nx + nw) * esize    # dy, y, x, w read; dx, dw written
    return {"fwd": fwd, "dgrad": dgrad, "wgrad": wgrad, "bwd": bwd}


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


def run_gpu(wl, steps, warmup, x_scale=1.0, extras=True, copies=True):
    """Times workload wl.  x_scale multiplies the input x (a power of two
    leaves every product exact up to the exponent); extras=False skips the
    eager and bias timings; copies=False skips the same-bytes copies of an
    HBM-bound workload's calls."""
    import torch

    from backward_implicit_gemm_amd import binding as gb
    from backward_implicit_gemm_amd import inputs

    dev = torch.device("cuda:0")
    td = inputs.torch_dtype(wl.dtype)
    t = inputs.workload_inputs(wl)
    layers = wl.layers
    convs = [gb.Conv(L.x_shape, L.w_shape, L.stride, L.relu, td, dev) for L in layers]
    if x_scale != 1.0:
        t["x"] = (t["x"].float() * x_scale).to(td)
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

    # calls of one step, in order: forward through the layers, then the
    # backward of each layer (d_input and wgrad in one gc_conv_bwd call), last
    # layer first
    calls = []
    for i, c in enumerate(convs):
        calls.append((f"fwd{i + 1}", lambda c=c, i=i: c.fwd(xs[i], ws[i], ys[i])))
    for i in reversed(range(len(convs))):
        c = convs[i]
        calls.append((f"bwd{i + 1}",
                      lambda c=c, i=i: c.bwd(xs[i], ws[i], dys[i], ys[i], dxs[i], dws[i])))
    # the two backward passes of each layer as separate calls, timed beside
    # the step
    pass_calls = []
    for i in reversed(range(len(convs))):
        c = convs[i]
        pass_calls.append((f"dgrad{i + 1}", lambda c=c, i=i: c.bwd_data(dys[i], ws[i], ys[i], dxs[i])))
        pass_calls.append((f"wgrad{i + 1}", lambda c=c, i=i: c.bwd_weight(xs[i], dys[i], ys[i], dws[i])))

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
    # Untimed pre-warm of PREWARM_S seconds, then the W warmup steps: a few
    # dozen steps of a 0.1 ms step leave the GPU short of its steady clocks,
    # and the first steps timed after them read up to ~10 % slow.
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PREWARM_S:
        for _ in range(20):
            step_graph.replay()
        torch.cuda.synchronize()
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
    nk = sum(len(call_kernels(wl, name)) for name, _ in calls)
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
    ms_eager = None
    if extras:
        start.record(stream)
        for _ in range(steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        ms_eager = start.elapsed_time(end) / steps

    # Per call: a graph of REPS back-to-back copies of the call, replayed and
    # timed with HIP events on the launch stream, so each figure is the
    # call's GPU time (its kernels plus the gaps between graph nodes), over
    # at least 10 replays whatever K is (with 2, a 20-step run's per-call
    # figures read up to 10 % slow).
    reps = 10
    replays = max(10, min(20, steps // reps))
    per_call = {}
    for name, f in calls + pass_calls:
        f()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < PREWARM_CALL_S:
            g.replay()
            torch.cuda.synchronize()
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        per_call[name] = start.elapsed_time(end) / (replays * reps) * 1e3
        del g
    per_call_cold = {name: cold_call_us(f, stream, dev, reps=cold_reps(per_call[name]))
                     for name, f in calls + pass_calls}
    # HBM-bound calls: a plain copy of the same number of bytes, timed the same
    # way, as the yardstick of what one launch of that size reaches here
    same_copy = {}
    if copies and wl.dtype != "f32":
        work = call_work(wl)
        for name in per_call:
            same_copy[name] = same_bytes_copy_us(work[name][1], stream, dev, reps, replays)

    # The step with the backward as the two separate calls per layer.
    fwd_calls = [c for c in calls if c[0].startswith("fwd")]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, f in fwd_calls + pass_calls:
            f()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step_separate = start.elapsed_time(end) / steps
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
        dwb = torch.empty_like(dws[i])
        bias_calls.append((f"wgrad_bias{i + 1}",
                           lambda c=c, i=i, db=db, dwb=dwb: c.bwd_weight_bias(xs[i], dys[i], ys[i], dwb, db)))
    bias_us = {}
    for name, f in (bias_calls if extras else []):
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
    return {"ms_step": ms_step, "ms_eager": ms_eager, "per_call": per_call,
            "per_call_cold": per_call_cold, "bias_us": bias_us, "ms_cold": ms_cold,
            "floor": floor, "step_calls": [n for n, _ in calls],
            "ms_step_separate": ms_step_separate, "same_copy": same_copy}


def same_bytes_copy_us(nbytes, stream, dev, reps, replays):
    """A plain device-to-device copy moving nbytes (half read, half written),
    the algorithmic bytes of one call: hot (a graph of `reps` back-to-back
    copies, warmed like the calls' graphs, `replays` replays timed) and cold
    (cold_call_us), in microseconds per copy."""
    import torch

    half = max(16, nbytes // 2 // 16 * 16)
    src = torch.ones(half, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)

    def f():
        dst.copy_(src)

    f()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            f()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PREWARM_CALL_S:
        g.replay()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    hot = start.elapsed_time(end) / (replays * reps) * 1e3
    del g
    cold = cold_call_us(f, stream, dev, reps=cold_reps(hot))
    del src, dst
    return {"us_hot": round(hot, 3), "us_cold": round(cold, 3), "bytes": 2 * half}


def cold_reps(us_hot):
    """Copies per cold-timing graph: the difference of two graph timings is
    divided by it, so short calls get more copies (their difference is a small
    part of the 640 MB writes' time)."""
    return 16 if us_hot < 30.0 else 4


def cold_call_us(f, stream, dev, reps=4, rounds=5):
    """One call's GPU time from HBM.  Graph A holds `reps` copies of [a 640 MB
    write, the call], graph B the same writes alone; the write is more than
    the 256 MB MALL and every L2 together, so each copy of the call starts
    with cold caches.  A and B are replayed in turn between HIP events on the
    launch stream, and the call's time is (median A - median B) / reps, which
    leaves out the writes and the graph launch."""
    import torch

    flush = torch.empty(640 << 20, dtype=torch.uint8, device=dev)
    f()
    ga, gb_ = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for _ in range(reps):
            flush.fill_(1)
            f()
    with torch.cuda.graph(gb_):
        for _ in range(reps):
            flush.fill_(1)
    ga.replay()
    gb_.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ta, tb = [], []
    for _ in range(rounds):
        for g, ts in ((ga, ta), (gb_, tb)):
            start.record(stream)
            g.replay()
            end.record(stream)
            torch.cuda.synchronize()
            ts.append(start.elapsed_time(end) * 1e3)
    del ga, gb_, flush
    return max(0.0, (statistics.median(ta) - statistics.median(tb)) / reps)


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


def call_kernels(wl, name):
    """The kernels a call launches: fixed per pass, and for gc_conv_bwd the
    ones its plan (as the library reports it) runs."""
    op = name.rstrip("0123456789")
    if op != "bwd":
        return CALL_KERNELS[op][wl.dtype]
    from backward_implicit_gemm_amd import binding as gb

    L = wl.layers[int(name[len(op):]) - 1]
    d = gb.make_desc(L.B, L.IC, L.H, L.W, L.OC, L.KH, L.KW, L.stride)
    plan = gb.gc_conv_plan_name(gb.GC_OP_BWD, d, gb.GC_F32 if wl.dtype == "f32" else gb.GC_BF16)
    if plan.startswith("bwd_fused_f32"):
        return ["bwd_fused_f32", "wgrad_reduce"]
    if plan.startswith("bwd_fused_bf16 fuse_main=1"):
        return ["bwd_prep_bf16", "bwd_fused_bf16", "wgrad_reduce"]
    if plan.startswith("bwd_fused_bf16"):
        return ["bwd_prep_bf16", "dgrad_ig_bf16", "wgrad_ws_bf16", "wgrad_reduce"]
    return CALL_KERNELS["dgrad"][wl.dtype] + CALL_KERNELS["wgrad"][wl.dtype]


def call_work(wl):
    """Algorithmic (flops, bytes) of every call: the step's (fwd, bwd) and the
    separate backward passes (dgrad, wgrad)."""
    esize = 4 if wl.dtype == "f32" else 2
    work = {}
    for i, L in enumerate(wl.layers):
        b = layer_bytes(L, esize)
        for op in ("fwd", "dgrad", "wgrad"):
            work[f"{op}{i + 1}"] = (layer_flops(L), b[op])
        work[f"bwd{i + 1}"] = (2 * layer_flops(L), b["bwd"])
    return work


def call_roofline(wl, name, us_hot, us_cold):
    """A call against its binding roofline: fp32 is MFMA-bound at these
    arithmetic intensities (priced on the hot time), bf16 HBM-bound (priced on
    the cold time, with the hot figure beside it as possibly MALL-resident)."""
    fl, by = call_work(wl)[name]
    if wl.dtype == "f32":
        a = fl / (us_hot * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(a, 3), "peak": PEAK["mfma_f32"],
                "unit": "TFLOP/s", "frac": round(a / PEAK["mfma_f32"], 4)}
    a = by / (us_cold * 1e-6) / 1e9
    a_hot = by / (us_hot * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(a, 3), "peak": PEAK["hbm_gbs"], "unit": "GB/s",
            "frac": round(a / PEAK["hbm_gbs"], 4), "frac_hot": round(a_hot / PEAK["hbm_gbs"], 4)}


def workload_summary(wl, m):
    """Step and per-call figures of one workload, each call against its roofline."""
    calls = {}
    for name, us in m["per_call"].items():
        cold = m["per_call_cold"][name]
        r = call_roofline(wl, name, us, cold)
        calls[name] = {"us_hot": round(us, 3), "us_cold": round(cold, 3), "frac": r["frac"],
                       **({"frac_hot": r["frac_hot"]} if "frac_hot" in r else {})}
        cp = m.get("same_copy", {}).get(name)
        if cp:
            # the copy's own fraction of the HBM peak, and how close the call
            # comes to it (both cold)
            calls[name]["same_bytes_copy"] = {
                **cp, "frac": round(cp["bytes"] / (cp["us_cold"] * 1e-6) / 1e9 / PEAK["hbm_gbs"], 4)
                if cp["us_cold"] > 0 else None}
            calls[name]["frac_of_same_bytes_copy"] = round(cp["us_cold"] / cold, 4) if cold > 0 else None
    return {"dtype": wl.dtype, "bound": "mfma" if wl.dtype == "f32" else "hbm",
            "ms_per_step": round(m["ms_step"], 5), "ms_per_step_cold": round(m["ms_cold"], 5),
            "tflops_step": round(sum(3 * layer_flops(L) for L in wl.layers)
                                 / (m["ms_step"] * 1e-3) / 1e12, 3),
            "ms_per_step_separate_calls": round(m["ms_step_separate"], 5),
            "calls": calls, "launch_floor": m["floor"]}


def hbm_copy():
    """A plain device-to-device copy of 1 GiB, four copies per graph replay,
    median of five replays: bytes read plus bytes written per second."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            dst.copy_(src)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        ts.append(start.elapsed_time(end) * 1e-3)
    t = statistics.median(ts)
    del g, src, dst
    gbs = 2 * 4 * n / t / 1e9
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK["hbm_gbs"], 4),
            "bytes_per_copy": 2 * n, "us_per_copy": round(t / 4 * 1e6, 2)}


def add_copy_fractions(line, copy):
    """frac_copy for every HBM-bound call: its algorithmic bytes over its cold
    time, as a fraction of the measured copy rate."""
    def upd(calls):
        for c in calls.values():
            if "frac" in c and c.get("bound", "hbm") == "hbm":
                c["frac_copy"] = round(c["frac"] * PEAK["hbm_gbs"] / copy["gbs"], 4)
    for w in line.get("workloads", {}).values():
        if w["bound"] == "hbm":
            upd(w["calls"])
    if line["roofline"]["bound"] == "hbm":
        upd(line["calls"])
        line["roofline"]["frac_copy"] = round(line["roofline"]["achieved"] / copy["gbs"], 4)
    line["hbm_copy"] = copy
    return line


def report(wl, m, steps, warmup, cpu, others=None, data_ind=None):
    L0 = wl.layers[0]
    flops_step = sum(3 * layer_flops(L) for L in wl.layers)
    per_call, ms_step = m["per_call"], m["ms_step"]
    # the dominant call: the step's slowest, hot for fp32 (MFMA-bound), cold
    # for bf16
    times = per_call if wl.dtype == "f32" else m["per_call_cold"]
    dom = max(m["step_calls"], key=times.get)
    roof = call_roofline(wl, dom, per_call[dom], m["per_call_cold"][dom])
    roof.pop("frac_hot", None)
    roof.update({"traffic": measured_traffic(wl.name, dom), "kernel_call": dom,
                 "kernels": call_kernels(wl, dom),
                 "us_per_launch": round(times[dom], 3),
                 "timing": "hot graph replays" if wl.dtype == "f32"
                 else "cold: each launch after a 640 MB cache flush, median"})
    value = flops_step / (ms_step * 1e-3) / 1e12
    fwd_us = sum(v for k, v in per_call.items() if k.startswith("fwd"))
    bwd_us = sum(v for k, v in per_call.items() if k.startswith("bwd"))
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
        "ms_per_step_eager": None if m["ms_eager"] is None else round(m["ms_eager"], 5),
        "ms_per_step_cold": round(m["ms_cold"], 5),
        "launch_floor": m["floor"],
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
        "us_per_call_cold": {k: round(v, 3) for k, v in m["per_call_cold"].items()},
        "tflops": {"fwd": round(sum(layer_flops(L) for L in wl.layers) / (fwd_us * 1e-6) / 1e12, 3),
                   "bwd": round(sum(2 * layer_flops(L) for L in wl.layers) / (bwd_us * 1e-6) / 1e12, 3)},
        "roofline": roof,
        "calls": workload_summary(wl, m)["calls"],
        "bias_us_per_call": {k: round(v, 3) for k, v in m["bias_us"].items()},
        "ms_per_step_separate_calls": round(m["ms_step_separate"], 5),
        "cpu_baseline": cpu,
    }
    if vs is not None:
        line["baseline_note"] = ("page 1 gemm_fast fwd+bwd on an unnamed NVIDIA GPU: "
                                 f"{PAGE1_US[wl.name][0]} + {PAGE1_US[wl.name][1]} us; context only")
    if others:
        line["workloads"] = others
    if data_ind:
        line["data_independence"] = data_ind
    return line


DATA_INDEPENDENCE_WORKLOAD = "layer1_bf16_relu_b1024"


def data_independence(wl, base, steps, warmup):
    """The workload's calls again with x scaled by 1/8 and by 8 (the method's
    work does not depend on the values): hot and cold microseconds per call,
    and each as a ratio to the unscaled run's."""
    out = {}
    for scale in (0.125, 8.0):
        m = run_gpu(wl, steps, warmup, x_scale=scale, extras=False, copies=False)
        out[f"x*{scale:g}"] = {
            name: {"us_hot": round(m["per_call"][name], 3),
                   "us_cold": round(m["per_call_cold"][name], 3),
                   "ratio_hot": round(m["per_call"][name] / base["per_call"][name], 4),
                   "ratio_cold": round(m["per_call_cold"][name] / base["per_call_cold"][name], 4)}
            for name in m["per_call"]}
    return out


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
    byname = {w.name: w for w in inputs.WORKLOADS}
    default_run = not a.all and a.workload == DEFAULT_WORKLOAD
    for name in todo:
        wl = byname[name]
        m = run_gpu(wl, a.steps, a.warmup)
        print(f"# {name}: {m['ms_step'] * 1e3:.1f} us per step", file=sys.stderr, flush=True)
        others, dind = None, None
        if default_run and not a.headline_only:
            # every other workload's figures, and the data-independence leg
            others = {}
            for other in names:
                if other == name:
                    continue
                mo = run_gpu(byname[other], a.steps, a.warmup, extras=False)
                others[other] = workload_summary(byname[other], mo)
                print(f"# {other}: {mo['ms_step'] * 1e3:.1f} us per step", file=sys.stderr,
                      flush=True)
                if other == DATA_INDEPENDENCE_WORKLOAD:
                    dind = data_independence(byname[other], mo, a.steps, a.warmup)
        cpu = None
        if not a.no_cpu and name == DEFAULT_WORKLOAD:
            cpu = cpu_baseline(wl, a.cpu_seconds)
        line = report(wl, m, a.steps, a.warmup, cpu, others, dind)
        if default_run and not a.headline_only:
            line = add_copy_fractions(line, hbm_copy())
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
