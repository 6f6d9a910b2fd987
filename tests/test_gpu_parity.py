"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Covers the policy-network layer shapes of "Speedups to gemm_conv_forward and
gemm_conv_backward kernels" (PufferLib pull request #522) at their full
batch of 1024 in fp32 and bf16, the two-layer chain at B=16384 and 32768
stage by stage on every element, an odd-shape sweep whose tiles end
mid-tile, integer-valued inputs that must match bit for bit (at the
workloads' batch sizes too), and run-to-run determinism of wgrad.
"""
import numpy as np
import pytest
import torch

from backward_implicit_gemm_amd import binding as gb
from backward_implicit_gemm_amd import inputs
from oracle import oracle as orc

from parity import TOL, Layer, check_layer, draw, f64, gpu_layer, rel_err

pytestmark = pytest.mark.gpu


def setup_module():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gb.lib()


# ---------------------------------------------------------------------------
# Full-size workloads (B=1024), every output element against the oracle
# ---------------------------------------------------------------------------

@pytest.fixture
def kernel_policy(request):
    prev = gb.gc_set_kernel_policy(request.param)
    yield request.param
    gb.gc_set_kernel_policy(prev)


POLICIES = [gb.GC_POLICY_AUTO, gb.GC_POLICY_GENERIC]


@pytest.mark.parametrize("kernel_policy", POLICIES, ids=["auto", "generic"], indirect=True)
@pytest.mark.parametrize("idx", [0, 1, 2, 3], ids=[w.name for w in inputs.WORKLOADS[:4]])
def test_workload_full_parity(idx, kernel_policy):
    wl = inputs.WORKLOADS[idx]
    L = wl.layers[0]
    layer = Layer.of(L)
    x, w, dy = inputs.layer_inputs(L, wl.seeds, wl.dtype)
    errs, (y, dx, dw), (y_ref, _, _) = check_layer(layer, wl.dtype, x=x, w=w, dy=dy)
    print(f"{wl.name} policy={kernel_policy}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    if layer.relu:
        flips = int(np.sum((f64(y) > 0) != (y_ref > 0)))
        print(f"{wl.name}: ReLU mask disagreements with the oracle's y: {flips}", flush=True)
    if layer.W == 15 and layer.KW == 5 and layer.stride == 3:
        # layer-1 input column 14 is covered by no window
        assert torch.all(dx[..., 14] == 0)


# ---------------------------------------------------------------------------
# Two-layer chain at B=16384 and B=32768, stage-wise, every element: each
# oracle stage gets exactly the bf16 tensors the GPU stage got (y1 as conv2's
# input and conv1's mask, dy1 as conv1's dy)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [4, 5], ids=[w.name for w in inputs.WORKLOADS[4:6]])
def test_chain_stagewise_full(idx):
    from parity import Guarded
    wl = inputs.WORKLOADS[idx]
    l1, l2 = (Layer.of(L) for L in wl.layers)
    t = inputs.workload_inputs(wl)
    dev = "cuda"
    td = torch.bfloat16
    c1 = gb.Conv(l1.x_shape, l1.w_shape, l1.stride, l1.relu, td, dev)
    c2 = gb.Conv(l2.x_shape, l2.w_shape, l2.stride, l2.relu, td, dev)
    x, w1, w2, dy2 = (t[k].to(dev) for k in ("x", "w1", "w2", "dy"))
    g = {k: Guarded(shape, td, dev) for k, shape in (
        ("y1", l1.y_shape), ("y2", l2.y_shape), ("dy1", l1.y_shape), ("dw2", l2.w_shape),
        ("dx1", l1.x_shape), ("dw1", l1.w_shape))}
    y1, y2, dy1, dw2, dx1, dw1 = (g[k].t for k in ("y1", "y2", "dy1", "dw2", "dx1", "dw1"))
    c1.fwd(x, w1, y1)
    c2.fwd(y1, w2, y2)
    c2.bwd_data(dy2, w2, None, dy1)
    c2.bwd_weight(y1, dy2, None, dw2)
    c1.bwd_data(dy1, w1, y1, dx1)
    c1.bwd_weight(x, dy1, y1, dw1)
    torch.cuda.synchronize()
    for k, gd in g.items():
        gd.check(k)
    print(f"chain B={l1.B}: copied, running the oracle", flush=True)

    X, W1, W2, DY2 = f64(t["x"]), f64(t["w1"]), f64(t["w2"]), f64(t["dy"])
    Y1, DY1 = f64(y1), f64(dy1)
    stages = (
        ("y1", y1, lambda: orc.conv_fwd(X, W1, l1.stride, 1)),
        ("y2", y2, lambda: orc.conv_fwd(Y1, W2, l2.stride, 0)),
        ("dy1", dy1, lambda: orc.conv_bwd_data(DY2, W2, None, l2.x_shape, l2.stride, 0)),
        ("dw2", dw2, lambda: orc.conv_bwd_weight(Y1, DY2, None, l2.w_shape, l2.stride, 0)),
        ("dx1", dx1, lambda: orc.conv_bwd_data(DY1, W1, Y1, l1.x_shape, l1.stride, 1)),
        ("dw1", dw1, lambda: orc.conv_bwd_weight(X, DY1, Y1, l1.w_shape, l1.stride, 1)),
    )
    for name, got, ref_fn in stages:
        ref = ref_fn()
        e = rel_err(f64(got), ref)
        print(f"chain B={l1.B} {name}: max|diff|/max|ref| = {e:.2e}", flush=True)
        assert e <= TOL["bf16"], (name, e)
        del ref
    assert torch.all(dx1[..., 14] == 0)


# ---------------------------------------------------------------------------
# Odd shapes: ragged batches, channel counts around tile edges, H != W,
# KH != KW, strides 1-4, full-window and pointwise kernels
# ---------------------------------------------------------------------------

ODD = [
    # B, IC, H, W, OC, KH, KW, S
    (1, 1, 1, 1, 1, 1, 1, 1),
    (1, 1, 5, 5, 1, 3, 3, 1),
    (3, 3, 7, 8, 4, 3, 3, 2),
    (17, 59, 11, 15, 128, 5, 5, 3),
    (17, 128, 3, 4, 128, 3, 3, 1),
    (3, 64, 9, 6, 65, 2, 4, 1),
    (2, 65, 10, 10, 33, 3, 2, 4),
    (5, 7, 6, 6, 130, 6, 6, 1),
    (4, 16, 12, 20, 24, 1, 1, 1),
    (2, 3, 32, 32, 8, 5, 5, 2),
    (2, 200, 3, 3, 7, 3, 3, 1),
    (33, 1, 11, 15, 3, 5, 5, 3),
    (9, 59, 11, 15, 128, 5, 5, 3),      # last image group ragged (9 = 2*4 + 1)
    (37, 128, 3, 4, 96, 3, 3, 1),       # OC not a multiple of 64
    (6, 13, 9, 7, 20, 3, 2, 2),         # P = 12 from a rectangular kernel
]


@pytest.mark.parametrize("kernel_policy", POLICIES, ids=["auto", "generic"], indirect=True)
@pytest.mark.parametrize("shape", ODD, ids=["x".join(map(str, s)) for s in ODD])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("relu", [0, 1])
def test_odd_shapes(shape, dtype, relu, kernel_policy):
    layer = Layer(*shape, relu)
    errs, _, _ = check_layer(layer, dtype, seeds=(sum(shape), 7, 8 + relu))
    print(f"{shape} {dtype} relu={relu}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)


# ---------------------------------------------------------------------------
# Integer-valued inputs: every partial sum is an exact small integer, so the
# result cannot depend on summation order and must match exactly.
# ---------------------------------------------------------------------------

INT_SHAPES = [
    # B, IC, H, W, OC, KH, KW, S, relu: the two layer shapes at B=64, at the
    # workloads' B=1024 (the instances the bench times) and at the chain's
    # B=16384, and the auto-policy instance of B=600 for layer 1
    (64, 59, 11, 15, 128, 5, 5, 3, 1), (64, 128, 3, 4, 128, 3, 3, 1, 1),
    (600, 59, 11, 15, 128, 5, 5, 3, 1),
    (1024, 59, 11, 15, 128, 5, 5, 3, 1), (1024, 128, 3, 4, 128, 3, 3, 1, 0),
    (16384, 59, 11, 15, 128, 5, 5, 3, 1), (16384, 128, 3, 4, 128, 3, 3, 1, 0),
]
INT_CASES = [(s, p) for s in INT_SHAPES for p in POLICIES if s[0] <= 64 or p == gb.GC_POLICY_AUTO]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,kernel_policy", INT_CASES, indirect=["kernel_policy"],
                         ids=[f"b{s[0]}-ic{s[1]}-{'auto' if p == 0 else 'generic'}" for s, p in INT_CASES])
def test_integer_inputs_exact(shape, dtype, kernel_policy):
    layer = Layer(*shape)
    relu = layer.relu
    x = inputs.integers(layer.x_shape, 21, dtype=dtype)
    w = inputs.integers(layer.w_shape, 22, dtype=dtype)
    dy = inputs.integers(layer.y_shape, 23, dtype=dtype)
    _, y, dx, dw = gpu_layer(layer, x, w, dy, dtype)
    ym = f64(y) if relu else None
    y_ref = orc.conv_fwd(f64(x), f64(w), layer.stride, relu)
    dx_ref = orc.conv_bwd_data(f64(dy), f64(w), ym, layer.x_shape, layer.stride, relu)
    dw_ref = orc.conv_bwd_weight(f64(x), f64(dy), ym, layer.w_shape, layer.stride, relu)
    td = inputs.torch_dtype(dtype)
    rne = lambda a: torch.from_numpy(a).to(torch.float32).to(td).to(torch.float64).numpy()
    for name, got, ref in (("y", y, y_ref), ("dx", dx, dx_ref), ("dw", dw, dw_ref)):
        assert np.all(np.abs(ref) < 2 ** 24)
        assert np.array_equal(f64(got), rne(ref)), name


# ---------------------------------------------------------------------------
# wgrad is bit-reproducible (fixed-order split-K reduction, no atomics)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wgrad_deterministic(dtype):
    L = inputs.LAYER1
    layer = Layer.of(L)
    x, w, dy = inputs.layer_inputs(L, (11, 12, 13), dtype)
    conv, y, dx, dw = gpu_layer(layer, x, w, dy, dtype)
    xd, dyd = x.cuda(), dy.cuda()
    for _ in range(3):
        dw2 = torch.empty_like(dw)
        conv.bwd_weight(xd, dyd, y, dw2)
        dx2 = torch.empty_like(dx)
        conv.bwd_data(dyd, w.cuda(), y, dx2)
        torch.cuda.synchronize()
        assert torch.equal(dw2.view(torch.int16) if dtype == "bf16" else dw2.view(torch.int32),
                           dw.view(torch.int16) if dtype == "bf16" else dw.view(torch.int32))
        assert torch.equal(dx2, dx)


def test_outputs_fully_overwritten():
    # Outputs start as NaN in gpu_layer; every element must have been written.
    layer = Layer(5, 59, 11, 15, 128, 5, 5, 3, 1)
    x, w, dy = draw(layer, (1, 2, 3), "bf16")
    _, y, dx, dw = gpu_layer(layer, x, w, dy, "bf16")
    for t in (y, dx, dw):
        assert torch.isfinite(t.float()).all()


def test_bf16_rounding_is_nearest_even():
    # 1x1 conv with w = 1 copies x through the fp32 accumulator; pick fp32
    # values that sit exactly on bf16 ties is impossible from bf16 inputs, so
    # use w = 1 + 2^-8 on bf16 x: products land between bf16 neighbours and
    # the stored result must equal torch's round-to-nearest-even of the fp32
    # product.
    B, C = 4, 1
    x = inputs.normal((B, C, 8, 8), 5, "bf16")
    w = torch.full((1, 1, 1, 1), 1.0 + 2 ** -7, dtype=torch.bfloat16)
    layer = Layer(B, C, 8, 8, 1, 1, 1, 1, 0)
    dy = torch.zeros(layer.y_shape, dtype=torch.bfloat16)
    _, y, _, _ = gpu_layer(layer, x, w, dy, "bf16")
    want = (x.float() * w.float()).to(torch.bfloat16)
    assert torch.equal(y.cpu(), want)


# ---------------------------------------------------------------------------
# Batches with more image groups than the bf16 forward's single round of
# workgroups: each workgroup walks two or three groups, the last one ragged
# (2054 = 513*4 + 2 images of layer 1; 8300 = 259*32 + 12 of layer 2)
# ---------------------------------------------------------------------------

SEVERAL_GROUPS = [(2054, 59, 11, 15, 128, 5, 5, 3, 1), (8300, 128, 3, 4, 128, 3, 3, 1, 0)]


@pytest.mark.parametrize("shape", SEVERAL_GROUPS, ids=["layer1_b2054", "layer2_b8300"])
def test_bf16_several_groups_per_workgroup(shape):
    layer = Layer(*shape)
    errs, _, _ = check_layer(layer, "bf16", seeds=(5, 6, 7))
    print(f"{shape}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
