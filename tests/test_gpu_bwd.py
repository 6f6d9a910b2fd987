"""GPU tests of gc_conv_bwd, the whole backward of a layer in one call.

It must give dx and dw bit for bit equal to gc_conv_bwd_data followed by
gc_conv_bwd_weight (shapes with a fused plan run the same kernel bodies in
fewer launches; other shapes make the two calls), and so match the oracle
to the same tolerance.  The layer shapes are those of the policy network at
B=1024 and of the two-layer chain at B=16384.
"""
import numpy as np
import pytest
import torch

from backward_implicit_gemm_amd import binding as gb
from backward_implicit_gemm_amd import inputs

from cases import FUSED_BF16_BWD, FUSED_F32_BWD, LAYER_SHAPES, fused_pair
from parity import TOL, Layer, draw, f64, oracle_layer, rel_err

pytestmark = pytest.mark.gpu


def setup_module():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gb.lib()


def _both(layer, dtype, x, w, dy):
    """(y, dx, dw) from gc_conv_bwd and (dx, dw) from the separate calls."""
    dev = "cuda"
    td = inputs.torch_dtype(dtype)
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    xd, wd, dyd = x.to(dev), w.to(dev), dy.to(dev)
    y = torch.empty(layer.y_shape, dtype=td, device=dev)
    conv.fwd(xd, wd, y)
    dx = torch.full(layer.x_shape, float("nan"), dtype=td, device=dev)
    dw = torch.full(layer.w_shape, float("nan"), dtype=td, device=dev)
    conv.bwd(xd, wd, dyd, y, dx, dw)
    dx2 = torch.full_like(dx, float("nan"))
    dw2 = torch.full_like(dw, float("nan"))
    conv.bwd_data(dyd, wd, y, dx2)
    conv.bwd_weight(xd, dyd, y, dw2)
    torch.cuda.synchronize()
    return y, dx, dw, dx2, dw2


def _bits_equal(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("idx", [0, 1, 2, 3], ids=[w.name for w in inputs.WORKLOADS[:4]])
def test_workload_bwd_matches_separate_calls_and_oracle(idx):
    wl = inputs.WORKLOADS[idx]
    L = wl.layers[0]
    layer = Layer.of(L)
    x, w, dy = inputs.layer_inputs(L, wl.seeds, wl.dtype)
    y, dx, dw, dx2, dw2 = _both(layer, wl.dtype, x, w, dy)
    assert _bits_equal(dx, dx2) and _bits_equal(dw, dw2)
    _, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    edx, edw = rel_err(f64(dx), dx_ref), rel_err(f64(dw), dw_ref)
    print(f"{wl.name}: gc_conv_bwd dx={edx:.2e} dw={edw:.2e}", flush=True)
    assert edx <= TOL[wl.dtype] and edw <= TOL[wl.dtype]


@pytest.mark.parametrize("layer_idx", [0, 1], ids=["conv1", "conv2"])
def test_chain_shapes_b16384_match_separate_calls(layer_idx):
    wl = inputs.WORKLOADS[4]
    layer = Layer.of(wl.layers[layer_idx])
    x, w, dy = draw(layer, (71 + layer_idx, 72, 73), "bf16")
    y, dx, dw, dx2, dw2 = _both(layer, "bf16", x, w, dy)
    assert _bits_equal(dx, dx2) and _bits_equal(dw, dw2)
    _, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    edx, edw = rel_err(f64(dx), dx_ref), rel_err(f64(dw), dw_ref)
    print(f"chain conv{layer_idx + 1} B=16384: gc_conv_bwd dx={edx:.2e} dw={edw:.2e}", flush=True)
    assert edx <= TOL["bf16"] and edw <= TOL["bf16"]


SHAPES = [
    (17, 59, 11, 15, 128, 5, 5, 3),
    (37, 128, 3, 4, 96, 3, 3, 1),
    (3, 3, 7, 8, 4, 3, 3, 2),
    (2, 65, 10, 10, 33, 3, 2, 4),
]


@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("relu", [0, 1])
def test_bwd_shapes(shape, dtype, relu):
    layer = Layer(*shape, relu)
    x, w, dy = draw(layer, (sum(shape), 8, 9 + relu), dtype)
    y, dx, dw, dx2, dw2 = _both(layer, dtype, x, w, dy)
    assert _bits_equal(dx, dx2) and _bits_equal(dw, dw2)
    _, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    assert rel_err(f64(dx), dx_ref) <= TOL[dtype] and rel_err(f64(dw), dw_ref) <= TOL[dtype]


def test_bwd_repeated_calls_are_identical():
    wl = inputs.WORKLOADS[2]     # layer 1, bf16: the fused path
    L = wl.layers[0]
    layer = Layer.of(L)
    x, w, dy = inputs.layer_inputs(L, wl.seeds, wl.dtype)
    y, dx, dw, _, _ = _both(layer, wl.dtype, x, w, dy)
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, torch.bfloat16, "cuda")
    xd, wd, dyd = x.cuda(), w.cuda(), dy.cuda()
    for _ in range(3):
        dx3, dw3 = torch.empty_like(dx), torch.empty_like(dw)
        conv.bwd(xd, wd, dyd, y, dx3, dw3)
        torch.cuda.synchronize()
        assert _bits_equal(dx3, dx) and _bits_equal(dw3, dw)
    assert np.isfinite(f64(dw)).all()


@pytest.mark.parametrize("relu", [0, 1])
@pytest.mark.parametrize("pair", sorted(FUSED_F32_BWD), ids=lambda p: "{}-B{}".format(*FUSED_F32_BWD[p]))
def test_fused_f32_pairs(pair, relu):
    # every (d_input, wgrad) pair of the one-launch fp32 backward, with and
    # without the ReLU, at a batch that leaves a ragged last image group and
    # quad
    layer_name, B = FUSED_F32_BWD[pair]
    shape = LAYER_SHAPES[layer_name][:7]
    layer = Layer(B, *shape, relu)
    name = gb.gc_conv_plan_name(gb.GC_OP_BWD, gb.make_desc(B, *shape), gb.GC_F32)
    print(f"{layer_name} B={B} relu={relu}: {name}", flush=True)
    assert fused_pair(name) == pair
    x, w, dy = draw(layer, (B, 5, 6 + relu), "f32")
    y, dx, dw, dx2, dw2 = _both(layer, "f32", x, w, dy)
    assert _bits_equal(dx, dx2) and _bits_equal(dw, dw2)
    _, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    edx, edw = rel_err(f64(dx), dx_ref), rel_err(f64(dw), dw_ref)
    print(f"  dx={edx:.2e} dw={edw:.2e}", flush=True)
    assert edx <= TOL["f32"] and edw <= TOL["f32"]


@pytest.mark.parametrize("relu", [0, 1])
@pytest.mark.parametrize("form", sorted(FUSED_BF16_BWD), ids=lambda f: "{}-B{}".format(*FUSED_BF16_BWD[f]))
def test_fused_bf16_forms(form, relu):
    # every fused form of the bf16 backward (pre-pass, the two main grids in
    # one launch or one after the other, reduction) against the separate
    # calls and the oracle
    layer_name, B = FUSED_BF16_BWD[form]
    shape = LAYER_SHAPES[layer_name][:7]
    layer = Layer(B, *shape, relu)
    name = gb.gc_conv_plan_name(gb.GC_OP_BWD, gb.make_desc(B, *shape), gb.GC_BF16)
    print(f"{layer_name} B={B} relu={relu}: {name}", flush=True)
    assert fused_pair(name) == form
    x, w, dy = draw(layer, (B, 15, 16 + relu), "bf16")
    y, dx, dw, dx2, dw2 = _both(layer, "bf16", x, w, dy)
    assert _bits_equal(dx, dx2) and _bits_equal(dw, dw2)
    _, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    edx, edw = rel_err(f64(dx), dx_ref), rel_err(f64(dw), dw_ref)
    print(f"  dx={edx:.2e} dw={edw:.2e}", flush=True)
    assert edx <= TOL["bf16"] and edw <= TOL["bf16"]
