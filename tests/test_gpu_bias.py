"""GPU parity for the bias entry points (gc_conv_fwd_bias, gc_conv_bwd_bias)
against the oracle's forward-with-bias and bias gradient.

The bias is drawn like the weights, U(+-1/sqrt(IC*KH*KW)).  The bias
gradient of each layer takes the GPU's own forward output as its ReLU mask,
as the other backward passes do.
"""
import numpy as np
import pytest
import torch

from backward_implicit_gemm_amd import binding as gb
from backward_implicit_gemm_amd import inputs
from oracle import oracle as orc

from parity import TOL, Layer, draw, f64, rel_err

pytestmark = pytest.mark.gpu


def setup_module():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gb.lib()


def _bias(layer, seed, dtype):
    bound = 1.0 / np.sqrt(layer.IC * layer.KH * layer.KW)
    return inputs.uniform((layer.OC,), seed, bound, dtype)


def _run(layer, dtype, x, w, b, dy):
    dev = "cuda"
    td = inputs.torch_dtype(dtype)
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    xd, wd, bd, dyd = (t.to(dev) for t in (x, w, b, dy))
    y = torch.full(layer.y_shape, float("nan"), dtype=td, device=dev)
    db = torch.full((layer.OC,), float("nan"), dtype=td, device=dev)
    conv.fwd_bias(xd, wd, bd, y)
    conv.bwd_bias(dyd, y, db)
    torch.cuda.synchronize()
    return conv, y, db


def _check(layer, dtype, x, w, b, dy):
    conv, y, db = _run(layer, dtype, x, w, b, dy)
    y_ref = orc.conv_fwd_bias(f64(x), f64(w), f64(b), layer.stride, layer.relu)
    db_ref = orc.conv_bwd_bias(f64(dy), f64(y), layer.relu)
    ey, eb = rel_err(f64(y), y_ref), rel_err(f64(db), db_ref)
    assert ey <= TOL[dtype] and eb <= TOL[dtype], (ey, eb)
    return ey, eb, y, db


@pytest.mark.parametrize("idx", [0, 1, 2, 3], ids=[w.name for w in inputs.WORKLOADS[:4]])
def test_workload_bias_parity(idx):
    wl = inputs.WORKLOADS[idx]
    layer = Layer.of(wl.layers[0])
    x, w, dy = inputs.layer_inputs(wl.layers[0], wl.seeds, wl.dtype)
    b = _bias(layer, wl.seeds[1] + 100, wl.dtype)
    ey, eb, _, _ = _check(layer, wl.dtype, x, w, b, dy)
    print(f"{wl.name}: y(bias)={ey:.2e} db={eb:.2e}", flush=True)


BIAS_SHAPES = [
    (1, 1, 1, 1, 1, 1, 1, 1),
    (3, 3, 7, 8, 4, 3, 3, 2),
    (17, 59, 11, 15, 128, 5, 5, 3),
    (17, 128, 3, 4, 128, 3, 3, 1),
    (2, 65, 10, 10, 33, 3, 2, 4),
    (5, 7, 6, 6, 130, 6, 6, 1),
    (2, 3, 32, 32, 8, 5, 5, 2),
    (9, 59, 11, 15, 128, 5, 5, 3),
    (300, 8, 5, 5, 16, 3, 3, 1),        # more images than a bias-grad workgroup has threads
    (2, 3, 5, 5, 260, 3, 3, 1),         # more channels than a bias-grad workgroup has threads
    (3, 4, 20, 20, 64, 3, 3, 1),        # a 4-image chunk too large to stage in LDS
]


@pytest.fixture
def kernel_policy(request):
    prev = gb.gc_set_kernel_policy(request.param)
    yield request.param
    gb.gc_set_kernel_policy(prev)


@pytest.mark.parametrize("kernel_policy", [gb.GC_POLICY_AUTO, gb.GC_POLICY_GENERIC],
                         ids=["auto", "generic"], indirect=True)
@pytest.mark.parametrize("shape", BIAS_SHAPES, ids=["x".join(map(str, s)) for s in BIAS_SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("relu", [0, 1])
def test_bias_shapes(shape, dtype, relu, kernel_policy):
    layer = Layer(*shape, relu)
    x, w, dy = draw(layer, (sum(shape), 5, 6 + relu), dtype)
    b = _bias(layer, 77, dtype)
    _check(layer, dtype, x, w, b, dy)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bias_integer_inputs_exact(dtype):
    layer = Layer(64, 59, 11, 15, 128, 5, 5, 3, 1)
    x = inputs.integers(layer.x_shape, 31, dtype=dtype)
    w = inputs.integers(layer.w_shape, 32, dtype=dtype)
    b = inputs.integers((layer.OC,), 33, dtype=dtype)
    dy = inputs.integers(layer.y_shape, 34, dtype=dtype)
    _, y, db = _run(layer, dtype, x, w, b, dy)
    y_ref = orc.conv_fwd_bias(f64(x), f64(w), f64(b), layer.stride, 1)
    db_ref = orc.conv_bwd_bias(f64(dy), f64(y), 1)
    td = inputs.torch_dtype(dtype)
    rne = lambda a: torch.from_numpy(a).to(torch.float32).to(td).to(torch.float64).numpy()
    assert np.array_equal(f64(y), rne(y_ref))
    assert np.array_equal(f64(db), rne(db_ref))


def test_bias_grad_deterministic():
    layer = Layer(1024, 59, 11, 15, 128, 5, 5, 3, 1)
    x, w, dy = draw(layer, (1, 2, 3), "f32")
    b = _bias(layer, 4, "f32")
    conv, y, db = _run(layer, "f32", x, w, b, dy)
    dyd = dy.cuda()
    for _ in range(3):
        db2 = torch.empty_like(db)
        conv.bwd_bias(dyd, y, db2)
        torch.cuda.synchronize()
        assert torch.equal(db2.view(torch.int32), db.view(torch.int32))


@pytest.mark.parametrize("shape", [(2054, 59, 11, 15, 128, 5, 5, 3, 1), (8300, 128, 3, 4, 128, 3, 3, 1, 0)],
                         ids=["layer1_b2054", "layer2_b8300"])
def test_bias_bf16_several_groups_per_workgroup(shape):
    # batches whose bf16 forward workgroups each walk two or three image
    # groups, the last one ragged, with the bias added in the staged epilogue
    layer = Layer(*shape)
    x, w, dy = draw(layer, (9, 10, 11), "bf16")
    b = _bias(layer, 78, "bf16")
    ey, eb, _, _ = _check(layer, "bf16", x, w, b, dy)
    print(f"{shape}: y(bias)={ey:.2e} db={eb:.2e}", flush=True)


# ---------------------------------------------------------------------------
# gc_conv_bwd_weight_bias: dw and db from one wgrad pass (db as the wgrad
# tiles' extra column with x = 1), against the oracle and against the two
# separate calls
# ---------------------------------------------------------------------------

def _wb(layer, dtype, x, dy, seeds_y):
    dev = "cuda"
    td = inputs.torch_dtype(dtype)
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    xd, dyd = x.to(dev), dy.to(dev)
    # a ReLU mask from a forward pass of random weights
    w = inputs.uniform(layer.w_shape, seeds_y, 1.0 / np.sqrt(layer.IC * layer.KH * layer.KW), dtype)
    y = torch.empty(layer.y_shape, dtype=td, device=dev)
    conv.fwd(xd, w.to(dev), y)
    from parity import Guarded
    gdw, gdb = Guarded(layer.w_shape, td, dev), Guarded((layer.OC,), td, dev)
    conv.bwd_weight_bias(xd, dyd, y, gdw.t, gdb.t)
    dw2 = torch.empty_like(gdw.t)
    db2 = torch.empty_like(gdb.t)
    conv.bwd_weight(xd, dyd, y, dw2)
    conv.bwd_bias(dyd, y, db2)
    torch.cuda.synchronize()
    gdw.check("dw")
    gdb.check("db")
    return conv, y, gdw.t, gdb.t, dw2, db2


WB_SHAPES = [
    # the two layer shapes at the batches that run 128- and 256-column wgrad
    # tiles, ragged and odd shapes (some without a bias column: separate calls)
    (1024, 59, 11, 15, 128, 5, 5, 3, 1), (1024, 128, 3, 4, 128, 3, 3, 1, 0),
    (16384, 59, 11, 15, 128, 5, 5, 3, 1), (16384, 128, 3, 4, 128, 3, 3, 1, 0),
    (37, 128, 3, 4, 96, 3, 3, 1, 1), (9, 59, 11, 15, 128, 5, 5, 3, 0),
    # layer 1's shape with the other ReLU setting of each fp32 bias-column
    # kernel (48-column tiles with a ReLU, 96-column tiles without)
    (101, 59, 11, 15, 128, 5, 5, 3, 1), (301, 59, 11, 15, 128, 5, 5, 3, 0),
    (3, 3, 7, 8, 4, 3, 3, 2, 1), (5, 7, 6, 6, 130, 6, 6, 1, 0),
]


@pytest.mark.parametrize("shape", WB_SHAPES, ids=["x".join(map(str, s)) for s in WB_SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wgrad_with_bias_column(shape, dtype):
    layer = Layer(*shape)
    d = gb.make_desc(*shape[:8])
    name = gb.gc_conv_plan_name(gb.GC_OP_BWD_WEIGHT_BIAS, d,
                                gb.GC_F32 if dtype == "f32" else gb.GC_BF16)
    x, _, dy = draw(layer, (shape[0] + 3, 4, 5), dtype)
    _, y, dw, db, dw2, db2 = _wb(layer, dtype, x, dy, 6)
    ym = f64(y) if layer.relu else None
    dw_ref = orc.conv_bwd_weight(f64(x), f64(dy), ym, layer.w_shape, layer.stride, layer.relu)
    db_ref = orc.conv_bwd_bias(f64(dy), ym, layer.relu)
    ew, eb = rel_err(f64(dw), dw_ref), rel_err(f64(db), db_ref)
    print(f"{shape} {dtype} [{name}]: dw={ew:.2e} db={eb:.2e}", flush=True)
    assert ew <= TOL[dtype] and eb <= TOL[dtype], (ew, eb)
    # with the same splits, the same dw as gc_conv_bwd_weight bit for bit
    # (same kernel and summation order, one more column)
    plain = gb.gc_conv_plan_name(gb.GC_OP_BWD_WEIGHT, d, gb.GC_F32 if dtype == "f32" else gb.GC_BF16)
    splits = lambda n: n.split("splits=")[1].split()[0]
    if "bias column" not in name:
        assert torch.equal(dw, dw2) and torch.equal(db, db2)
    elif splits(name) == splits(plain):
        view = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(dw.view(view), dw2.view(view))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wgrad_with_bias_column_integer_exact(dtype):
    # integer inputs: every partial sum is exact, so db and dw must equal the
    # rounded exact results whatever the order
    layer = Layer(1024, 59, 11, 15, 128, 5, 5, 3, 1)
    x = inputs.integers(layer.x_shape, 41, dtype=dtype)
    dy = inputs.integers(layer.y_shape, 42, dtype=dtype)
    _, y, dw, db, _, _ = _wb(layer, dtype, x, dy, 43)
    ym = f64(y)
    dw_ref = orc.conv_bwd_weight(f64(x), f64(dy), ym, layer.w_shape, layer.stride, 1)
    db_ref = orc.conv_bwd_bias(f64(dy), ym, 1)
    td = inputs.torch_dtype(dtype)
    rne = lambda a: torch.from_numpy(a).to(torch.float32).to(td).to(torch.float64).numpy()
    assert np.array_equal(f64(dw), rne(dw_ref))
    assert np.array_equal(f64(db), rne(db_ref))


def test_wgrad_with_bias_column_deterministic():
    layer = Layer(1024, 59, 11, 15, 128, 5, 5, 3, 1)
    x, _, dy = draw(layer, (7, 8, 9), "bf16")
    conv, y, dw, db, _, _ = _wb(layer, "bf16", x, dy, 10)
    xd, dyd = x.cuda(), dy.cuda()
    for _ in range(3):
        dw2, db2 = torch.empty_like(dw), torch.empty_like(db)
        conv.bwd_weight_bias(xd, dyd, y, dw2, db2)
        torch.cuda.synchronize()
        assert torch.equal(dw2.view(torch.int16), dw.view(torch.int16))
        assert torch.equal(db2.view(torch.int16), db.view(torch.int16))
