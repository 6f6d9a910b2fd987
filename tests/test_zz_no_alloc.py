"""gc_conv_fwd_noalloc, the forward for callers that cannot allocate: it
must give exactly gc_conv_fwd's output (same kernels, its scratch in the
library's static per-GPU array instead of a workspace) and so match the
oracle, on two calls in a row with the second on a smaller batch (the
scratch keeps the first call's packed weights, which the second must
rewrite), for both layer shapes and storage types.
"""
import numpy as np
import pytest
import torch

from backward_implicit_gemm_amd import binding as gb
from backward_implicit_gemm_amd import inputs

from cases import LAYER_SHAPES
from parity import TOL, Guarded, Layer, draw, f64, rel_err
from oracle import oracle as orc

pytestmark = pytest.mark.gpu


def setup_module():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gb.lib()


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layer_name", sorted(LAYER_SHAPES))
def test_noalloc_forward_matches_gc_conv_fwd(layer_name, dtype):
    IC, H, W, OC, KH, KW, S, relu = LAYER_SHAPES[layer_name]
    td = inputs.torch_dtype(dtype)
    # the second call is smaller, and its weights differ from the first's
    for B, seeds in ((1024, (1, 2, 3)), (37, (4, 5, 6))):
        layer = Layer(B, IC, H, W, OC, KH, KW, S, relu)
        x, w, _ = draw(layer, seeds, dtype)
        xd, wd = x.cuda(), w.cuda()
        conv = gb.Conv(layer.x_shape, layer.w_shape, S, relu, td, "cuda")
        y_ref = torch.empty(layer.y_shape, dtype=td, device="cuda")
        conv.fwd(xd, wd, y_ref)
        g = Guarded(layer.y_shape, td, "cuda")
        gb.gc_conv_fwd_noalloc(xd, wd, g.t, relu, S)
        torch.cuda.synchronize()
        g.check("y")
        assert torch.equal(_bits(g.t), _bits(y_ref)), (layer_name, dtype, B)
        e = rel_err(f64(g.t), orc.conv_fwd(f64(x), f64(w), S, relu))
        print(f"{layer_name} {dtype} B={B}: noalloc == gc_conv_fwd, oracle {e:.2e}", flush=True)
        assert e <= TOL[dtype]


def test_noalloc_forward_rejects_a_problem_beyond_its_scratch():
    # layer 1 with 512 output channels: 3.4 MB of packed fp32 weights > 2 MiB
    x = torch.zeros((2, 59, 11, 15), device="cuda")
    w = torch.zeros((512, 59, 5, 5), device="cuda")
    y = torch.full((2, 512, 3, 4), 7.0, device="cuda")
    with pytest.raises(gb.GcError, match="GC_ERR_WORKSPACE"):
        gb.gc_conv_fwd_noalloc(x, w, y, 1, 3)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)                      # nothing was enqueued
