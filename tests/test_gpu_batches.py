"""GPU parity at every batch size tests/cases.py lists for the two
policy-network layer shapes of "Speedups to gemm_conv_forward and
gemm_conv_backward kernels" (PufferLib pull request #522): together these
runs reach every kernel instance the planners can pick for those shapes
(a CPU test pins that through gc_conv_plan_name).  Each run compares all
three passes with the oracle element by element, with guard bands around
every output.  Also: the forward writing into output views of lower
alignment than the kernels' 16-byte stores.
"""
import numpy as np
import pytest
import torch

from backward_implicit_gemm_amd import binding as gb

from cases import LAYER_BATCHES, LAYER_SHAPES
from parity import Layer, check_layer

pytestmark = pytest.mark.gpu


def setup_module():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gb.lib()


CASES = [(layer, dtype, B) for (layer, dtype), bs in sorted(LAYER_BATCHES.items()) for B in bs]


def _plans(layer, dtype):
    d = gb.make_desc(layer.B, layer.IC, layer.H, layer.W, layer.OC, layer.KH, layer.KW,
                     layer.stride)
    dt = gb.GC_F32 if dtype == "f32" else gb.GC_BF16
    return " | ".join(gb.gc_conv_plan_name(op, d, dt)
                      for op in (gb.GC_OP_FWD, gb.GC_OP_BWD_DATA, gb.GC_OP_BWD_WEIGHT))


@pytest.mark.parametrize("layer_name,dtype,B", CASES, ids=[f"{l}-{d}-b{b}" for l, d, b in CASES])
def test_layer_batch_parity(layer_name, dtype, B):
    IC, H, W, OC, KH, KW, S, relu = LAYER_SHAPES[layer_name]
    layer = Layer(B, IC, H, W, OC, KH, KW, S, relu)
    print(f"{layer_name} {dtype} B={B}: {_plans(layer, dtype)}", flush=True)
    errs, (y, dx, dw), _ = check_layer(layer, dtype, seeds=(B, 5, 6))
    print("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    if layer_name == "layer1":
        assert torch.all(dx[..., 14] == 0)      # column 14 is covered by no window


@pytest.mark.parametrize("layer_name", sorted(LAYER_SHAPES))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("offset", [1, 3])
def test_forward_into_unaligned_output(layer_name, dtype, offset):
    # y starts `offset` elements past a 1 KiB boundary: 2-byte (bf16) or
    # 4-byte (fp32) alignment only; the result must not change
    IC, H, W, OC, KH, KW, S, relu = LAYER_SHAPES[layer_name]
    layer = Layer(1024, IC, H, W, OC, KH, KW, S, relu)
    print(f"{layer_name} {dtype} y offset {offset}: {_plans(layer, dtype)}", flush=True)
    errs, _, _ = check_layer(layer, dtype, seeds=(31, 32, 33), y_offset=offset)
    print("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
