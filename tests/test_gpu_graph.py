"""GPU: a captured HIP graph of one forward + d_input + wgrad step gives the
same bits as the eager calls, on every replay.

Between replays the outputs are refilled with NaN and unrelated eager calls
run on other buffers, so a replay that skipped a kernel, read a stale
workspace or depended on state left by the eager run would show.
"""
import pytest
import torch

from backward_implicit_gemm_amd import binding as gb
from backward_implicit_gemm_amd import inputs

from parity import Layer, draw

pytestmark = pytest.mark.gpu


def setup_module():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gb.lib()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    ("layer1_f32", Layer(256, 59, 11, 15, 128, 5, 5, 3, 1), "f32"),
    ("layer1_bf16", Layer(256, 59, 11, 15, 128, 5, 5, 3, 1), "bf16"),
    ("layer2_f32", Layer(1024, 128, 3, 4, 128, 3, 3, 1, 0), "f32"),
    ("layer2_bf16", Layer(1024, 128, 3, 4, 128, 3, 3, 1, 0), "bf16"),
]


@pytest.mark.parametrize("name,layer,dtype", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, layer, dtype):
    dev = "cuda"
    td = inputs.torch_dtype(dtype)
    x, w, dy = (t.to(dev) for t in draw(layer, (5, 6, 7), dtype))
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    y = torch.empty(layer.y_shape, dtype=td, device=dev)
    dx = torch.empty(layer.x_shape, dtype=td, device=dev)
    dw = torch.empty(layer.w_shape, dtype=td, device=dev)
    ym = y if layer.relu else None

    def step():
        conv.fwd(x, w, y)
        conv.bwd_data(dy, w, ym, dx)
        conv.bwd_weight(x, dy, ym, dw)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (y, dx, dw)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    # other work between replays: the same layer on different inputs
    other = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    x2, w2, dy2 = (t.to(dev) for t in draw(layer, (15, 16, 17), dtype))
    y2 = torch.empty_like(y)
    dx2 = torch.empty_like(dx)
    dw2 = torch.empty_like(dw)
    for rep in range(4):
        for t in (y, dx, dw):
            t.fill_(float("nan"))
        other.fwd(x2, w2, y2)
        other.bwd_data(dy2, w2, y2 if layer.relu else None, dx2)
        other.bwd_weight(x2, dy2, y2 if layer.relu else None, dw2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for tname, got, ref in zip(("y", "dx", "dw"), (y, dx, dw), want):
            assert torch.equal(_bits(got), _bits(ref)), (name, rep, tname)
    print(f"{name}: 4 replays bit-identical to eager", flush=True)
