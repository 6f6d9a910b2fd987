"""Helpers for the GPU parity tests: run one layer's three passes through the
C ABI and compare with the CPU oracle.

Error metric, per output tensor: max|gpu - ref| / max|ref| (the page's
element-wise relative error blows up near zero, so it is not used).  Bounds:
1e-4 for fp32 storage, 1e-2 for bf16 storage with the oracle fed the same
bf16-rounded inputs upcast exactly.  Backward passes take the GPU's own
forward output as the ReLU mask source on both sides, so a pre-activation
within rounding of zero cannot flip the mask between the two.
"""
import numpy as np
import torch

from backward_implicit_gemm_amd import binding as gb
from backward_implicit_gemm_amd import inputs
from oracle import oracle as orc

TOL = {"f32": 1e-4, "bf16": 1e-2}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    denom = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(got - ref)))
    if denom == 0.0:
        return diff
    return diff / denom


class Layer:
    """Geometry of one call, with or without the workload table's output sizes."""

    def __init__(self, B, IC, H, W, OC, KH, KW, S, relu):
        self.B, self.IC, self.H, self.W, self.OC, self.KH, self.KW = B, IC, H, W, OC, KH, KW
        self.stride, self.relu = S, relu
        self.OH, self.OW = orc.out_dim(H, KH, S), orc.out_dim(W, KW, S)
        self.x_shape = (B, IC, H, W)
        self.w_shape = (OC, IC, KH, KW)
        self.y_shape = (B, OC, self.OH, self.OW)

    @classmethod
    def of(cls, L):
        return cls(L.B, L.IC, L.H, L.W, L.OC, L.KH, L.KW, L.stride, L.relu)


def draw(layer, seeds, dtype):
    sx, sw, sdy = seeds
    x = inputs.normal(layer.x_shape, sx, dtype)
    bound = 1.0 / np.sqrt(layer.IC * layer.KH * layer.KW)
    w = inputs.uniform(layer.w_shape, sw, bound, dtype)
    dy = inputs.normal(layer.y_shape, sdy, dtype)
    return x, w, dy


def gpu_layer(layer, x, w, dy, dtype, dev="cuda"):
    """Forward, d_input and wgrad on the GPU; returns device tensors."""
    td = inputs.torch_dtype(dtype)
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    xd, wd, dyd = x.to(dev), w.to(dev), dy.to(dev)
    y = torch.full(layer.y_shape, float("nan"), dtype=td, device=dev)
    dx = torch.full(layer.x_shape, float("nan"), dtype=td, device=dev)
    dw = torch.full(layer.w_shape, float("nan"), dtype=td, device=dev)
    conv.fwd(xd, wd, y)
    conv.bwd_data(dyd, wd, y, dx)
    conv.bwd_weight(xd, dyd, y, dw)
    torch.cuda.synchronize()
    return conv, y, dx, dw


def oracle_layer(layer, x, w, dy, y_gpu):
    ym = f64(y_gpu) if layer.relu else None
    y = orc.conv_fwd(f64(x), f64(w), layer.stride, layer.relu)
    dx = orc.conv_bwd_data(f64(dy), f64(w), ym, layer.x_shape, layer.stride, layer.relu)
    dw = orc.conv_bwd_weight(f64(x), f64(dy), ym, layer.w_shape, layer.stride, layer.relu)
    return y, dx, dw


def check_layer(layer, dtype, seeds=(1, 2, 3), x=None, w=None, dy=None):
    """Full element-by-element parity of all three passes; returns the errors."""
    if x is None:
        x, w, dy = draw(layer, seeds, dtype)
    _, y, dx, dw = gpu_layer(layer, x, w, dy, dtype)
    y_ref, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    errs = {"y": rel_err(f64(y), y_ref), "dx": rel_err(f64(dx), dx_ref),
            "dw": rel_err(f64(dw), dw_ref)}
    for k, v in errs.items():
        assert np.isfinite(v) and v <= TOL[dtype], (k, v, errs)
    return errs, (y, dx, dw), (y_ref, dx_ref, dw_ref)
