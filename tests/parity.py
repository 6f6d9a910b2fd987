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


GUARD_BYTES = 1024
# bit patterns no output can take: quiet NaNs with a payload
_SENTINEL = {torch.float32: 0x7FC0A5A5, torch.bfloat16: 0x7FA5}


class Guarded:
    """An output tensor inside a device buffer with GUARD_BYTES of sentinel
    words before and after it (and `offset` more elements in front, to place
    the tensor at an address of lower alignment).  check() asserts that no
    kernel wrote outside the tensor."""

    def __init__(self, shape, dtype, dev="cuda", offset=0):
        es = torch.tensor([], dtype=dtype).element_size()
        self.g = GUARD_BYTES // es + offset
        n = 1
        for s in shape:
            n *= int(s)
        self.n = n
        ib = torch.int32 if es == 4 else torch.int16
        pat = _SENTINEL[dtype]
        if es == 2 and pat >= 1 << 15:
            pat -= 1 << 16
        self.buf = torch.full((n + 2 * self.g,), pat, dtype=ib, device=dev).view(dtype)
        self.t = self.buf[self.g:self.g + n].view(shape)   # starts as sentinel NaNs
        self.pat, self.ib = pat, ib

    def check(self, name):
        raw = self.buf.view(self.ib)
        for part, sl in (("before", raw[:self.g]), ("after", raw[self.g + self.n:])):
            bad = int((sl != self.pat).sum())
            assert bad == 0, f"{name}: {bad} guard words {part} the tensor were overwritten"


def gpu_layer(layer, x, w, dy, dtype, dev="cuda", y_offset=0):
    """Forward, d_input and wgrad on the GPU; returns device tensors.  Every
    output sits between guard bands that must come back untouched; y can be
    placed `y_offset` elements past a 1 KiB boundary."""
    td = inputs.torch_dtype(dtype)
    conv = gb.Conv(layer.x_shape, layer.w_shape, layer.stride, layer.relu, td, dev)
    xd, wd, dyd = x.to(dev), w.to(dev), dy.to(dev)
    gy = Guarded(layer.y_shape, td, dev, offset=y_offset)
    gdx = Guarded(layer.x_shape, td, dev)
    gdw = Guarded(layer.w_shape, td, dev)
    y, dx, dw = gy.t, gdx.t, gdw.t
    conv.fwd(xd, wd, y)
    conv.bwd_data(dyd, wd, y, dx)
    conv.bwd_weight(xd, dyd, y, dw)
    torch.cuda.synchronize()
    for gd, name in ((gy, "y"), (gdx, "dx"), (gdw, "dw")):
        gd.check(name)
    return conv, y, dx, dw


def oracle_layer(layer, x, w, dy, y_gpu):
    ym = f64(y_gpu) if layer.relu else None
    y = orc.conv_fwd(f64(x), f64(w), layer.stride, layer.relu)
    dx = orc.conv_bwd_data(f64(dy), f64(w), ym, layer.x_shape, layer.stride, layer.relu)
    dw = orc.conv_bwd_weight(f64(x), f64(dy), ym, layer.w_shape, layer.stride, layer.relu)
    return y, dx, dw


def check_layer(layer, dtype, seeds=(1, 2, 3), x=None, w=None, dy=None, y_offset=0):
    """Full element-by-element parity of all three passes; returns the errors."""
    if x is None:
        x, w, dy = draw(layer, seeds, dtype)
    _, y, dx, dw = gpu_layer(layer, x, w, dy, dtype, y_offset=y_offset)
    y_ref, dx_ref, dw_ref = oracle_layer(layer, x, w, dy, y)
    errs = {"y": rel_err(f64(y), y_ref), "dx": rel_err(f64(dx), dx_ref),
            "dw": rel_err(f64(dw), dw_ref)}
    for k, v in errs.items():
        assert np.isfinite(v) and v <= TOL[dtype], (k, v, errs)
    return errs, (y, dx, dw), (y_ref, dx_ref, dw_ref)
