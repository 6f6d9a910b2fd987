"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds only random-number recipes and the workload table; it does
none of the convolution's arithmetic, and both the HIP path's callers and the
oracle's callers draw from it.  Draws are made on the CPU in fp32 with
``torch.Generator().manual_seed(seed)``; bf16 workloads take the
round-to-nearest-even bf16 value of the same fp32 draw.

Workload shapes are the two policy-network layers benchmarked in "Speedups to
gemm_conv_forward and gemm_conv_backward kernels" (PufferLib pull request
#522, layer-1 and layer-2 benchmark blocks): layer 1 is B=1024, 59->128
channels on an 11x15 input with a 5x5 kernel at stride 3 and a ReLU; layer 2
is B=1024, 128->128 channels on 3x4 with a 3x3 kernel at stride 1, no ReLU.
The page does not state its input distributions; x and dy are drawn N(0,1)
and weights U(-1/sqrt(fan_in), +1/sqrt(fan_in)) with fan_in = IC*KH*KW.
Output shapes are written out literally below, as the workloads state them.
"""
import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class ConvLayer:
    B: int
    IC: int
    H: int
    W: int
    OC: int
    KH: int
    KW: int
    stride: int
    relu: int
    OH: int
    OW: int

    @property
    def x_shape(self):
        return (self.B, self.IC, self.H, self.W)

    @property
    def w_shape(self):
        return (self.OC, self.IC, self.KH, self.KW)

    @property
    def y_shape(self):
        return (self.B, self.OC, self.OH, self.OW)

    @property
    def w_bound(self):
        return 1.0 / math.sqrt(self.IC * self.KH * self.KW)

    def with_batch(self, B):
        return ConvLayer(B, self.IC, self.H, self.W, self.OC, self.KH, self.KW,
                         self.stride, self.relu, self.OH, self.OW)


LAYER1 = ConvLayer(B=1024, IC=59, H=11, W=15, OC=128, KH=5, KW=5, stride=3, relu=1, OH=3, OW=4)
LAYER2 = ConvLayer(B=1024, IC=128, H=3, W=4, OC=128, KH=3, KW=3, stride=1, relu=0, OH=1, OW=2)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": storage type of every tensor
    layers: tuple              # one layer, or the two layers of the chain
    seeds: tuple               # (x, w[, w2], dy)
    note: str = field(default="")


WORKLOADS = (
    Workload("layer2_fp32_b1024", "f32", (LAYER2,), (1, 2, 3),
             "layer-2 shape, fp32, no ReLU"),
    Workload("layer1_fp32_relu_b1024", "f32", (LAYER1,), (11, 12, 13),
             "layer-1 shape, fp32, fused ReLU"),
    Workload("layer1_bf16_relu_b1024", "bf16", (LAYER1,), (11, 12, 13),
             "layer-1 shape, bf16 storage, fp32 accumulation, fused ReLU"),
    Workload("layer2_bf16_b1024", "bf16", (LAYER2,), (1, 2, 3),
             "layer-2 shape, bf16 storage, fp32 accumulation"),
    Workload("chain_bf16_b16384", "bf16", (LAYER1.with_batch(16384), LAYER2.with_batch(16384)),
             (41, 42, 43, 44), "conv1 (ReLU) -> conv2, bf16, B=16384"),
    Workload("chain_bf16_b32768", "bf16", (LAYER1.with_batch(32768), LAYER2.with_batch(32768)),
             (51, 52, 53, 54), "conv1 (ReLU) -> conv2, bf16, B=32768, the encoder's batch"),
)


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal(shape, seed, dtype="f32"):
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return t.to(torch_dtype(dtype))


def uniform(shape, seed, bound, dtype="f32"):
    g = torch.Generator().manual_seed(int(seed))
    t = torch.rand(tuple(shape), generator=g, dtype=torch.float32)
    t = (t * 2.0 - 1.0) * float(bound)
    return t.to(torch_dtype(dtype))


def integers(shape, seed, lo=-2, hi=2, dtype="f32"):
    """Integer values in [lo, hi]; sums of their products stay exact in fp32."""
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randint(lo, hi + 1, tuple(shape), generator=g).to(torch.float32)
    return t.to(torch_dtype(dtype))


def layer_inputs(layer, seeds, dtype="f32"):
    """(x, w, dy) CPU tensors for one layer, drawn from the workload recipe."""
    sx, sw, sdy = seeds
    x = normal(layer.x_shape, sx, dtype)
    w = uniform(layer.w_shape, sw, layer.w_bound, dtype)
    dy = normal(layer.y_shape, sdy, dtype)
    return x, w, dy


def workload_inputs(wl):
    """CPU tensors for a workload: dict with x, w (or w1, w2) and dy."""
    if len(wl.layers) == 1:
        x, w, dy = layer_inputs(wl.layers[0], wl.seeds, wl.dtype)
        return {"x": x, "w": w, "dy": dy}
    l1, l2 = wl.layers
    sx, sw1, sw2, sdy = wl.seeds
    return {
        "x": normal(l1.x_shape, sx, wl.dtype),
        "w1": uniform(l1.w_shape, sw1, l1.w_bound, wl.dtype),
        "w2": uniform(l2.w_shape, sw2, l2.w_bound, wl.dtype),
        "dy": normal(l2.y_shape, sdy, wl.dtype),
    }
