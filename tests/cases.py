"""Batch sizes the GPU parity tests run for the two policy-network layer
shapes of "Speedups to gemm_conv_forward and gemm_conv_backward kernels"
(PufferLib pull request #522, layer-1 and layer-2 benchmark blocks), and the
kernel instances the library can pick for those shapes.

The planners choose a compiled kernel instance per batch size (images per
workgroup, channel groups per staging phase, ...).  LAYER_BATCHES is chosen
so that the GPU tests reach every instance in INSTANCES -- the set a sweep of
every batch size from 1 to 4200 and a sample up to 40000 reaches -- and a CPU
test checks that both still hold through gc_conv_plan_name.
"""
LAYER_SHAPES = {
    # IC, H, W, OC, KH, KW, stride, relu
    "layer1": (59, 11, 15, 128, 5, 5, 3, 1),
    "layer2": (128, 3, 4, 128, 3, 3, 1, 0),
}

# (layer, dtype) -> batch sizes run element by element against the oracle
LAYER_BATCHES = {
    ("layer1", "f32"): (64, 512, 600, 800, 1024),
    ("layer1", "bf16"): (64, 512, 600, 800, 1024, 4096),
    ("layer2", "f32"): (64, 400, 512, 600, 1024, 2048, 4096),
    ("layer2", "bf16"): (8, 64, 639, 1024, 1227, 1542, 2048, 4096, 16384),
}

# (layer, dtype, op) -> kernel instances (family<compile-time parameters>)
INSTANCES = {
    ("layer1", "f32", "fwd"): {
        "fwd_ws_f32<NWM=8,MB=1,TS=7,NCG=15,CPP=12,LO=1>",
        "fwd_ws_f32<NWM=8,MB=2,TS=7,NCG=15,CPP=6,LO=1>",
        "fwd_ws_f32<NWM=8,MB=3,TS=7,NCG=15,CPP=3,LO=1>",
    },
    ("layer1", "f32", "bwd_data"): {"dgrad_rf_f32<MB=3,KS4=8,TAPS=4>"},
    ("layer1", "f32", "bwd_weight"): {"wgrad_rf_f32<NBWV=3>", "wgrad_rf_f32<NBWV=6>"},
    ("layer1", "bf16", "fwd"): {
        "fwd_ws_bf16<NBW=2,MB=1,TS=7,NCG=8,CPP=8>",
        "fwd_ws_bf16<NBW=1,MB=3,TS=7,NCG=8,CPP=3>",
        "fwd_ws_bf16<NBW=2,MB=3,TS=7,NCG=8,CPP=3>",
    },
    ("layer1", "bf16", "bwd_data"): {
        "dgrad_ig_bf16<MB=3,KS=4,TAPS=4,NBW=1>",
        "dgrad_ig_bf16<MB=3,KS=4,TAPS=4,NBW=2>",
    },
    ("layer1", "bf16", "bwd_weight"): {"wgrad_ws_bf16<NSTEP=3,JW=2>", "wgrad_ws_bf16<NSTEP=3,JW=4>"},
    ("layer2", "f32", "fwd"): {
        "fwd_ws_f32<NWM=4,MB=1,TS=3,NCG=32,CPP=32,LO=1>",
        "fwd_ws_f32<NWM=4,MB=1,TS=3,NCG=32,CPP=21,LO=1>",
        "fwd_ws_f32<NWM=4,MB=1,TS=3,NCG=32,CPP=10,LO=1>",
        "fwd_ws_f32<NWM=4,MB=2,TS=3,NCG=32,CPP=5,LO=1>",
        "fwd_ws_f32<NWM=4,MB=4,TS=3,NCG=32,CPP=2,LO=1>",
    },
    ("layer2", "f32", "bwd_data"): {
        "dgrad_rf_f32<MB=1,KS4=8,TAPS=2>",
        "dgrad_rf_f32<MB=2,KS4=8,TAPS=2>",
        "dgrad_rf_f32<MB=3,KS4=8,TAPS=2>",
    },
    ("layer2", "f32", "bwd_weight"): {"wgrad_rf_f32<NBWV=3>"},
    ("layer2", "bf16", "fwd"): {
        "fwd_ws_bf16<NBW=1,MB=1,TS=3,NCG=16,CPP=16>",
        "fwd_ws_bf16<NBW=1,MB=2,TS=3,NCG=16,CPP=8>",
        "fwd_ws_bf16<NBW=1,MB=4,TS=3,NCG=16,CPP=4>",
    },
    ("layer2", "bf16", "bwd_data"): {
        "dgrad_ig_bf16<MB=1,KS=4,TAPS=2,NBW=1>",
        "dgrad_ig_bf16<MB=2,KS=4,TAPS=2,NBW=1>",
        "dgrad_ig_bf16<MB=2,KS=4,TAPS=2,NBW=2>",
        "dgrad_ig_bf16<MB=3,KS=4,TAPS=2,NBW=1>",
        "dgrad_ig_bf16<MB=3,KS=4,TAPS=2,NBW=2>",
        "dgrad_ig_bf16<MB=4,KS=4,TAPS=2,NBW=1>",
    },
    ("layer2", "bf16", "bwd_weight"): {"wgrad_ws_bf16<NSTEP=1,JW=2>", "wgrad_ws_bf16<NSTEP=1,JW=4>"},
}

# batch sizes other GPU tests run for these shapes (the workload table at
# B=1024, the several-groups tests, the chain at 16384 and 32768, smoke at 8)
OTHER_GPU_BATCHES = {
    "layer1": (8, 1024, 2054, 16384, 32768),
    "layer2": (1024, 8300, 16384, 32768),
}


# gc_conv_bwd in fp32 runs the d_input and wgrad bodies in one launch; each
# (d_input, wgrad) pair the planners can pick for the layer shapes -> a
# (layer, batch size) case that reaches it (run with and without the ReLU,
# which selects a kernel of its own)
FUSED_F32_BWD = {
    "bwd_fused_f32: dgrad_rf_f32<MB=3,KS4=8,TAPS=4> + wgrad_rf_f32<NBWV=3>": ("layer1", 97),
    "bwd_fused_f32: dgrad_rf_f32<MB=3,KS4=8,TAPS=4> + wgrad_rf_f32<NBWV=6>": ("layer1", 250),
    "bwd_fused_f32: dgrad_rf_f32<MB=1,KS4=8,TAPS=2> + wgrad_rf_f32<NBWV=3>": ("layer2", 66),
    "bwd_fused_f32: dgrad_rf_f32<MB=2,KS4=8,TAPS=2> + wgrad_rf_f32<NBWV=3>": ("layer2", 203),
    "bwd_fused_f32: dgrad_rf_f32<MB=3,KS4=8,TAPS=2> + wgrad_rf_f32<NBWV=3>": ("layer2", 409),
}


# gc_conv_bwd in bf16 for the layer shapes: each fused form the planners can
# pick (one pre-pass, then the two main grids in one launch or one after the
# other) -> a (layer, batch size) case that reaches it
FUSED_BF16_BWD = {
    "bwd_fused_bf16 fuse_main=0: dgrad_ig_bf16<MB=3,KS=4,TAPS=4,NBW=1> + wgrad_ws_bf16<NSTEP=3,JW=2>":
        ("layer1", 205),
    "bwd_fused_bf16 fuse_main=0: dgrad_ig_bf16<MB=3,KS=4,TAPS=4,NBW=1> + wgrad_ws_bf16<NSTEP=3,JW=4>":
        ("layer1", 2130),
    "bwd_fused_bf16 fuse_main=1: dgrad_ig_bf16<MB=2,KS=4,TAPS=2,NBW=2> + wgrad_ws_bf16<NSTEP=1,JW=2>":
        ("layer2", 9),
    "bwd_fused_bf16 fuse_main=1: dgrad_ig_bf16<MB=3,KS=4,TAPS=2,NBW=1> + wgrad_ws_bf16<NSTEP=1,JW=2>":
        ("layer2", 17),
    "bwd_fused_bf16 fuse_main=0: dgrad_ig_bf16<MB=2,KS=4,TAPS=2,NBW=2> + wgrad_ws_bf16<NSTEP=1,JW=2>":
        ("layer2", 3290),
    "bwd_fused_bf16 fuse_main=0: dgrad_ig_bf16<MB=3,KS=4,TAPS=2,NBW=1> + wgrad_ws_bf16<NSTEP=1,JW=2>":
        ("layer2", 4102),
    "bwd_fused_bf16 fuse_main=0: dgrad_ig_bf16<MB=2,KS=4,TAPS=2,NBW=2> + wgrad_ws_bf16<NSTEP=1,JW=4>":
        ("layer2", 15167),
    "bwd_fused_bf16 fuse_main=0: dgrad_ig_bf16<MB=3,KS=4,TAPS=2,NBW=1> + wgrad_ws_bf16<NSTEP=1,JW=4>":
        ("layer2", 17161),
}


def fused_pair(plan_name):
    """'bwd_fused_f32: <d_input instance> + <wgrad instance>' of a
    gc_conv_bwd plan name (the per-batch parameters dropped)."""
    head, _, rest = plan_name.partition(": ")
    d, _, w = rest.partition(" + ")
    return f"{head}: {instance_key(d)} + {instance_key(w)}"


def instance_key(plan_name):
    """The kernel instance of one part of a plan name: 'family<...>', or the
    bare family name for kernels without compile-time parameters."""
    head = plan_name.strip().split(" ")[0]
    return head
