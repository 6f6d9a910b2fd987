"""Which kernels the library runs, checked on the host through
gc_conv_plan_name (no GPU needed).

For the two policy-network layer shapes of "Speedups to gemm_conv_forward
and gemm_conv_backward kernels" (PufferLib pull request #522) the
shape-generic fallback must never run, at any batch size the encoder uses,
and every kernel instance the planners can pick must be one the GPU parity
tests run (tests/cases.py lists both).
"""
import pytest

from backward_implicit_gemm_amd import binding as gb

from cases import (FUSED_BF16_BWD, FUSED_F32_BWD, INSTANCES, LAYER_BATCHES, LAYER_SHAPES, OTHER_GPU_BATCHES,
                   fused_pair, instance_key)

OPS = {"fwd": gb.GC_OP_FWD, "bwd_data": gb.GC_OP_BWD_DATA, "bwd_weight": gb.GC_OP_BWD_WEIGHT,
       "bwd": gb.GC_OP_BWD}
DT = {"f32": gb.GC_F32, "bf16": gb.GC_BF16}


def plan(layer, B, dtype, op):
    IC, H, W, OC, KH, KW, S, _ = LAYER_SHAPES[layer]
    return gb.gc_conv_plan_name(OPS[op], gb.make_desc(B, IC, H, W, OC, KH, KW, S), DT[dtype])


def keys(layer, dtype, op, batches):
    return {instance_key(plan(layer, B, dtype, op)) for B in batches}


def test_plan_name_errors():
    import ctypes
    L = gb.lib()
    d = gb.make_desc(4, 3, 5, 5, 2, 3, 3, 1)
    buf = ctypes.create_string_buffer(8)
    assert L.gc_conv_plan_name(gb.GC_OP_FWD, ctypes.byref(d), gb.GC_F32, None, 8) == gb.GC_ERR_INVALID_ARG
    assert L.gc_conv_plan_name(gb.GC_OP_FWD, ctypes.byref(d), gb.GC_F32, buf, 0) == gb.GC_ERR_INVALID_ARG
    assert L.gc_conv_plan_name(99, ctypes.byref(d), gb.GC_F32, buf, 8) == gb.GC_ERR_INVALID_ARG
    assert L.gc_conv_plan_name(gb.GC_OP_FWD, ctypes.byref(d), 7, buf, 8) == gb.GC_ERR_INVALID_ARG
    bad = gb.make_desc(4, 3, 2, 5, 2, 3, 3, 1)
    assert L.gc_conv_plan_name(gb.GC_OP_FWD, ctypes.byref(bad), gb.GC_F32, buf, 8) == gb.GC_ERR_INVALID_ARG
    # truncated, but NUL-terminated
    assert L.gc_conv_plan_name(gb.GC_OP_FWD, ctypes.byref(d), gb.GC_F32, buf, 8) == gb.GC_OK
    assert len(buf.value) == 7


def test_policy_generic_is_reported():
    prev = gb.gc_set_kernel_policy(gb.GC_POLICY_GENERIC)
    try:
        assert plan("layer1", 1024, "bf16", "fwd") == "igemm_generic_fwd"
        assert plan("layer1", 1024, "f32", "bwd_data") == "igemm_generic_dgrad"
        assert plan("layer2", 1024, "bf16", "bwd_weight").startswith("igemm_generic_wgrad")
    finally:
        gb.gc_set_kernel_policy(prev)


def test_headline_plans():
    # the kernels the B=1024 workloads run (the bench's per-call figures)
    assert plan("layer1", 1024, "f32", "fwd").startswith("fwd_ws_f32<NWM=8,MB=3,TS=7,NCG=15,CPP=3,LO=1> G=4")
    assert plan("layer1", 1024, "f32", "bwd_weight").startswith("wgrad_rf_f32<NBWV=6>")
    assert plan("layer1", 1024, "bf16", "fwd").startswith("fwd_ws_bf16<NBW=2,MB=3,TS=7,NCG=8,CPP=3> G=4")
    assert plan("layer2", 1024, "bf16", "fwd").startswith("fwd_ws_bf16<NBW=1,MB=1,TS=3,NCG=16,CPP=16> G=8")


ENCODER_BATCHES = (256, 512, 768, 1024, 2048, 4096, 8192, 16384, 32768)


@pytest.mark.parametrize("layer", sorted(LAYER_SHAPES))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_shapes_never_run_the_generic_kernels(layer, dtype):
    for B in ENCODER_BATCHES:
        for op in (gb.GC_OP_FWD, gb.GC_OP_BWD_DATA, gb.GC_OP_BWD_WEIGHT, gb.GC_OP_BWD):
            IC, H, W, OC, KH, KW, S, _ = LAYER_SHAPES[layer]
            name = gb.gc_conv_plan_name(op, gb.make_desc(B, IC, H, W, OC, KH, KW, S), DT[dtype])
            assert "generic" not in name, (layer, dtype, B, op, name)


def _sweep():
    # every batch size up to 70, then a stride-29 walk to 4200 plus the
    # points where the planners switch, then a sample up to 40000
    s = set(range(1, 71)) | set(range(71, 4200, 29)) | set(range(4200, 40000, 997))
    s |= {205, 226, 387, 415, 510, 511, 512, 513, 618, 639, 765, 766, 772, 1016, 1017, 1020,
          1021, 1227, 1542, 2033, 2039, 4065, 4069}
    return sorted(s)


@pytest.mark.parametrize("key", sorted(INSTANCES), ids=["-".join(k) for k in sorted(INSTANCES)])
def test_every_reachable_instance_is_gpu_tested(key):
    layer, dtype, op = key
    tested = keys(layer, dtype, op, LAYER_BATCHES[(layer, dtype)])
    # the GPU batch list reaches exactly the listed instances ...
    assert tested == INSTANCES[key], (tested ^ INSTANCES[key])
    # ... and a sweep of batch sizes reaches no other
    reached = keys(layer, dtype, op, _sweep())
    assert reached <= INSTANCES[key], reached - INSTANCES[key]
    for B in OTHER_GPU_BATCHES[layer]:
        assert instance_key(plan(layer, B, dtype, op)) in INSTANCES[key]


def test_fp32_backward_is_fused_and_every_pair_is_gpu_tested():
    # gc_conv_bwd in fp32 takes the one-launch path at every batch size of
    # both layer shapes, and each (d_input, wgrad) pair it can pick has a
    # GPU case
    for layer in LAYER_SHAPES:
        for B in _sweep():
            name = plan(layer, B, "f32", "bwd")
            assert fused_pair(name) in FUSED_F32_BWD, (layer, B, name)
    for pair, (layer, B) in FUSED_F32_BWD.items():
        assert fused_pair(plan(layer, B, "f32", "bwd")) == pair


def test_forward_planners_respect_the_pack_grid_limit():
    # the forward's weight packing runs one grid row per 16-channel block, so
    # more than 65535 blocks must go to the shape-generic kernel
    for dt in (gb.GC_F32, gb.GC_BF16):
        # layer 1's geometry (59 -> OC, 11x15, 5x5, stride 3) with a huge OC
        big = gb.gc_conv_plan_name(gb.GC_OP_FWD, gb.make_desc(1, 59, 11, 15, 65536 * 16, 5, 5, 3), dt)
        assert big == "igemm_generic_fwd", big
        ok = gb.gc_conv_plan_name(gb.GC_OP_FWD, gb.make_desc(1, 59, 11, 15, 65535 * 16, 5, 5, 3), dt)
        assert ok.startswith("fwd_ws_"), ok


def test_every_bf16_fused_backward_form_is_gpu_tested():
    # gc_conv_bwd in bf16 takes a fused form (or the separate calls, which the
    # per-pass tests cover) at every batch size; each fused form it can pick
    # for the layer shapes has a GPU case
    for layer in LAYER_SHAPES:
        for B in _sweep():
            name = plan(layer, B, "bf16", "bwd")
            if name.startswith("bwd_fused_bf16"):
                assert fused_pair(name) in FUSED_BF16_BWD, (layer, B, name)
    for form, (layer, B) in FUSED_BF16_BWD.items():
        assert fused_pair(plan(layer, B, "bf16", "bwd")) == form
