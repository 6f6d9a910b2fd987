"""Host-side checks of libgc's C ABI (no GPU needed).

The library must load and export every function include/gc.h declares; the
pure-host entry points (output size, workspace size, status strings, the
index-mapper self-check) must be right; and every invalid call must be
rejected before the first HIP call, which is why these run without a GPU.
"""
import ctypes
import os
import re

import pytest

from backward_implicit_gemm_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(gc_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gc_conv_fwd", "gc_conv_bwd_data", "gc_conv_bwd_weight"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = gb.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(gb.EXPORTED)


def test_out_dims_page1_layers():
    assert gb.gc_conv_out_dims(gb.make_desc(1024, 59, 11, 15, 128, 5, 5, 3)) == (3, 4)
    assert gb.gc_conv_out_dims(gb.make_desc(1024, 128, 3, 4, 128, 3, 3, 1)) == (1, 2)
    assert gb.gc_conv_out_dims(gb.make_desc(1, 1, 7, 9, 1, 2, 3, 2)) == (3, 4)


@pytest.mark.parametrize("bad", [
    (0, 1, 3, 3, 1, 3, 3, 1), (1, 0, 3, 3, 1, 3, 3, 1), (1, 1, 2, 3, 1, 3, 3, 1),
    (1, 1, 3, 2, 1, 3, 3, 1), (1, 1, 3, 3, 0, 3, 3, 1), (1, 1, 3, 3, 1, 3, 3, 0),
    (1, 1, 3, 3, 1, 0, 3, 1), (-1, 1, 3, 3, 1, 3, 3, 1),
    (1 << 16, 1 << 10, 64, 64, 1, 1, 1, 1),      # B*IC*H*W >= 2^31
    (1 << 20, 1, 1, 1, 4096, 1, 1, 1),          # B*OC*OH*OW >= 2^31
])
def test_invalid_descriptors_rejected(bad):
    d = gb.make_desc(*bad)
    oh, ow = ctypes.c_int(), ctypes.c_int()
    assert gb.lib().gc_conv_out_dims(ctypes.byref(d), ctypes.byref(oh), ctypes.byref(ow)) == gb.GC_ERR_INVALID_ARG
    assert gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_WEIGHT, d, gb.GC_F32) == 0


def test_null_descriptor_rejected():
    L = gb.lib()
    assert L.gc_conv_out_dims(None, None, None) == gb.GC_ERR_INVALID_ARG
    assert L.gc_conv_fwd(None, None, None, None, 0, None, 0, 0, None) == gb.GC_ERR_INVALID_ARG


FAKE = ctypes.c_void_p(0x10000)    # never dereferenced: every call below fails validation


def _call(fn, *ptrs, desc, relu, dtype, ws=None, ws_bytes=0):
    L = gb.lib()
    return getattr(L, fn)(*ptrs, ws, ws_bytes, ctypes.byref(desc), relu, dtype, None)


L1 = gb.make_desc(1024, 59, 11, 15, 128, 5, 5, 3)


def test_fwd_argument_errors():
    assert _call("gc_conv_fwd", None, FAKE, FAKE, desc=L1, relu=1, dtype=0) == gb.GC_ERR_INVALID_ARG
    assert _call("gc_conv_fwd", FAKE, FAKE, None, desc=L1, relu=1, dtype=0) == gb.GC_ERR_INVALID_ARG
    assert _call("gc_conv_fwd", FAKE, FAKE, FAKE, desc=L1, relu=2, dtype=0) == gb.GC_ERR_INVALID_ARG
    assert _call("gc_conv_fwd", FAKE, FAKE, FAKE, desc=L1, relu=0, dtype=7) == gb.GC_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x10002)
    assert _call("gc_conv_fwd", odd, FAKE, FAKE, desc=L1, relu=0, dtype=gb.GC_F32) == gb.GC_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x10001)
    assert _call("gc_conv_fwd", odd, FAKE, FAKE, desc=L1, relu=0, dtype=gb.GC_BF16) == gb.GC_ERR_INVALID_ARG
    bad = gb.make_desc(1, 1, 2, 2, 1, 3, 3, 1)
    assert _call("gc_conv_fwd", FAKE, FAKE, FAKE, desc=bad, relu=0, dtype=0) == gb.GC_ERR_INVALID_ARG


def test_backward_mask_must_match_relu():
    # relu=1 needs y_mask; relu=0 forbids it
    assert _call("gc_conv_bwd_data", FAKE, FAKE, None, FAKE, desc=L1, relu=1, dtype=0) == gb.GC_ERR_INVALID_ARG
    assert _call("gc_conv_bwd_data", FAKE, FAKE, FAKE, FAKE, desc=L1, relu=0, dtype=0) == gb.GC_ERR_INVALID_ARG
    assert _call("gc_conv_bwd_weight", FAKE, FAKE, None, FAKE, desc=L1, relu=1, dtype=0) == gb.GC_ERR_INVALID_ARG
    assert _call("gc_conv_bwd_weight", FAKE, FAKE, FAKE, FAKE, desc=L1, relu=0, dtype=0) == gb.GC_ERR_INVALID_ARG


def test_wgrad_workspace_errors():
    need = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_WEIGHT, L1, gb.GC_BF16)
    assert need > 0
    assert _call("gc_conv_bwd_weight", FAKE, FAKE, FAKE, FAKE, desc=L1, relu=1, dtype=gb.GC_BF16,
                 ws=None, ws_bytes=0) == gb.GC_ERR_WORKSPACE
    assert _call("gc_conv_bwd_weight", FAKE, FAKE, FAKE, FAKE, desc=L1, relu=1, dtype=gb.GC_BF16,
                 ws=FAKE, ws_bytes=need - 1) == gb.GC_ERR_WORKSPACE


def test_workspace_sizes_are_sane():
    for d in (L1, gb.make_desc(1024, 128, 3, 4, 128, 3, 3, 1), gb.make_desc(3, 2, 5, 5, 3, 2, 2, 1)):
        K = d.IC * d.KH * d.KW
        OH, OW = gb.gc_conv_out_dims(d)
        # regrouped dz: images padded to 8, channels to 128, positions to 4
        dz_bytes = (d.B + 7) // 8 * 8 * max(d.OC, 128) * ((OH * OW + 3) // 4 * 4) * 2 + 256
        for dt in (gb.GC_F32, gb.GC_BF16):
            n = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_WEIGHT, d, dt)
            # fp32 partial tiles (at least one), plus for bf16 at most a
            # regrouped copy of dz (positions and channels padded)
            assert n >= d.OC * K * 4
            if dt == gb.GC_F32:
                assert n % (d.OC * K * 4) == 0 and n <= 64 * d.OC * K * 4
            else:
                assert n <= 64 * d.OC * K * 4 + dz_bytes
        # packed weights for the bf16 forward and d_input kernels: a padded copy of w
        for op, dt, es in ((gb.GC_OP_FWD, gb.GC_BF16, 2), (gb.GC_OP_BWD_DATA, gb.GC_BF16, 2),
                           (gb.GC_OP_FWD, gb.GC_F32, 4), (gb.GC_OP_BWD_DATA, gb.GC_F32, 4)):
            n = gb.gc_conv_workspace_bytes(op, d, dt)
            assert n == 0 or d.OC * K * es <= n <= 16 * max(d.OC, 32) * max(K, 64) * es
    assert gb.gc_conv_workspace_bytes(99, L1, 0) == 0


def test_dgrad_workspace_errors():
    # the fp32 d_input kernel reads the weights in place; bf16 packs them
    assert gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_DATA, L1, gb.GC_F32) == 0
    dtype = gb.GC_BF16
    need = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_DATA, L1, dtype)
    assert need > 0
    assert _call("gc_conv_bwd_data", FAKE, FAKE, FAKE, FAKE, desc=L1, relu=1, dtype=dtype,
                 ws=None, ws_bytes=0) == gb.GC_ERR_WORKSPACE
    assert _call("gc_conv_bwd_data", FAKE, FAKE, FAKE, FAKE, desc=L1, relu=1, dtype=dtype,
                 ws=FAKE, ws_bytes=need - 1) == gb.GC_ERR_WORKSPACE


def test_bias_argument_errors():
    lib = gb.lib()
    d = L1
    # fwd_bias needs a bias pointer; the rest is validated as for gc_conv_fwd
    assert lib.gc_conv_fwd_bias(FAKE, FAKE, None, FAKE, None, 0, ctypes.byref(d), 1, 0,
                                None) == gb.GC_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x10002)
    assert lib.gc_conv_fwd_bias(FAKE, FAKE, odd, FAKE, None, 0, ctypes.byref(d), 1, gb.GC_F32,
                                None) == gb.GC_ERR_INVALID_ARG
    assert gb.gc_conv_workspace_bytes(gb.GC_OP_FWD, d, gb.GC_BF16) > 0
    assert lib.gc_conv_fwd_bias(FAKE, FAKE, FAKE, FAKE, None, 0, ctypes.byref(d), 1, gb.GC_BF16,
                                None) == gb.GC_ERR_WORKSPACE
    # bwd_bias: the mask must match relu; null outputs and bad flags are rejected
    def bb(dy, m, db, relu, dt, desc=d, ws=FAKE, wn=1 << 30):
        return lib.gc_conv_bwd_bias(dy, m, db, ws, wn, ctypes.byref(desc), relu, dt, None)
    assert bb(FAKE, None, FAKE, 1, 0) == gb.GC_ERR_INVALID_ARG
    assert bb(FAKE, FAKE, FAKE, 0, 0) == gb.GC_ERR_INVALID_ARG
    assert bb(FAKE, FAKE, None, 1, 0) == gb.GC_ERR_INVALID_ARG
    assert bb(FAKE, FAKE, FAKE, 2, 0) == gb.GC_ERR_INVALID_ARG
    assert bb(FAKE, FAKE, FAKE, 1, 5) == gb.GC_ERR_INVALID_ARG
    assert bb(FAKE, None, FAKE, 0, 0, desc=gb.make_desc(1, 1, 2, 2, 1, 3, 3, 1)) == gb.GC_ERR_INVALID_ARG
    need = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_BIAS, d, gb.GC_F32)
    assert need >= d.OC * 4
    assert bb(FAKE, FAKE, FAKE, 1, 0, ws=None, wn=0) == gb.GC_ERR_WORKSPACE
    assert bb(FAKE, FAKE, FAKE, 1, 0, wn=need - 1) == gb.GC_ERR_WORKSPACE


def test_status_strings():
    for s in range(5):
        assert gb.status_string(s).startswith("GC_")
    assert "unknown" in gb.status_string(42)


# Divisors the kernels split by at the page's layer shapes and the chain:
# P = OH*OW, OW, KK = KH*KW, KW, HW = H*W, W, S.
LAYER_DIVISORS = [12, 4, 25, 5, 165, 15, 3, 2, 9, 1]


@pytest.mark.parametrize("d", LAYER_DIVISORS)
def test_fastdiv_exhaustive_over_used_ranges(d):
    # largest numerator: B*H*W at B=32768 on the 11x15 input (5.4M), doubled
    assert gb.lib().gc_fastdiv_selfcheck(d, 11_000_000) == 0


@pytest.mark.parametrize("d", [1, 3, 7, 1475, 1152, 9735, 65537, 2**31 - 1, 2**30 + 3])
def test_fastdiv_random_divisors_prefix(d):
    assert gb.lib().gc_fastdiv_selfcheck(d, 4_000_000) == 0


@pytest.mark.slow
@pytest.mark.parametrize("d", [3, 165])
def test_fastdiv_full_31bit_range(d):
    assert gb.lib().gc_fastdiv_selfcheck(d, 2**31) == 0


def test_fastdiv_rejects_bad_args():
    assert gb.lib().gc_fastdiv_selfcheck(0, 10) == -1
    assert gb.lib().gc_fastdiv_selfcheck(3, 2**31 + 1) == -1


def test_version():
    assert gb.lib().gc_version() >= 100


def _bwd(*ptrs, desc, relu, dtype, ws=None, ws_bytes=0):
    return gb.lib().gc_conv_bwd(*ptrs, ws, ws_bytes, ctypes.byref(desc), relu, dtype, None)


L2 = gb.make_desc(1024, 128, 3, 4, 128, 3, 3, 1)


@pytest.mark.parametrize("dtype", [gb.GC_F32, gb.GC_BF16])
def test_bwd_argument_errors(dtype):
    F = FAKE
    for i in range(5):      # each of x, w, dy, dx, dw missing
        ptrs = [F, F, F, F, F]
        ptrs[i] = None
        x, w, dy, dx, dw = ptrs
        assert _bwd(x, w, dy, F, dx, dw, desc=L1, relu=1, dtype=dtype) == gb.GC_ERR_INVALID_ARG
    assert _bwd(F, F, F, None, F, F, desc=L1, relu=1, dtype=dtype) == gb.GC_ERR_INVALID_ARG
    assert _bwd(F, F, F, F, F, F, desc=L2, relu=0, dtype=dtype) == gb.GC_ERR_INVALID_ARG
    assert _bwd(F, F, F, F, F, F, desc=L1, relu=3, dtype=dtype) == gb.GC_ERR_INVALID_ARG
    for d, relu, m in ((L1, 1, F), (L2, 0, None)):
        need = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD, d, dtype)
        assert need > 0
        assert _bwd(F, F, F, m, F, F, desc=d, relu=relu, dtype=dtype) == gb.GC_ERR_WORKSPACE
        assert _bwd(F, F, F, m, F, F, desc=d, relu=relu, dtype=dtype,
                    ws=F, ws_bytes=need - 1) == gb.GC_ERR_WORKSPACE
        off = ctypes.c_void_p(0x10010)     # 16- but not 256-byte aligned
        assert _bwd(F, F, F, m, F, F, desc=d, relu=relu, dtype=dtype,
                    ws=off, ws_bytes=need) == gb.GC_ERR_WORKSPACE


def test_bwd_workspace_covers_both_passes():
    for d in (L1, L2, gb.make_desc(16384, 59, 11, 15, 128, 5, 5, 3),
              gb.make_desc(16384, 128, 3, 4, 128, 3, 3, 1), gb.make_desc(3, 2, 5, 5, 3, 2, 2, 1)):
        for dt in (gb.GC_F32, gb.GC_BF16):
            nd = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_DATA, d, dt)
            nw = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_WEIGHT, d, dt)
            n = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD, d, dt)
            assert max(nd, nw) <= n <= nd + nw + 256, (d.B, d.IC, dt, nd, nw, n)


# ---------------------------------------------------------------------------
# The Python binding checks every tensor's shape against the problem before
# anything reaches the device (so these run on host tensors, without a GPU)
# ---------------------------------------------------------------------------

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float32)


def test_binding_rejects_wrong_output_shapes():
    x, w = _t(4, 59, 11, 15), _t(128, 59, 5, 5)
    with pytest.raises(ValueError, match="y has shape"):
        gb.gc_conv_fwd(x, w, _t(5, 128, 3, 4), relu=1, stride=3)
    with pytest.raises(ValueError, match="y has shape"):
        gb.gc_conv_fwd_bias(x, w, _t(128), _t(4, 128, 4, 4), relu=1, stride=3)
    with pytest.raises(ValueError, match="bias has shape"):
        gb.gc_conv_fwd_bias(x, w, _t(127), _t(4, 128, 3, 4), relu=1, stride=3)


def test_binding_rejects_wrong_backward_shapes():
    x, w, y = _t(4, 59, 11, 15), _t(128, 59, 5, 5), _t(4, 128, 3, 4)
    dx, dw = _t(4, 59, 11, 15), _t(128, 59, 5, 5)
    with pytest.raises(ValueError, match="dy has shape"):
        gb.gc_conv_bwd_data(_t(8, 128, 3, 4), w, y, dx, relu=1, stride=3)
    with pytest.raises(ValueError, match="y_mask has shape"):
        gb.gc_conv_bwd_data(y, w, _t(4, 128, 3, 3), dx, relu=1, stride=3)
    with pytest.raises(ValueError, match="dy has shape"):
        gb.gc_conv_bwd_weight(x, _t(4, 128, 1, 2), y, dw, relu=1, stride=3, workspace=None)
    with pytest.raises(ValueError, match="dx has shape"):
        gb.gc_conv_bwd(x, w, y, y, _t(4, 59, 11, 14), dw, relu=1, stride=3, workspace=None)
    with pytest.raises(ValueError, match="dw has shape"):
        gb.gc_conv_bwd(x, w, y, y, dx, _t(128, 59, 5, 4), relu=1, stride=3, workspace=None)
    with pytest.raises(ValueError, match="db has shape"):
        gb.gc_conv_bwd_bias(y, y, _t(64), relu=1, x_shape=x.shape, w_shape=w.shape, stride=3,
                            workspace=None)
    with pytest.raises(ValueError, match="channels"):
        gb.gc_conv_fwd(x, _t(128, 58, 5, 5), y, relu=1, stride=3)


def test_binding_reaches_the_device_check_with_right_shapes():
    # with every shape right, the next check is that tensors live on the GPU
    x, w, y = _t(4, 59, 11, 15), _t(128, 59, 5, 5), _t(4, 128, 3, 4)
    with pytest.raises(ValueError, match="device tensor"):
        gb.gc_conv_fwd(x, w, y, relu=1, stride=3)


def test_noalloc_forward_rejects_before_any_launch():
    # validation and the scratch-size check come before anything is enqueued,
    # so they run without a GPU (FAKE pointers are never touched)
    L = gb.lib()
    big = gb.make_desc(2, 59, 11, 15, 512, 5, 5, 3)      # layer 1 with 512 output channels
    assert gb.gc_conv_workspace_bytes(gb.GC_OP_FWD, big, gb.GC_F32) > (2 << 20)
    assert L.gc_conv_fwd_noalloc(FAKE, FAKE, FAKE, ctypes.byref(big), 0, gb.GC_F32, None) == gb.GC_ERR_WORKSPACE
    assert L.gc_conv_fwd_noalloc(None, FAKE, FAKE, ctypes.byref(L1), 1, gb.GC_F32, None) == gb.GC_ERR_INVALID_ARG
    assert L.gc_conv_fwd_noalloc(FAKE, FAKE, FAKE, ctypes.byref(L1), 2, gb.GC_F32, None) == gb.GC_ERR_INVALID_ARG
    assert L.gc_conv_fwd_noalloc(FAKE, FAKE, FAKE, None, 1, gb.GC_F32, None) == gb.GC_ERR_INVALID_ARG
    # both page-1 layer shapes fit the scratch at any batch size
    for B in (1, 1024, 32768):
        for shape in ((59, 11, 15, 128, 5, 5, 3), (128, 3, 4, 128, 3, 3, 1)):
            for dt in (gb.GC_F32, gb.GC_BF16):
                assert gb.gc_conv_workspace_bytes(gb.GC_OP_FWD, gb.make_desc(B, *shape), dt) <= (2 << 20)


def test_wgrad_bias_argument_errors():
    L = gb.lib()
    call = lambda *p, relu=1, dt=0, ws=None, wsb=0: L.gc_conv_bwd_weight_bias(
        *p, ws, wsb, ctypes.byref(L1), relu, dt, None)
    assert call(FAKE, FAKE, FAKE, FAKE, None) == gb.GC_ERR_INVALID_ARG          # db NULL
    assert call(FAKE, FAKE, None, FAKE, FAKE) == gb.GC_ERR_INVALID_ARG          # relu without mask
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, relu=0) == gb.GC_ERR_INVALID_ARG  # mask without relu
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE) == gb.GC_ERR_WORKSPACE            # no workspace
    for dt in (gb.GC_F32, gb.GC_BF16):
        n = gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_WEIGHT_BIAS, L1, dt)
        assert n >= gb.gc_conv_workspace_bytes(gb.GC_OP_BWD_WEIGHT, L1, dt) > 0
        assert "bias column" in gb.gc_conv_plan_name(gb.GC_OP_BWD_WEIGHT_BIAS, L1, dt)
