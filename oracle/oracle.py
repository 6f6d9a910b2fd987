"""ctypes wrapper around the CPU oracle (conv_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.  Every function takes and returns fp64 numpy arrays; bf16 or
fp32 inputs are upcast exactly by the caller.

The operation is the one defined in "Speedups to gemm_conv_forward and
gemm_conv_backward kernels" (PufferLib pull request #522): forward conv with
an optional ReLU, and a backward pass yielding wgrad and d_input, at stride S
without padding.  See conv_oracle.c for the readings of what that page leaves
open.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src=_SRC, out=_LIB, quiet=True):
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-o", out + ".tmp", src]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # GC_ORACLE_LIB names another build of conv_oracle.c (the tests' run of
    # the pins under AddressSanitizer and UBSan)
    other = os.environ.get("GC_ORACLE_LIB")
    if other:
        _lib = _bind(ctypes.CDLL(os.path.abspath(other)))
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


class use_library:
    """Context manager: route the functions below through another build of
    conv_oracle.c (used by the tests that plant a mistake in a copy of it)."""

    def __init__(self, path):
        self.lib = _bind(ctypes.CDLL(os.path.abspath(path)))

    def __enter__(self):
        global _lib
        _load()
        self.saved, _lib = _lib, self.lib
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    i = ctypes.c_int
    lib.oracle_out_dim.argtypes = [i, i, i]
    lib.oracle_out_dim.restype = i
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i
    dims = [i] * 9  # B IC H W OC KH KW S relu
    lib.oracle_conv_fwd.argtypes = [dp, dp, dp] + dims
    lib.oracle_conv_bwd_data.argtypes = [dp, dp, dp, dp] + dims
    lib.oracle_conv_bwd_weight.argtypes = [dp, dp, dp, dp] + dims
    lib.oracle_conv_fwd_at.argtypes = [dp, dp, ip, i, dp] + dims
    lib.oracle_conv_bwd_data_at.argtypes = [dp, dp, dp, ip, i, dp] + dims
    lib.oracle_conv_bwd_weight_at.argtypes = [dp, dp, dp, ip, i, dp] + dims
    lib.oracle_conv_fwd_bias.argtypes = [dp, dp, dp, dp] + dims
    lib.oracle_conv_bwd_bias.argtypes = [dp, dp, dp, i, i, i, i, i]
    for f in ("oracle_conv_fwd", "oracle_conv_bwd_data", "oracle_conv_bwd_weight",
              "oracle_conv_fwd_at", "oracle_conv_bwd_data_at", "oracle_conv_bwd_weight_at",
              "oracle_conv_fwd_bias", "oracle_conv_bwd_bias"):
        getattr(lib, f).restype = None
    return lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def out_dim(n, k, s):
    """floor((n - k) / s) + 1, or -1 for an invalid extent."""
    return _load().oracle_out_dim(int(n), int(k), int(s))


def _dims(x_shape, w_shape, stride):
    B, IC, H, W = (int(v) for v in x_shape)
    OC, IC2, KH, KW = (int(v) for v in w_shape)
    if IC2 != IC:
        raise ValueError("channel mismatch between x and w")
    OH, OW = out_dim(H, KH, stride), out_dim(W, KW, stride)
    if OH < 1 or OW < 1:
        raise ValueError("invalid convolution extents")
    return B, IC, H, W, OC, KH, KW, OH, OW


def conv_fwd(x, w, stride, relu):
    """y = f(conv(x, w)), fp64; x NCHW, w OIHW."""
    x, w = _f64(x), _f64(w)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x.shape, w.shape, stride)
    y = np.empty((B, OC, OH, OW), np.float64)
    _load().oracle_conv_fwd(_ptr(x), _ptr(w), _ptr(y), B, IC, H, W, OC, KH, KW,
                            int(stride), int(bool(relu)))
    return y


def conv_fwd_bias(x, w, bias, stride, relu):
    """y = f(conv(x, w) + bias[oc]), fp64; bias has OC entries."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x.shape, w.shape, stride)
    if bias.shape != (OC,):
        raise ValueError("bias shape mismatch")
    y = np.empty((B, OC, OH, OW), np.float64)
    _load().oracle_conv_fwd_bias(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), B, IC, H, W, OC, KH, KW,
                                 int(stride), int(bool(relu)))
    return y


def conv_bwd_bias(dy, y_mask, relu):
    """db[oc] = sum over (b, oh, ow) of dy, masked by (y_mask > 0) when relu."""
    dy = _f64(dy)
    B, OC, OH, OW = (int(v) for v in dy.shape)
    m = _mask_arg(y_mask, relu, dy.shape)
    db = np.empty((OC,), np.float64)
    _load().oracle_conv_bwd_bias(_ptr(dy), _ptr(m), _ptr(db), B, OC, OH, OW, int(bool(relu)))
    return db


def _mask_arg(y_mask, relu, shape):
    if not relu:
        return None
    m = _f64(y_mask)
    if m.shape != shape:
        raise ValueError("y_mask shape mismatch")
    return m


def conv_bwd_data(dy, w, y_mask, x_shape, stride, relu):
    """dx for input shape x_shape; dy masked by (y_mask > 0) when relu."""
    dy, w = _f64(dy), _f64(w)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x_shape, w.shape, stride)
    if dy.shape != (B, OC, OH, OW):
        raise ValueError("dy shape mismatch")
    m = _mask_arg(y_mask, relu, dy.shape)
    dx = np.empty((B, IC, H, W), np.float64)
    _load().oracle_conv_bwd_data(_ptr(dy), _ptr(w), _ptr(m), _ptr(dx), B, IC, H, W,
                                 OC, KH, KW, int(stride), int(bool(relu)))
    return dx


def conv_bwd_weight(x, dy, y_mask, w_shape, stride, relu):
    """dw of shape w_shape; dy masked by (y_mask > 0) when relu."""
    x, dy = _f64(x), _f64(dy)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x.shape, w_shape, stride)
    if dy.shape != (B, OC, OH, OW):
        raise ValueError("dy shape mismatch")
    m = _mask_arg(y_mask, relu, dy.shape)
    dw = np.empty((OC, IC, KH, KW), np.float64)
    _load().oracle_conv_bwd_weight(_ptr(x), _ptr(dy), _ptr(m), _ptr(dw), B, IC, H, W,
                                   OC, KH, KW, int(stride), int(bool(relu)))
    return dw


def _coords(c):
    c = np.ascontiguousarray(c, dtype=np.int32).reshape(-1, 4)
    return c


def conv_fwd_at(x, w, coords, stride, relu):
    """y at the given (b, oc, oh, ow) coordinates."""
    x, w = _f64(x), _f64(w)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x.shape, w.shape, stride)
    c = _coords(coords)
    out = np.empty(len(c), np.float64)
    _load().oracle_conv_fwd_at(_ptr(x), _ptr(w), _iptr(c), len(c), _ptr(out),
                               B, IC, H, W, OC, KH, KW, int(stride), int(bool(relu)))
    return out


def conv_bwd_data_at(dy, w, y_mask, x_shape, coords, stride, relu):
    """dx at the given (b, ic, ih, iw) coordinates (gather form)."""
    dy, w = _f64(dy), _f64(w)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x_shape, w.shape, stride)
    m = _mask_arg(y_mask, relu, dy.shape)
    c = _coords(coords)
    out = np.empty(len(c), np.float64)
    _load().oracle_conv_bwd_data_at(_ptr(dy), _ptr(w), _ptr(m), _iptr(c), len(c),
                                    _ptr(out), B, IC, H, W, OC, KH, KW, int(stride),
                                    int(bool(relu)))
    return out


def conv_bwd_weight_at(x, dy, y_mask, w_shape, coords, stride, relu):
    """dw at the given (oc, ic, kh, kw) coordinates."""
    x, dy = _f64(x), _f64(dy)
    B, IC, H, W, OC, KH, KW, OH, OW = _dims(x.shape, w_shape, stride)
    m = _mask_arg(y_mask, relu, dy.shape)
    c = _coords(coords)
    out = np.empty(len(c), np.float64)
    _load().oracle_conv_bwd_weight_at(_ptr(x), _ptr(dy), _ptr(m), _iptr(c), len(c),
                                      _ptr(out), B, IC, H, W, OC, KH, KW, int(stride),
                                      int(bool(relu)))
    return out


def thread_count():
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())
