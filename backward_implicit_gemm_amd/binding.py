"""Python binding of libgc (include/gc.h): argument marshalling only.

Every function here turns torch tensors into device pointers, a descriptor
and the current HIP stream, and calls the C entry point of the same name;
all computation happens in the HIP kernels behind it.  There is no fallback:
if ``libgc.so`` is missing or a call fails, an exception is raised.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgc.so")

GC_OK, GC_ERR_INVALID_ARG, GC_ERR_UNSUPPORTED, GC_ERR_WORKSPACE, GC_ERR_HIP = range(5)
GC_F32, GC_BF16 = 0, 1
GC_OP_FWD, GC_OP_BWD_DATA, GC_OP_BWD_WEIGHT, GC_OP_BWD_BIAS, GC_OP_BWD = 0, 1, 2, 3, 4
GC_OP_BWD_WEIGHT_BIAS = 5

EXPORTED = (
    "gc_conv_out_dims", "gc_conv_workspace_bytes", "gc_conv_fwd", "gc_conv_bwd_data",
    "gc_conv_bwd_weight", "gc_status_string", "gc_fastdiv_selfcheck", "gc_version",
    "gc_set_kernel_policy", "gc_conv_fwd_bias", "gc_conv_bwd_bias", "gc_conv_bwd",
    "gc_conv_plan_name", "gc_conv_fwd_noalloc", "gc_conv_bwd_weight_bias",
)
GC_POLICY_AUTO, GC_POLICY_GENERIC = 0, 1


class GcError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}")


class gc_conv_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "IC", "H", "W", "OC", "KH", "KW", "stride")]


_lib = None


def lib():
    """The loaded libgc.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libgc.so not found at {LIB_PATH}; run __graft_entry__.build() "
                           "(python -m backward_implicit_gemm_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i, dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(gc_conv_desc)
    L.gc_conv_out_dims.argtypes = [dp, ctypes.POINTER(i), ctypes.POINTER(i)]
    L.gc_conv_out_dims.restype = i
    L.gc_conv_workspace_bytes.argtypes = [i, dp, i]
    L.gc_conv_workspace_bytes.restype = sz
    L.gc_conv_fwd.argtypes = [vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_fwd.restype = i
    L.gc_conv_fwd_noalloc.argtypes = [vp, vp, vp, dp, i, i, vp]
    L.gc_conv_fwd_noalloc.restype = i
    L.gc_conv_fwd_bias.argtypes = [vp, vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_fwd_bias.restype = i
    L.gc_conv_bwd_bias.argtypes = [vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_bwd_bias.restype = i
    L.gc_conv_bwd_data.argtypes = [vp, vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_bwd_data.restype = i
    L.gc_conv_bwd_weight.argtypes = [vp, vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_bwd_weight.restype = i
    L.gc_conv_bwd_weight_bias.argtypes = [vp, vp, vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_bwd_weight_bias.restype = i
    L.gc_conv_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, dp, i, i, vp]
    L.gc_conv_bwd.restype = i
    L.gc_status_string.argtypes = [i]
    L.gc_status_string.restype = ctypes.c_char_p
    L.gc_fastdiv_selfcheck.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    L.gc_fastdiv_selfcheck.restype = ctypes.c_int64
    L.gc_conv_plan_name.argtypes = [i, dp, i, ctypes.c_char_p, sz]
    L.gc_conv_plan_name.restype = i
    L.gc_version.argtypes = []
    L.gc_version.restype = i
    L.gc_set_kernel_policy.argtypes = [i]
    L.gc_set_kernel_policy.restype = i
    _lib = L
    return L


def gc_set_kernel_policy(policy):
    """Process-wide kernel selection (GC_POLICY_AUTO or GC_POLICY_GENERIC);
    returns the previous policy."""
    prev = lib().gc_set_kernel_policy(int(policy))
    if prev < 0:
        raise ValueError(f"unknown kernel policy {policy}")
    return prev


def status_string(status):
    return lib().gc_status_string(int(status)).decode()


def make_desc(B, IC, H, W, OC, KH, KW, stride):
    return gc_conv_desc(int(B), int(IC), int(H), int(W), int(OC), int(KH), int(KW), int(stride))


def desc_from(x_shape, w_shape, stride):
    B, IC, H, W = (int(v) for v in x_shape)
    OC, IC2, KH, KW = (int(v) for v in w_shape)
    if IC2 != IC:
        raise ValueError(f"x has {IC} channels but w expects {IC2}")
    return make_desc(B, IC, H, W, OC, KH, KW, stride)


def gc_conv_out_dims(desc):
    oh, ow = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().gc_conv_out_dims(ctypes.byref(desc), ctypes.byref(oh), ctypes.byref(ow))
    if st != GC_OK:
        raise GcError("gc_conv_out_dims", st)
    return oh.value, ow.value


def gc_conv_workspace_bytes(op, desc, dtype):
    return int(lib().gc_conv_workspace_bytes(int(op), ctypes.byref(desc), int(dtype)))


def gc_conv_plan_name(op, desc, dtype):
    """The kernels `op` would run for this problem (host only, enqueues nothing)."""
    buf = ctypes.create_string_buffer(256)
    st = lib().gc_conv_plan_name(int(op), ctypes.byref(desc), int(dtype), buf, len(buf))
    _check("gc_conv_plan_name", st)
    return buf.value.decode()


def _dtype_code(t):
    if t.dtype == torch.float32:
        return GC_F32
    if t.dtype == torch.bfloat16:
        return GC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _expect(t, name, shape):
    """Raises ValueError unless tensor t (if given) has exactly this shape;
    checked before anything touches the device, so a wrongly sized buffer
    never reaches the kernels."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _y_shape(desc):
    oh, ow = gc_conv_out_dims(desc)
    return (desc.B, desc.OC, oh, ow)


def _dev(t, name, dtype):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _dtype_code(t) != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, the call uses another")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ws(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _check(fn, st):
    if st != GC_OK:
        raise GcError(fn, st)


def workspace_for(op, desc, dtype, device="cuda"):
    """A device buffer of the size gc_conv_workspace_bytes asks for (or None)."""
    n = gc_conv_workspace_bytes(op, desc, dtype)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def gc_conv_fwd(x, w, y, relu, stride, workspace=None, stream=None):
    """y = relu?(conv(x, w)) via the C entry point gc_conv_fwd."""
    dt = _dtype_code(x)
    desc = desc_from(x.shape, w.shape, stride)
    _expect(y, "y", _y_shape(desc))
    wp, wn = _ws(workspace)
    st = lib().gc_conv_fwd(_dev(x, "x", dt), _dev(w, "w", dt), _dev(y, "y", dt), wp, wn,
                           ctypes.byref(desc), int(relu), dt, _stream(stream))
    _check("gc_conv_fwd", st)
    return y


def gc_conv_fwd_noalloc(x, w, y, relu, stride, stream=None):
    """y = relu?(conv(x, w)) via gc_conv_fwd_noalloc (no workspace: the
    library's static per-GPU scratch)."""
    dt = _dtype_code(x)
    desc = desc_from(x.shape, w.shape, stride)
    _expect(y, "y", _y_shape(desc))
    st = lib().gc_conv_fwd_noalloc(_dev(x, "x", dt), _dev(w, "w", dt), _dev(y, "y", dt),
                                   ctypes.byref(desc), int(relu), dt, _stream(stream))
    _check("gc_conv_fwd_noalloc", st)
    return y


def gc_conv_fwd_bias(x, w, bias, y, relu, stride, workspace=None, stream=None):
    """y = relu?(conv(x, w) + bias) via the C entry point gc_conv_fwd_bias."""
    dt = _dtype_code(x)
    desc = desc_from(x.shape, w.shape, stride)
    _expect(y, "y", _y_shape(desc))
    _expect(bias, "bias", (desc.OC,))
    wp, wn = _ws(workspace)
    st = lib().gc_conv_fwd_bias(_dev(x, "x", dt), _dev(w, "w", dt), _dev(bias, "bias", dt),
                                _dev(y, "y", dt), wp, wn, ctypes.byref(desc), int(relu), dt,
                                _stream(stream))
    _check("gc_conv_fwd_bias", st)
    return y


def gc_conv_bwd_bias(dy, y_mask, db, relu, x_shape, w_shape, stride, workspace, stream=None):
    """db[oc] = sum of dy (masked by y_mask > 0 when relu) via gc_conv_bwd_bias."""
    dt = _dtype_code(dy)
    desc = desc_from(x_shape, w_shape, stride)
    ys = _y_shape(desc)
    _expect(dy, "dy", ys)
    _expect(y_mask, "y_mask", ys)
    _expect(db, "db", (desc.OC,))
    wp, wn = _ws(workspace)
    st = lib().gc_conv_bwd_bias(_dev(dy, "dy", dt), _dev(y_mask, "y_mask", dt), _dev(db, "db", dt),
                                wp, wn, ctypes.byref(desc), int(relu), dt, _stream(stream))
    _check("gc_conv_bwd_bias", st)
    return db


def gc_conv_bwd_data(dy, w, y_mask, dx, relu, stride, workspace=None, stream=None):
    """dx from dy (masked by y_mask > 0 when relu) via gc_conv_bwd_data."""
    dt = _dtype_code(dy)
    desc = desc_from(dx.shape, w.shape, stride)
    ys = _y_shape(desc)
    _expect(dy, "dy", ys)
    _expect(y_mask, "y_mask", ys)
    wp, wn = _ws(workspace)
    st = lib().gc_conv_bwd_data(_dev(dy, "dy", dt), _dev(w, "w", dt), _dev(y_mask, "y_mask", dt),
                                _dev(dx, "dx", dt), wp, wn, ctypes.byref(desc), int(relu), dt,
                                _stream(stream))
    _check("gc_conv_bwd_data", st)
    return dx


def gc_conv_bwd_weight(x, dy, y_mask, dw, relu, stride, workspace, stream=None):
    """dw from x and dy (masked by y_mask > 0 when relu) via gc_conv_bwd_weight."""
    dt = _dtype_code(x)
    desc = desc_from(x.shape, dw.shape, stride)
    ys = _y_shape(desc)
    _expect(dy, "dy", ys)
    _expect(y_mask, "y_mask", ys)
    wp, wn = _ws(workspace)
    st = lib().gc_conv_bwd_weight(_dev(x, "x", dt), _dev(dy, "dy", dt), _dev(y_mask, "y_mask", dt),
                                  _dev(dw, "dw", dt), wp, wn, ctypes.byref(desc), int(relu), dt,
                                  _stream(stream))
    _check("gc_conv_bwd_weight", st)
    return dw


def gc_conv_bwd_weight_bias(x, dy, y_mask, dw, db, relu, stride, workspace, stream=None):
    """dw and db together (dy masked by y_mask > 0 when relu) via gc_conv_bwd_weight_bias."""
    dt = _dtype_code(x)
    desc = desc_from(x.shape, dw.shape, stride)
    ys = _y_shape(desc)
    _expect(dy, "dy", ys)
    _expect(y_mask, "y_mask", ys)
    _expect(db, "db", (desc.OC,))
    wp, wn = _ws(workspace)
    st = lib().gc_conv_bwd_weight_bias(_dev(x, "x", dt), _dev(dy, "dy", dt),
                                       _dev(y_mask, "y_mask", dt), _dev(dw, "dw", dt),
                                       _dev(db, "db", dt), wp, wn, ctypes.byref(desc), int(relu),
                                       dt, _stream(stream))
    _check("gc_conv_bwd_weight_bias", st)
    return dw, db


def gc_conv_bwd(x, w, dy, y_mask, dx, dw, relu, stride, workspace, stream=None):
    """dx and dw together (dy masked by y_mask > 0 when relu) via gc_conv_bwd."""
    dt = _dtype_code(x)
    desc = desc_from(x.shape, w.shape, stride)
    ys = _y_shape(desc)
    _expect(dy, "dy", ys)
    _expect(y_mask, "y_mask", ys)
    _expect(dx, "dx", x.shape)
    _expect(dw, "dw", w.shape)
    wp, wn = _ws(workspace)
    st = lib().gc_conv_bwd(_dev(x, "x", dt), _dev(w, "w", dt), _dev(dy, "dy", dt),
                           _dev(y_mask, "y_mask", dt), _dev(dx, "dx", dt), _dev(dw, "dw", dt),
                           wp, wn, ctypes.byref(desc), int(relu), dt, _stream(stream))
    _check("gc_conv_bwd", st)
    return dx, dw


class Conv:
    """One convolution layer's three passes with their workspaces allocated
    once (torch allocates; the library only receives pointers)."""

    def __init__(self, x_shape, w_shape, stride, relu, dtype, device="cuda"):
        self.stride, self.relu = int(stride), int(relu)
        self.dt = {torch.float32: GC_F32, torch.bfloat16: GC_BF16}[dtype]
        self.dtype = dtype
        self.desc = desc_from(x_shape, w_shape, stride)
        self.x_shape, self.w_shape = tuple(x_shape), tuple(w_shape)
        OH, OW = gc_conv_out_dims(self.desc)
        self.y_shape = (x_shape[0], w_shape[0], OH, OW)
        self.ws = {op: workspace_for(op, self.desc, self.dt, device)
                   for op in (GC_OP_FWD, GC_OP_BWD_DATA, GC_OP_BWD_WEIGHT, GC_OP_BWD_BIAS,
                              GC_OP_BWD, GC_OP_BWD_WEIGHT_BIAS)}

    def fwd(self, x, w, y, stream=None):
        return gc_conv_fwd(x, w, y, self.relu, self.stride, self.ws[GC_OP_FWD], stream)

    def bwd_data(self, dy, w, y, dx, stream=None):
        return gc_conv_bwd_data(dy, w, y if self.relu else None, dx, self.relu, self.stride,
                                self.ws[GC_OP_BWD_DATA], stream)

    def bwd_weight(self, x, dy, y, dw, stream=None):
        return gc_conv_bwd_weight(x, dy, y if self.relu else None, dw, self.relu, self.stride,
                                  self.ws[GC_OP_BWD_WEIGHT], stream)

    def bwd(self, x, w, dy, y, dx, dw, stream=None):
        return gc_conv_bwd(x, w, dy, y if self.relu else None, dx, dw, self.relu, self.stride,
                           self.ws[GC_OP_BWD], stream)

    def fwd_bias(self, x, w, bias, y, stream=None):
        return gc_conv_fwd_bias(x, w, bias, y, self.relu, self.stride, self.ws[GC_OP_FWD], stream)

    def bwd_weight_bias(self, x, dy, y, dw, db, stream=None):
        return gc_conv_bwd_weight_bias(x, dy, y if self.relu else None, dw, db, self.relu,
                                       self.stride, self.ws[GC_OP_BWD_WEIGHT_BIAS], stream)

    def bwd_bias(self, dy, y, db, stream=None):
        return gc_conv_bwd_bias(dy, y if self.relu else None, db, self.relu, self.x_shape,
                                self.w_shape, self.stride, self.ws[GC_OP_BWD_BIAS], stream)
