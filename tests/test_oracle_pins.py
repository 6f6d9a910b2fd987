"""Pins for the CPU oracle against facts that do not come from the oracle.

Each pin is chosen so that a plausible slip in the oracle -- a dropped term, a
wrong sign, a wrong or transposed index, a missing ReLU mask, an output size
that rounds instead of floors -- fails at least one of them
(``test_planted_mistakes_are_caught`` plants such slips in copies of the
oracle's source and checks exactly that).

Sources of truth used here:
  * the layer shapes, output sizes and element counts printed in "Speedups to
    gemm_conv_forward and gemm_conv_backward kernels" (PufferLib pull request
    #522), stored with citations in tests/golden/page1_shapes.json;
  * tiny examples worked by hand from the convolution's definition;
  * closed forms for constant inputs, with tap counts listed by hand;
  * the adjoint identity <conv(x), dz> = <x, dgrad(dz)> = <w, wgrad(x, dz)>;
  * central finite differences of L = <relu(conv(x, w)), dy>;
  * the special cases that reduce to a dense matrix product (numpy);
  * PyTorch's CPU conv2d and its autograd in fp64 (a library routine);
  * an im2col + matmul formulation written here, test-only;
  * exactness on small-integer inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Output size and element counts printed on the page
# --------------------------------------------------------------------------

def test_output_dims_match_page_layers():
    g = json.load(open(os.path.join(GOLDEN, "page1_shapes.json")))
    for L in g["layers"]:
        assert orc.out_dim(L["H"], L["K"], L["S"]) == L["OH"], L["cite"]
        assert orc.out_dim(L["W"], L["K"], L["S"]) == L["OW"], L["cite"]


def test_element_counts_match_page():
    g = json.load(open(os.path.join(GOLDEN, "page1_shapes.json")))
    layers = g["layers"]
    for c in g["element_counts"]:
        L = layers[c["layer"]]
        OH = orc.out_dim(L["H"], L["K"], L["S"])
        OW = orc.out_dim(L["W"], L["K"], L["S"])
        if c["what"] == "B*IC*H*W":
            n = c["B"] * L["IC"] * L["H"] * L["W"]
        else:
            n = c["B"] * L["OC"] * OH * OW
        assert n == c["value"], c["cite"]


def test_output_dim_rejects_invalid():
    assert orc.out_dim(4, 5, 1) == -1
    assert orc.out_dim(5, 5, 0) == -1
    assert orc.out_dim(0, 1, 1) == -1
    assert orc.out_dim(5, 5, 7) == 1
    assert orc.out_dim(7, 2, 2) == 3  # (7-2)/2 = 2.5 floors to 2, plus one


# --------------------------------------------------------------------------
# Tiny examples worked by hand
# --------------------------------------------------------------------------

X33 = np.arange(1, 10, dtype=np.float64).reshape(1, 1, 3, 3)   # [[1,2,3],[4,5,6],[7,8,9]]
W22 = np.array([[1, 2], [3, 4]], np.float64).reshape(1, 1, 2, 2)


def test_hand_forward_stride1():
    # y[oh,ow] = x[oh,ow]*1 + x[oh,ow+1]*2 + x[oh+1,ow]*3 + x[oh+1,ow+1]*4
    #   (0,0): 1 + 4 + 12 + 20 = 37   (0,1): 2 + 6 + 15 + 24 = 47
    #   (1,0): 4 + 10 + 21 + 32 = 67  (1,1): 5 + 12 + 24 + 36 = 77
    y = orc.conv_fwd(X33, W22, 1, 0)
    np.testing.assert_array_equal(y[0, 0], [[37, 47], [67, 77]])


def test_hand_forward_stride2_floors():
    # (3-2)/2 + 1 = 1: a single window at the top-left corner.
    y = orc.conv_fwd(X33, W22, 2, 0)
    assert y.shape == (1, 1, 1, 1) and y[0, 0, 0, 0] == 37


def test_hand_forward_relu_and_channels():
    # Two input channels, two output channels, 2x2 input, 2x2 kernel -> 1x1.
    x = np.array([[[[1, 2], [3, 4]], [[5, 6], [7, 8]]]], np.float64)
    w = np.zeros((2, 2, 2, 2))
    w[0, 0, 0, 0] = 1.0    # picks x[ic=0, 0, 0] = 1
    w[0, 1, 1, 1] = 1.0    # picks x[ic=1, 1, 1] = 8     -> oc0 = 9
    w[1, 0, 0, 1] = 1.0    # picks x[ic=0, 0, 1] = 2
    w[1, 1, 1, 0] = -1.0   # picks -x[ic=1, 1, 0] = -7   -> oc1 = -5
    y = orc.conv_fwd(x, w, 1, 0)
    np.testing.assert_array_equal(y.ravel(), [9, -5])
    y = orc.conv_fwd(x, w, 1, 1)
    np.testing.assert_array_equal(y.ravel(), [9, 0])


def test_hand_dgrad_stride1():
    # A unit gradient at one output places the kernel at that window.
    dy = np.zeros((1, 1, 2, 2)); dy[0, 0, 0, 0] = 1
    dx = orc.conv_bwd_data(dy, W22, None, (1, 1, 3, 3), 1, 0)
    np.testing.assert_array_equal(dx[0, 0], [[1, 2, 0], [3, 4, 0], [0, 0, 0]])
    dy = np.zeros((1, 1, 2, 2)); dy[0, 0, 1, 1] = 1
    dx = orc.conv_bwd_data(dy, W22, None, (1, 1, 3, 3), 1, 0)
    np.testing.assert_array_equal(dx[0, 0], [[0, 0, 0], [0, 1, 2], [0, 3, 4]])


def test_hand_dgrad_stride3_uncovered_pixels():
    # 4x5 input, 2x2 kernel, stride 3 -> 1x2 output; windows at columns 0-1
    # and 3-4, rows 0-1.  dy = [1, 2]: window 0 gets w, window 1 gets 2w.
    # Column 2 and rows 2-3 are covered by no window and stay 0.
    dy = np.array([[[[1, 2]]]], np.float64)
    dx = orc.conv_bwd_data(dy, W22, None, (1, 1, 4, 5), 3, 0)
    np.testing.assert_array_equal(dx[0, 0], [[1, 2, 0, 2, 4],
                                             [3, 4, 0, 6, 8],
                                             [0, 0, 0, 0, 0],
                                             [0, 0, 0, 0, 0]])


def test_hand_wgrad_stride1():
    # dy = 1 everywhere: dw[kh,kw] = sum of the 2x2 block of x starting at (kh,kw)
    #   (0,0): 1+2+4+5 = 12  (0,1): 2+3+5+6 = 16
    #   (1,0): 4+5+7+8 = 24  (1,1): 5+6+8+9 = 28
    dy = np.ones((1, 1, 2, 2))
    dw = orc.conv_bwd_weight(X33, dy, None, (1, 1, 2, 2), 1, 0)
    np.testing.assert_array_equal(dw[0, 0], [[12, 16], [24, 28]])


def test_hand_relu_mask_is_strict():
    # y_mask = [+1, 0, -1, +2]: only the strictly positive entries pass dy.
    x = np.arange(1, 6, dtype=np.float64).reshape(1, 1, 1, 5)
    w = np.ones((1, 1, 1, 2))
    dy = np.array([[[[10, 20, 30, 40]]]], np.float64)
    ym = np.array([[[[1, 0, -1, 2]]]], np.float64)
    dx = orc.conv_bwd_data(dy, w, ym, x.shape, 1, 1)
    # windows (0,1),(1,2),(2,3),(3,4); live gradients 10 at window 0, 40 at window 3
    np.testing.assert_array_equal(dx.ravel(), [10, 10, 0, 40, 40])
    dw = orc.conv_bwd_weight(x, dy, ym, w.shape, 1, 1)
    # dw[0] = 10*x0 + 40*x3 = 10 + 160 ; dw[1] = 10*x1 + 40*x4 = 20 + 200
    np.testing.assert_array_equal(dw.ravel(), [170, 220])


# --------------------------------------------------------------------------
# Closed forms with constant inputs at the page's layer shapes
# --------------------------------------------------------------------------

# Number of output windows covering each input row / column, listed by hand.
# Layer 1 rows (11, K=5, S=3 -> windows at rows 0-4, 3-7, 6-10):
L1_ROWS = [1, 1, 1, 2, 2, 1, 2, 2, 1, 1, 1]
# Layer 1 columns (15, K=5, S=3 -> windows at 0-4, 3-7, 6-10, 9-13; 14 uncovered):
L1_COLS = [1, 1, 1, 2, 2, 1, 2, 2, 1, 2, 2, 1, 1, 1, 0]
# Layer 2 rows (3, K=3, S=1 -> one window) and columns (4, K=3 -> windows 0-2, 1-3):
L2_ROWS = [1, 1, 1]
L2_COLS = [1, 2, 2, 1]


@pytest.mark.parametrize("layer", [0, 1])
def test_constant_closed_forms(layer):
    g = json.load(open(os.path.join(GOLDEN, "page1_shapes.json")))["layers"][layer]
    B, IC, OC, H, W, K, S = 2, g["IC"], g["OC"], g["H"], g["W"], g["K"], g["S"]
    OH, OW = g["OH"], g["OW"]
    rows, cols = (L1_ROWS, L1_COLS) if layer == 0 else (L2_ROWS, L2_COLS)
    assert sum(rows) == OH * K and sum(cols) == OW * K
    ones_x = np.ones((B, IC, H, W))
    ones_w = np.ones((OC, IC, K, K))
    ones_dy = np.ones((B, OC, OH, OW))
    y = orc.conv_fwd(ones_x, ones_w, S, g["relu"])
    assert y.shape == (B, OC, OH, OW)
    assert np.all(y == IC * K * K)
    mask = y  # all positive, so the ReLU mask passes every gradient
    dx = orc.conv_bwd_data(ones_dy, ones_w, mask, (B, IC, H, W), S, g["relu"])
    expect = OC * np.outer(rows, cols)
    assert np.all(dx == expect[None, None])
    dw = orc.conv_bwd_weight(ones_x, ones_dy, mask, (OC, IC, K, K), S, g["relu"])
    assert np.all(dw == B * OH * OW)


def test_layer1_uncovered_column_is_exactly_zero():
    r = rng(5)
    B, IC, H, W, OC, K, S = 3, 4, 11, 15, 5, 5, 3
    dy = r.standard_normal((B, OC, 3, 4))
    w = r.standard_normal((OC, IC, K, K))
    dx = orc.conv_bwd_data(dy, w, None, (B, IC, H, W), S, 0)
    assert np.all(dx[..., 14] == 0.0)
    assert np.all(dx[..., :14].any(axis=-1))


# --------------------------------------------------------------------------
# Adjoint identity, finite differences
# --------------------------------------------------------------------------

SHAPES = [
    # B, IC, H, W, OC, KH, KW, S
    (2, 3, 7, 8, 4, 3, 3, 2),
    (2, 3, 11, 15, 4, 5, 5, 3),
    (3, 5, 3, 4, 6, 3, 3, 1),
    (1, 2, 9, 6, 3, 2, 4, 1),
    (2, 1, 10, 10, 2, 3, 2, 4),
    (2, 4, 5, 5, 3, 5, 5, 1),      # 1x1 output
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("relu", [0, 1])
def test_adjoint_identity(shape, relu):
    B, IC, H, W, OC, KH, KW, S = shape
    r = rng(hash(shape) % 1000 + relu)
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, KH, KW))
    OH, OW = orc.out_dim(H, KH, S), orc.out_dim(W, KW, S)
    dy = r.standard_normal((B, OC, OH, OW))
    ym = r.standard_normal((B, OC, OH, OW))          # arbitrary fixed mask source
    dz = dy * (ym > 0) if relu else dy
    lin = orc.conv_fwd(x, w, S, 0)                   # pre-activation (linear map)
    lhs = float(np.sum(lin * dz))
    dx = orc.conv_bwd_data(dy, w, ym, x.shape, S, relu)
    dw = orc.conv_bwd_weight(x, dy, ym, w.shape, S, relu)
    scale = float(np.sum(np.abs(lin) * np.abs(dz))) + 1e-300
    assert abs(lhs - float(np.sum(x * dx))) <= 1e-12 * scale
    assert abs(lhs - float(np.sum(w * dw))) <= 1e-12 * scale


def _loss(x, w, dy, S):
    return float(np.sum(orc.conv_fwd(x, w, S, 1) * dy))


@pytest.mark.parametrize("shape", [(2, 3, 7, 8, 4, 3, 3, 2), (2, 3, 11, 15, 4, 5, 5, 3),
                                   (2, 2, 4, 5, 3, 3, 2, 1)])
def test_finite_differences_with_relu(shape):
    B, IC, H, W, OC, KH, KW, S = shape
    h = 1e-5
    for seed in range(100):
        r = rng(1000 + seed)
        x = r.standard_normal((B, IC, H, W))
        w = r.standard_normal((OC, IC, KH, KW)) * 0.5
        pre = orc.conv_fwd(x, w, S, 0)
        # keep every pre-activation away from the kink, so +-h never crosses it
        bound = h * (np.abs(w).sum() + np.abs(x).sum()) * 4
        if np.min(np.abs(pre)) > bound:
            break
    else:
        pytest.fail("no seed kept pre-activations off the ReLU kink")
    OH, OW = pre.shape[2:]
    dy = r.standard_normal((B, OC, OH, OW))
    y = orc.conv_fwd(x, w, S, 1)
    dx = orc.conv_bwd_data(dy, w, y, x.shape, S, 1)
    dw = orc.conv_bwd_weight(x, dy, y, w.shape, S, 1)
    for flat in r.choice(x.size, 12, replace=False):
        i = np.unravel_index(flat, x.shape)
        xp, xm = x.copy(), x.copy()
        xp[i] += h; xm[i] -= h
        fd = (_loss(xp, w, dy, S) - _loss(xm, w, dy, S)) / (2 * h)
        assert abs(fd - dx[i]) <= 1e-6 * (1 + abs(dx[i])), (i, fd, dx[i])
    for flat in r.choice(w.size, 12, replace=False):
        i = np.unravel_index(flat, w.shape)
        wp, wm = w.copy(), w.copy()
        wp[i] += h; wm[i] -= h
        fd = (_loss(x, wp, dy, S) - _loss(x, wm, dy, S)) / (2 * h)
        assert abs(fd - dw[i]) <= 1e-6 * (1 + abs(dw[i])), (i, fd, dw[i])


# --------------------------------------------------------------------------
# Special cases that are a dense matrix product
# --------------------------------------------------------------------------

def test_full_window_is_a_matmul():
    # H == KH and W == KW: one output per image, y = X_flat @ W_flat^T.
    r = rng(7)
    B, IC, H, W, OC = 5, 3, 4, 3, 6
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, H, W))
    dy = r.standard_normal((B, OC, 1, 1))
    X, Wf, DY = x.reshape(B, -1), w.reshape(OC, -1), dy.reshape(B, OC)
    np.testing.assert_allclose(orc.conv_fwd(x, w, 1, 0).reshape(B, OC), X @ Wf.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(orc.conv_bwd_data(dy, w, None, x.shape, 1, 0).reshape(B, -1),
                               DY @ Wf, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(orc.conv_bwd_weight(x, dy, None, w.shape, 1, 0).reshape(OC, -1),
                               DY.T @ X, rtol=1e-13, atol=1e-13)


def test_pointwise_kernel_is_per_pixel_matmul():
    # 1x1 kernel at stride 1: y[b,:,h,w] = W[:,:,0,0] @ x[b,:,h,w].
    r = rng(8)
    B, IC, H, W, OC = 2, 5, 3, 4, 7
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, 1, 1))
    y = orc.conv_fwd(x, w, 1, 0)
    np.testing.assert_allclose(y, np.einsum("oi,bihw->bohw", w[:, :, 0, 0], x), rtol=1e-13, atol=1e-13)
    # stride 2 keeps every other pixel
    y2 = orc.conv_fwd(x, w, 2, 0)
    np.testing.assert_allclose(y2, y[:, :, ::2, ::2], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Library routine: PyTorch CPU conv2d and autograd in fp64
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", SHAPES + [(3, 59, 11, 15, 8, 5, 5, 3), (4, 16, 3, 4, 8, 3, 3, 1)])
@pytest.mark.parametrize("relu", [0, 1])
def test_matches_torch_conv2d_fp64(shape, relu):
    B, IC, H, W, OC, KH, KW, S = shape
    r = rng(sum(shape) + relu)
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, KH, KW))
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    yt = torch.nn.functional.conv2d(xt, wt, stride=S)
    if relu:
        yt = torch.relu(yt)
    dy = r.standard_normal(tuple(yt.shape))
    yt.backward(torch.tensor(dy))
    y = orc.conv_fwd(x, w, S, relu)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    dx = orc.conv_bwd_data(dy, w, y, x.shape, S, relu)
    dw = orc.conv_bwd_weight(x, dy, y, w.shape, S, relu)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------
# Bias: forward with a per-channel bias and the bias gradient
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 7, 8, 4, 3, 3, 2), (3, 59, 11, 15, 8, 5, 5, 3),
                                   (4, 16, 3, 4, 8, 3, 3, 1)])
@pytest.mark.parametrize("relu", [0, 1])
def test_bias_matches_torch_fp64(shape, relu):
    """torch conv2d with a bias, and autograd's bias gradient, in fp64 on the CPU."""
    B, IC, H, W, OC, KH, KW, S = shape
    r = rng(7 * sum(shape) + relu)
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, KH, KW))
    b = r.standard_normal(OC)
    bt = torch.tensor(b, requires_grad=True)
    yt = torch.nn.functional.conv2d(torch.tensor(x), torch.tensor(w), bt, stride=S)
    if relu:
        yt = torch.relu(yt)
    dy = r.standard_normal(tuple(yt.shape))
    yt.backward(torch.tensor(dy))
    y = orc.conv_fwd_bias(x, w, b, S, relu)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.conv_bwd_bias(dy, y, relu), bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_bias_closed_forms():
    """dy = 1: db = B*OH*OW without a mask, and the count of positive outputs
    of each channel with one; a zero bias leaves the forward unchanged and a
    constant bias with w = 0 is copied to every output."""
    B, OC, OH, OW = 3, 5, 4, 6
    dy = np.ones((B, OC, OH, OW))
    np.testing.assert_array_equal(orc.conv_bwd_bias(dy, None, 0), np.full(OC, B * OH * OW))
    ym = np.zeros((B, OC, OH, OW))
    for oc in range(OC):
        ym.reshape(B, OC, -1)[:, oc, :oc + 1] = 1.0      # oc+1 positives per image
        ym.reshape(B, OC, -1)[:, oc, oc + 1:oc + 3] = -2.0
    np.testing.assert_array_equal(orc.conv_bwd_bias(dy, ym, 1), B * (np.arange(OC) + 1.0))
    x = rng(3).standard_normal((2, 3, 7, 8))
    w = rng(4).standard_normal((4, 3, 3, 3))
    np.testing.assert_array_equal(orc.conv_fwd_bias(x, w, np.zeros(4), 2, 0), orc.conv_fwd(x, w, 2, 0))
    y = orc.conv_fwd_bias(x, np.zeros_like(w), np.arange(4.0) - 1.5, 2, 1)
    np.testing.assert_array_equal(y, np.broadcast_to(np.maximum(np.arange(4.0) - 1.5, 0)[None, :, None, None], y.shape))


def test_bias_finite_differences():
    """dL/dbias for L = <relu(conv(x, w) + bias), dy>, central differences in fp64
    on inputs whose pre-activations stay away from the kink."""
    r = rng(11)
    x = r.standard_normal((2, 3, 11, 15))
    w = r.standard_normal((4, 3, 5, 5))
    b = r.standard_normal(4)
    pre = orc.conv_fwd_bias(x, w, b, 3, 0)
    b = b + np.where(np.abs(pre).min(axis=(0, 2, 3)) < 1e-2, 0.05, 0.0)   # keep off the kink
    y = orc.conv_fwd_bias(x, w, b, 3, 1)
    dy = r.standard_normal(y.shape)
    h = 1e-6
    num = np.empty(4)
    for oc in range(4):
        bp, bm = b.copy(), b.copy()
        bp[oc] += h; bm[oc] -= h
        num[oc] = (np.sum(orc.conv_fwd_bias(x, w, bp, 3, 1) * dy) -
                   np.sum(orc.conv_fwd_bias(x, w, bm, 3, 1) * dy)) / (2 * h)
    np.testing.assert_allclose(orc.conv_bwd_bias(dy, y, 1), num, rtol=1e-6, atol=1e-6)


# --------------------------------------------------------------------------
# A second formulation written here: im2col + matrix products
# --------------------------------------------------------------------------

def _im2col(x, KH, KW, S):
    B, IC, H, W = x.shape
    OH, OW = (H - KH) // S + 1, (W - KW) // S + 1
    cols = np.empty((B, OH, OW, IC, KH, KW))
    for oh in range(OH):
        for ow in range(OW):
            cols[:, oh, ow] = x[:, :, oh * S:oh * S + KH, ow * S:ow * S + KW]
    return cols.reshape(B * OH * OW, IC * KH * KW), OH, OW


def _col2im(cols, x_shape, KH, KW, S, OH, OW):
    B, IC, H, W = x_shape
    c = cols.reshape(B, OH, OW, IC, KH, KW)
    x = np.zeros(x_shape)
    for oh in range(OH):
        for ow in range(OW):
            x[:, :, oh * S:oh * S + KH, ow * S:ow * S + KW] += c[:, oh, ow]
    return x


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_im2col_formulation(shape):
    B, IC, H, W, OC, KH, KW, S = shape
    r = rng(31 + sum(shape))
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, KH, KW))
    cols, OH, OW = _im2col(x, KH, KW, S)
    Wf = w.reshape(OC, -1)
    pre = (cols @ Wf.T).reshape(B, OH, OW, OC).transpose(0, 3, 1, 2)
    y = np.maximum(pre, 0)
    dy = r.standard_normal(y.shape)
    dz = dy * (y > 0)
    DZ = dz.transpose(0, 2, 3, 1).reshape(-1, OC)
    np.testing.assert_allclose(orc.conv_fwd(x, w, S, 1), y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.conv_bwd_data(dy, w, y, x.shape, S, 1),
                               _col2im(DZ @ Wf, x.shape, KH, KW, S, OH, OW), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(orc.conv_bwd_weight(x, dy, y, w.shape, S, 1),
                               (DZ.T @ cols).reshape(w.shape), rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------
# Single-element forms agree with the full passes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", SHAPES)
def test_pointwise_forms_match_full_passes(shape):
    B, IC, H, W, OC, KH, KW, S = shape
    r = rng(77 + sum(shape))
    x = r.standard_normal((B, IC, H, W))
    w = r.standard_normal((OC, IC, KH, KW))
    y = orc.conv_fwd(x, w, S, 1)
    dy = r.standard_normal(y.shape)
    dx = orc.conv_bwd_data(dy, w, y, x.shape, S, 1)
    dw = orc.conv_bwd_weight(x, dy, y, w.shape, S, 1)
    cy = np.argwhere(np.ones(y.shape, bool))
    cx = np.argwhere(np.ones(x.shape, bool))
    cw = np.argwhere(np.ones(w.shape, bool))
    np.testing.assert_allclose(orc.conv_fwd_at(x, w, cy, S, 1), y.ravel(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(orc.conv_bwd_data_at(dy, w, y, x.shape, cx, S, 1), dx.ravel(),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.conv_bwd_weight_at(x, dy, y, w.shape, cw, S, 1), dw.ravel(),
                               rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Exactness on small integers, threads, homogeneity
# --------------------------------------------------------------------------

def test_integer_inputs_give_exact_integers():
    r = rng(3)
    B, IC, H, W, OC, K, S = 4, 59, 11, 15, 16, 5, 3
    x = r.integers(-2, 3, (B, IC, H, W)).astype(np.float64)
    w = r.integers(-2, 3, (OC, IC, K, K)).astype(np.float64)
    y = orc.conv_fwd(x, w, S, 1)
    dy = r.integers(-2, 3, y.shape).astype(np.float64)
    dx = orc.conv_bwd_data(dy, w, y, x.shape, S, 1)
    dw = orc.conv_bwd_weight(x, dy, y, w.shape, S, 1)
    for a in (y, dx, dw):
        assert np.all(a == np.round(a))
    yt = torch.relu(torch.nn.functional.conv2d(torch.tensor(x), torch.tensor(w), stride=S))
    assert np.array_equal(y, yt.numpy())


def test_positive_homogeneity_with_relu():
    r = rng(4)
    x = r.standard_normal((2, 3, 11, 15))
    w = r.standard_normal((4, 3, 5, 5))
    np.testing.assert_allclose(orc.conv_fwd(2.5 * x, w, 3, 1), 2.5 * orc.conv_fwd(x, w, 3, 1),
                               rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Planted mistakes in copies of the oracle's source are caught by the pins
# --------------------------------------------------------------------------

SRC = os.path.join(os.path.dirname(orc.__file__), "conv_oracle.c")

# (description, text in conv_oracle.c, replacement)
PLANTS = [
    ("fwd: kernel index transposed (kh <-> kw)",
     "* w[idx4(oc, IC, ic, KH, kh, KW, kw)];\n                    if (relu",
     "* w[idx4(oc, IC, ic, KH, kw, KW, kh)];\n                    if (relu"),
    ("fwd: ReLU keeps negatives", "if (relu && !(acc > 0.0)) acc = 0.0;\n                    y[",
     "if (relu && (acc > 0.0)) acc = acc;\n                    y["),
    ("fwd: stride ignored along w", "ow * S + kw)]", "ow + kw)]"),
    ("dgrad: sign flipped", "g * w[idx4(oc, IC, ic, KH, kh, KW, kw)];", "-g * w[idx4(oc, IC, ic, KH, kh, KW, kw)];"),
    ("dgrad: channel indices swapped", "g * w[idx4(oc, IC, ic, KH, kh, KW, kw)];",
     "g * w[idx4(ic % OC, IC, oc % IC, KH, kh, KW, kw)];"),
    ("mask: not strict", "if (relu && !(y_mask[i] > 0.0)) return 0.0;", "if (relu && !(y_mask[i] >= 0.0)) return 0.0;"),
    ("mask: ignored", "if (relu && !(y_mask[i] > 0.0)) return 0.0;", "(void)y_mask;"),
    ("wgrad: last output column dropped", "for (int ow = 0; ow < OW; ++ow)\n                            acc += masked_dy",
     "for (int ow = 0; ow < OW - 1; ++ow)\n                            acc += masked_dy"),
    ("out size rounds up", "return (in - k) / s + 1;", "return (in - k + s - 1) / s + 1;"),
    ("fwd_bias: bias dropped", "double acc = bias[oc];", "double acc = 0.0;"),
    ("fwd_bias: bias of the wrong channel", "double acc = bias[oc];", "double acc = bias[(oc + 1) % OC];"),
    ("bwd_bias: last output row dropped",
     "for (int oh = 0; oh < OH; ++oh)\n                for (int ow = 0; ow < OW; ++ow)\n                    acc += masked_dy",
     "for (int oh = 0; oh < OH - 1; ++oh)\n                for (int ow = 0; ow < OW; ++ow)\n                    acc += masked_dy"),
]


def _pins_pass():
    """Run a compact set of the pins above; False if any of them fails."""
    checks = [
        test_output_dims_match_page_layers,
        test_hand_forward_stride1, test_hand_forward_relu_and_channels,
        test_hand_dgrad_stride1, test_hand_dgrad_stride3_uncovered_pixels,
        test_hand_wgrad_stride1, test_hand_relu_mask_is_strict,
        lambda: test_constant_closed_forms(0),
        lambda: test_adjoint_identity((2, 3, 7, 8, 4, 3, 3, 2), 1),
        lambda: test_matches_torch_conv2d_fp64((2, 3, 11, 15, 4, 5, 5, 3), 1),
        lambda: test_matches_torch_conv2d_fp64((2, 3, 7, 8, 4, 3, 2, 2), 1),
        test_bias_closed_forms,
        lambda: test_bias_matches_torch_fp64((2, 3, 7, 8, 4, 3, 3, 2), 1),
    ]
    for c in checks:
        try:
            c()
        except Exception:
            return False
    return True


@pytest.mark.parametrize("plant", PLANTS, ids=[p[0] for p in PLANTS])
def test_planted_mistakes_are_caught(plant, tmp_path):
    desc, old, new = plant
    src = open(SRC).read()
    assert old in src, desc
    bad = tmp_path / "bad_oracle.c"
    bad.write_text(src.replace(old, new, 1))
    so = str(tmp_path / "libbad.so")
    orc.build(str(bad), so)
    with orc.use_library(so):
        assert not _pins_pass(), "pins missed: " + desc


def test_unmodified_oracle_passes_compact_pins():
    assert _pins_pass()
