"""Pins of the float64 convolution oracle (CPU): torch's float64 conv2d with
autograd (a library routine), central finite differences of L = sum(y * dy),
the bilinear adjoint identities, 1x1 convolution as a matrix product, a
one-hot filter as a shifted copy, and planted mistakes that the pins catch."""
import numpy as np
import pytest

import oracle
from oracle import conv as oc

CASES = [  # N, H, W, C, K, R, S, stride, pad
    (2, 7, 6, 3, 4, 3, 3, (1, 1), (1, 1)),
    (1, 9, 8, 2, 3, 3, 3, (2, 2), (1, 1)),
    (2, 11, 11, 3, 5, 7, 7, (2, 2), (3, 3)),   # the ResNet stem shape, scaled down
    (1, 6, 5, 4, 2, 1, 1, (2, 1), (0, 0)),
    (1, 5, 7, 2, 3, 2, 3, (1, 2), (0, 1)),     # even / rectangular filter
]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(c, seed=0):
    N, H, W, C, K, R, S, st, pd = c
    P, Q = oracle.out_size(H, W, R, S, st, pd)
    return (_rand((N, H, W, C), seed), _rand((K, R, S, C), seed + 1),
            _rand((N, P, Q, K), seed + 2), st, pd)


@pytest.mark.parametrize("c", CASES)
def test_against_torch_conv2d_float64(c):
    torch = pytest.importorskip("torch")
    x, w, dy, st, pd = _case(c)
    xt = torch.tensor(x.transpose(0, 3, 1, 2), dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w.transpose(0, 3, 1, 2), dtype=torch.float64, requires_grad=True)
    yt = torch.nn.functional.conv2d(xt, wt, stride=st, padding=pd)
    yt.backward(torch.tensor(dy.transpose(0, 3, 1, 2), dtype=torch.float64))
    y = oracle.conv2d_forward(x, w, st, pd)
    dx = oracle.conv2d_backward_data(dy, w, x.shape, st, pd)
    dw = oracle.conv2d_backward_filter(x, dy, w.shape, st, pd)
    np.testing.assert_allclose(y, yt.detach().numpy().transpose(0, 2, 3, 1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dx, xt.grad.numpy().transpose(0, 2, 3, 1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy().transpose(0, 2, 3, 1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("c", CASES[:4])
def test_finite_differences(c):
    x, w, dy, st, pd = _case(c, seed=3)
    dx = oracle.conv2d_backward_data(dy, w, x.shape, st, pd)
    dw = oracle.conv2d_backward_filter(x, dy, w.shape, st, pd)
    rng = np.random.default_rng(9)
    for arr, grad, is_x in ((x, dx, True), (w, dw, False)):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(24, flat.size), replace=False):
            h = 1e-6 * max(1.0, abs(flat[i]))
            orig = flat[i]
            flat[i] = orig + h
            lp = oracle.conv2d_loss(x, w, dy, st, pd)
            flat[i] = orig - h
            lm = oracle.conv2d_loss(x, w, dy, st, pd)
            flat[i] = orig
            assert abs((lp - lm) / (2 * h) - grad.reshape(-1)[i]) <= 1e-7 * max(1.0, abs(grad.reshape(-1)[i])), \
                ("dx" if is_x else "dw", i)


@pytest.mark.parametrize("c", CASES)
def test_adjoint_identities(c):
    # L = <conv(x, w), dy> is bilinear: <dx, x> = <dw, w> = L for the same dy
    x, w, dy, st, pd = _case(c, seed=5)
    L = oracle.conv2d_loss(x, w, dy, st, pd)
    dx = oracle.conv2d_backward_data(dy, w, x.shape, st, pd)
    dw = oracle.conv2d_backward_filter(x, dy, w.shape, st, pd)
    assert abs(np.sum(dx * x) - L) <= 1e-10 * max(1.0, abs(L))
    assert abs(np.sum(dw * w) - L) <= 1e-10 * max(1.0, abs(L))


def test_one_by_one_is_a_matrix_product():
    x, w = _rand((2, 4, 5, 6), 11), _rand((7, 1, 1, 6), 12)
    y = oracle.conv2d_forward(x, w)
    np.testing.assert_allclose(y, x @ w[:, 0, 0, :].T, rtol=0, atol=1e-13)
    # stride 2 samples every other pixel
    y2 = oracle.conv2d_forward(x, w, (2, 2))
    np.testing.assert_allclose(y2, x[:, ::2, ::2, :] @ w[:, 0, 0, :].T, rtol=0, atol=1e-13)


def test_one_hot_filter_is_a_shift():
    # a 3x3 filter whose only 1 is at tap (r, s) = (0, 2) on channel 0 copies
    # x shifted by (r - 1, s - 1) with zero padding 1
    x = _rand((1, 5, 6, 1), 13)
    w = np.zeros((1, 3, 3, 1))
    w[0, 0, 2, 0] = 1.0
    y = oracle.conv2d_forward(x, w, (1, 1), (1, 1))
    ref = np.zeros_like(x)
    ref[0, 1:, :-1, 0] = x[0, :-1, 1:, 0]
    np.testing.assert_array_equal(y, ref)


def test_output_sizes():
    assert oracle.out_size(224, 224, 7, 7, (2, 2), (3, 3)) == (112, 112)
    assert oracle.out_size(56, 56, 3, 3, (1, 1), (1, 1)) == (56, 56)
    assert oracle.out_size(56, 56, 1, 1, (2, 2), (0, 0)) == (28, 28)
    assert oracle.out_size(15, 15, 3, 3, (2, 2), (1, 1)) == (8, 8)


def test_planted_mistakes_are_caught():
    torch = pytest.importorskip("torch")
    x, w, dy, st, pd = _case(CASES[0], seed=7)
    ref = torch.nn.functional.conv2d(torch.tensor(x.transpose(0, 3, 1, 2)),
                                     torch.tensor(w.transpose(0, 3, 1, 2)),
                                     stride=st, padding=pd).numpy().transpose(0, 2, 3, 1)
    # a true convolution (flipped filter) instead of cross-correlation
    flipped = oracle.conv2d_forward(x, w[:, ::-1, ::-1, :], st, pd)
    assert np.abs(flipped - ref).max() > 1e-3
    # the weight gradient with the tap offset of the wrong sign
    good = oracle.conv2d_backward_filter(x, dy, w.shape, st, pd)
    bad = oracle.conv2d_backward_filter(x[:, ::-1, ::-1, :], dy, w.shape, st, pd)
    assert np.abs(good - bad).max() > 1e-3
    # dropping the padding in the data gradient
    dx = oracle.conv2d_backward_data(dy, w, x.shape, st, pd)
    dx_edge_cut = dx.copy()
    dx_edge_cut[:, 0] = 0
    L = oracle.conv2d_loss(x, w, dy, st, pd)
    assert abs(np.sum(dx_edge_cut * x) - L) > 1e-6
    assert oc.out_size(7, 6, 3, 3, st, pd) == (7, 6)
