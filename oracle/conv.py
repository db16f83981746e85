"""Plain float64 CPU oracle for 2-D convolution and its two derivatives.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

What is computed.  "Meganeura: Portable GPU Training and Inference through
Vulkan and Metal" (arXiv 2608.01563) lists convolution among its graph nodes
with a local derivative rule (Section 3.1), names the backward-only input and
weight derivatives of convolution (Section 3.1, automatic differentiation),
lowers them to implicit-GEMM and spatial kernels (Section 3.3), and profiles
three derivative kernels (weight gradient, small weight gradient, input
gradient) as most of a ResNet-50 training step (Section 7.3).  The pages never
write the operation, so this oracle is the textbook cross-correlation used by
deep-learning convolution layers, with zero padding and a stride, in NHWC
layout:

    y[n,p,q,k]  = sum_{r,s,c} x[n, p*sh + r - ph, q*sw + s - pw, c] * w[k,r,s,c]
                  (x outside [0,H) x [0,W) is zero)
    P = (H + 2 ph - R) // sh + 1,   Q = (W + 2 pw - S) // sw + 1

and, for a loss whose gradient with respect to y is dy, the two adjoints

    dx[n,h,w,c] = sum over (p,q,r,s) with p*sh + r - ph = h, q*sw + s - pw = w
                  of sum_k dy[n,p,q,k] * w[k,r,s,c]
    dw[k,r,s,c] = sum_{n,p,q} dy[n,p,q,k] * x[n, p*sh + r - ph, q*sw + s - pw, c]

Readings where the pages are silent: layouts x [N,H,W,C], w [K,R,S,C],
y and dy [N,P,Q,K]; no dilation, no groups, no bias; the output size rounds
down.  Everything is float64, one filter tap (r, s) at a time over a
zero-padded copy of x: no im2col matrix, no tiling.
"""
from __future__ import annotations

import numpy as np


def out_size(H: int, W: int, R: int, S: int, stride, pad):
    sh, sw = stride
    ph, pw = pad
    return (H + 2 * ph - R) // sh + 1, (W + 2 * pw - S) // sw + 1


def _tap_view(xp: np.ndarray, r: int, s: int, P: int, Q: int, stride):
    """The input pixels that filter tap (r, s) meets for every output (p, q):
    xp[n, p*sh + r, q*sw + s, :] of the padded input, as [N, P, Q, C]."""
    sh, sw = stride
    return xp[:, r:r + sh * (P - 1) + 1:sh, s:s + sw * (Q - 1) + 1:sw, :]


def conv2d_forward(x: np.ndarray, w: np.ndarray, stride=(1, 1), pad=(0, 0)) -> np.ndarray:
    """y [N,P,Q,K] from x [N,H,W,C] and w [K,R,S,C] (definition above)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    assert C == C2
    P, Q = out_size(H, W, R, S, stride, pad)
    xp = np.pad(x, ((0, 0), (pad[0], pad[0]), (pad[1], pad[1]), (0, 0)))
    y = np.zeros((N, P, Q, K))
    for r in range(R):
        for s in range(S):
            y += _tap_view(xp, r, s, P, Q, stride) @ w[:, r, s, :].T
    return y


def conv2d_backward_data(dy: np.ndarray, w: np.ndarray, x_shape, stride=(1, 1),
                         pad=(0, 0)) -> np.ndarray:
    """dx [N,H,W,C]: every output pixel sends dy[n,p,q,:] @ w[:,r,s,:] back to
    the input pixel that tap (r, s) read (padding positions are dropped)."""
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, H, W, C = x_shape
    K, R, S, _ = w.shape
    P, Q = out_size(H, W, R, S, stride, pad)
    assert dy.shape == (N, P, Q, K)
    dxp = np.zeros((N, H + 2 * pad[0], W + 2 * pad[1], C))
    for r in range(R):
        for s in range(S):
            _tap_view(dxp, r, s, P, Q, stride)[...] += dy @ w[:, r, s, :]
    return dxp[:, pad[0]:pad[0] + H, pad[1]:pad[1] + W, :]


def conv2d_backward_filter(x: np.ndarray, dy: np.ndarray, w_shape, stride=(1, 1),
                           pad=(0, 0)) -> np.ndarray:
    """dw [K,R,S,C]: for every tap, the sum over all output pixels of
    dy[n,p,q,k] times the input pixel the tap read."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    N, H, W, C = x.shape
    K, R, S, _ = w_shape
    P, Q = out_size(H, W, R, S, stride, pad)
    assert dy.shape == (N, P, Q, K)
    xp = np.pad(x, ((0, 0), (pad[0], pad[0]), (pad[1], pad[1]), (0, 0)))
    dw = np.zeros((K, R, S, C))
    dyf = dy.reshape(-1, K)
    for r in range(R):
        for s in range(S):
            dw[:, r, s, :] = dyf.T @ _tap_view(xp, r, s, P, Q, stride).reshape(-1, C)
    return dw


def conv2d_loss(x, w, dy, stride=(1, 1), pad=(0, 0)) -> float:
    """L = sum y * dy, whose gradients are dx and dw above."""
    return float(np.sum(conv2d_forward(x, w, stride, pad) * np.asarray(dy, dtype=np.float64)))
