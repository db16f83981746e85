"""Rotary position embedding (RoPE) and strided row layouts: float64 CPU oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

What is computed.  "Meganeura: Portable GPU Training and Inference through
Vulkan and Metal" (arXiv 2608.01563) lists axial RoPE among the operations
of its DinoVision case study (Section 5.2) and packed projection forms among
its graph rewrites (Section 3.2), without writing either down.  The rotation
here is the textbook rotary embedding (Su et al., "RoFormer: Enhanced
Transformer with Rotary Position Embedding", 2021) in its rotate-half
arrangement: for a row x of even length D at position p and a table of
angles a[p][i], i < D/2, pair (i, i + D/2) is turned by a[p][i]:

    y_i       = x_i cos a - x_{i+D/2} sin a
    y_{i+D/2} = x_{i+D/2} cos a + x_i sin a

The transpose R^T (which maps a gradient with respect to y to one with
respect to x) turns each pair by -a.  The caller passes cos a and sin a as
two [P, D/2] tables, so 1-D and axial (2-D grid) positions are the same
operation with different tables:

    1-D   : a[p][i] = p * base^(-2i/D)
    axial : position p = r * W + c on an H x W grid; pair i < D/4 takes
            r * base^(-4i/D), pair i >= D/4 takes c * base^(-4(i - D/4)/D)

A strided layout names where element d of row s of head h of batch b lives:
offset b*sB + h*sH + s*sS + d (the head dimension contiguous).  [B, H, S, D]
row-major is (H*S*D, S*D, D); [B, S, H, D] is (S*H*D, D, H*D); a packed
[B, S, 3, H, D] projection holds Q, K, V at offsets 0, H*D, 2*H*D with
strides (S*3*H*D, D, 3*H*D).
"""
from __future__ import annotations

import numpy as np


def rope_angles_1d(positions, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """a[p][i] = positions[p] * base^(-2i/D), float64 [P, D/2]."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def rope_angles_axial(grid_h: int, grid_w: int, head_dim: int,
                      base: float = 10000.0) -> np.ndarray:
    """Axial angles for the H*W positions of a grid, row-major, [H*W, D/2]."""
    if head_dim % 4:
        raise ValueError("axial RoPE needs head_dim divisible by 4")
    q = head_dim // 4
    i = np.arange(q, dtype=np.float64)
    inv = base ** (-4.0 * i / head_dim)
    r, c = np.divmod(np.arange(grid_h * grid_w), grid_w)
    return np.concatenate([r[:, None] * inv[None, :], c[:, None] * inv[None, :]], axis=1)


def rope(x, cos, sin, pos_offset: int = 0) -> np.ndarray:
    """Rotate rows of x [..., S, D]: row s uses table row pos_offset + s."""
    x = np.asarray(x, dtype=np.float64)
    s, d = x.shape[-2], x.shape[-1]
    c = np.asarray(cos, dtype=np.float64)[pos_offset:pos_offset + s]
    sn = np.asarray(sin, dtype=np.float64)[pos_offset:pos_offset + s]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1)


def rope_transpose(g, cos, sin, pos_offset: int = 0) -> np.ndarray:
    """R^T g: each pair turned by the negated angle."""
    return rope(g, cos, -np.asarray(sin, dtype=np.float64), pos_offset)


def gather_rows(buf, offset: int, strides, shape) -> np.ndarray:
    """[B, H, S, D] view of a flat buffer: element (b, h, s, d) at
    offset + b*sB + h*sH + s*sS + d, gathered element by element."""
    B, H, S, D = shape
    sb, sh, ss = strides
    flat = np.asarray(buf).reshape(-1)
    out = np.empty(shape, dtype=flat.dtype)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                base = offset + b * sb + h * sh + s * ss
                out[b, h, s] = flat[base:base + D]
    return out


def scatter_rows(buf, offset: int, strides, x) -> None:
    """Write x [B, H, S, D] into a flat buffer at the strided offsets."""
    B, H, S, D = x.shape
    sb, sh, ss = strides
    flat = buf.reshape(-1)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                base = offset + b * sb + h * sh + s * ss
                flat[base:base + D] = x[b, h, s]
