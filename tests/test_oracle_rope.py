"""Pins for the RoPE and strided-layout oracle (CPU): a hand-worked rotation,
the complex-multiplication form of the rotation, orthogonality, the adjoint,
relative-position dependence of rotated dot products, the angle tables, and
strided gathers against numpy reshapes and transposes."""
import numpy as np
import pytest

import oracle


def test_hand_example():
    # D = 4, pairs (0, 2) and (1, 3); pair 0 turned by pi/2, pair 1 by 0:
    # (1, 3) -> (-3, 1) and (2, 4) unchanged, so [1, 2, 3, 4] -> [-3, 2, 1, 4]
    ang = np.array([[np.pi / 2, 0.0]])
    y = oracle.rope(np.array([[1.0, 2.0, 3.0, 4.0]]), np.cos(ang), np.sin(ang))
    assert np.allclose(y, [[-3.0, 2.0, 1.0, 4.0]], atol=1e-15, rtol=0)
    # a positive quarter turn of pair 1 instead: (2, 4) -> (-4, 2)
    ang = np.array([[0.0, np.pi / 2]])
    y = oracle.rope(np.array([[1.0, 2.0, 3.0, 4.0]]), np.cos(ang), np.sin(ang))
    assert np.allclose(y, [[1.0, -4.0, 3.0, 2.0]], atol=1e-15, rtol=0)


def test_complex_form():
    """Pair (i, i + D/2) as the complex number x_i + j x_{i+D/2}, multiplied
    by exp(j a)."""
    rng = np.random.default_rng(0)
    S, D = 7, 16
    x = rng.standard_normal((2, 3, S, D))
    ang = rng.uniform(-4, 4, (S + 2, D // 2))
    y = oracle.rope(x, np.cos(ang), np.sin(ang), pos_offset=2)
    z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * ang[2:2 + S])
    assert np.allclose(y, np.concatenate([z.real, z.imag], axis=-1), atol=1e-14, rtol=0)


def test_orthogonal_and_adjoint():
    rng = np.random.default_rng(1)
    S, D = 9, 32
    x, g = rng.standard_normal((2, 2, 3, S, D))
    ang = rng.uniform(-10, 10, (S, D // 2))
    c, s = np.cos(ang), np.sin(ang)
    y = oracle.rope(x, c, s)
    # pair norms kept, R^T R = I, and <R x, g> = <x, R^T g>
    n = lambda a: a[..., : D // 2] ** 2 + a[..., D // 2:] ** 2
    assert np.allclose(n(y), n(x), rtol=1e-13, atol=1e-13)
    assert np.allclose(oracle.rope_transpose(y, c, s), x, atol=1e-13, rtol=0)
    assert np.isclose((y * g).sum(), (x * oracle.rope_transpose(g, c, s)).sum(), rtol=1e-13)
    # the transpose is the inverse, not the same rotation
    assert not np.allclose(oracle.rope(y, c, s), x)


def test_relative_position():
    """With 1-D tables, <R_m q, R_n k> depends on m - n only."""
    rng = np.random.default_rng(2)
    D = 64
    q, k = rng.standard_normal((2, D))
    ang = oracle.rope_angles_1d(np.arange(40), D)
    c, s = np.cos(ang), np.sin(ang)
    rq = oracle.rope(np.tile(q, (40, 1)), c, s)
    rk = oracle.rope(np.tile(k, (40, 1)), c, s)
    sc = rq @ rk.T
    for t in range(-5, 6):
        d = np.diagonal(sc, offset=t)
        assert np.allclose(d, d[0], rtol=1e-12, atol=1e-12)
    assert not np.allclose(np.diagonal(sc, 1)[0], np.diagonal(sc, 2)[0])


def test_angle_tables():
    D = 16
    a = oracle.rope_angles_1d(np.arange(5), D, base=10000.0)
    assert a.shape == (5, 8) and np.all(a[0] == 0)
    assert np.allclose(a[:, 0], np.arange(5))                   # theta_0 = 1
    assert np.isclose(a[3, 7], 3 * 10000.0 ** (-14 / 16))
    g = oracle.rope_angles_axial(3, 4, D, base=100.0)
    assert g.shape == (12, 8)
    r, c = np.divmod(np.arange(12), 4)
    assert np.allclose(g[:, 0], r) and np.allclose(g[:, 4], c)   # first pair of each half
    assert np.isclose(g[7, 1], 1 * 100.0 ** (-4 / 16)) and np.isclose(g[7, 5], 3 * 100.0 ** (-4 / 16))
    with pytest.raises(ValueError):
        oracle.rope_angles_axial(2, 2, 18)


def test_strided_gather_scatter():
    rng = np.random.default_rng(3)
    B, H, S, D = 2, 3, 5, 8
    bhsd = rng.standard_normal((B, H, S, D))
    assert np.array_equal(oracle.gather_rows(bhsd, 0, (H * S * D, S * D, D), (B, H, S, D)), bhsd)
    bshd = rng.standard_normal((B, S, H, D))
    got = oracle.gather_rows(bshd, 0, (S * H * D, D, H * D), (B, H, S, D))
    assert np.array_equal(got, bshd.transpose(0, 2, 1, 3))
    packed = rng.standard_normal((B, S, 3, H, D))
    st = (S * 3 * H * D, D, 3 * H * D)
    for w in range(3):
        got = oracle.gather_rows(packed, w * H * D, st, (B, H, S, D))
        assert np.array_equal(got, packed[:, :, w].transpose(0, 2, 1, 3))
    out = np.zeros_like(packed)
    for w in range(3):
        oracle.scatter_rows(out, w * H * D, st, packed[:, :, w].transpose(0, 2, 1, 3))
    assert np.array_equal(out, packed)


def test_rotated_attention_scores_are_toeplitz():
    """Attention on rotated Q, K with equal query rows and equal key rows:
    the probabilities of the non-causal softmax depend on i - j only up to
    each row's normaliser, so the raw scores (through the LSE) are constant
    along diagonals."""
    rng = np.random.default_rng(4)
    S, D = 12, 32
    q = np.tile(rng.standard_normal(D), (1, 1, S, 1))
    k = np.tile(rng.standard_normal(D), (1, 1, S, 1))
    ang = oracle.rope_angles_1d(np.arange(S), D)
    rq = oracle.rope(q, np.cos(ang), np.sin(ang))
    rk = oracle.rope(k, np.cos(ang), np.sin(ang))
    p = oracle.attention_probs(rq, rk, False, 0.25)[0, 0]
    _, lse = oracle.attention_forward(rq, rk, rk, False, 0.25)
    scores = np.log(p) + lse[0, 0][:, None]
    for t in range(-3, 4):
        d = np.diagonal(scores, offset=t)
        assert np.allclose(d, d[0], rtol=1e-10, atol=1e-10)
