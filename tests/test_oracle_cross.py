"""Pins of the oracle's cross-attention generalisation (queries Sq, keys Sk,
L_b valid keys per batch, causal diagonal aligned with the end of the valid
keys; rows with no visible key give O = 0, LSE = -inf, no gradient).

Each pin checks the oracle against something other than its own vectorised
code: a pure-Python brute force, a property that fixes the reading (padding
equals truncation, padded rows cannot matter, the bottom-right alignment makes
a query row's result independent of how many queries precede it, a one-token
causal query sees every valid key), and central finite differences."""
import math

import numpy as np
import pytest

from oracle import attention_backward, attention_forward
from oracle.fdcheck import fd_full


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, causal, scale, L):
    """One (b, h) slice with loops: visibility by the stated rule, softmax by
    math.exp, O by explicit sums."""
    sq, sk, d = q.shape[0], k.shape[0], v.shape[1]
    o = [[0.0] * d for _ in range(sq)]
    lse = [-math.inf] * sq
    for i in range(sq):
        vis = [j for j in range(sk) if j < L and (not causal or j <= i + L - sq)]
        if not vis:
            continue
        sc = {j: scale * sum(q[i][t] * k[j][t] for t in range(q.shape[1])) for j in vis}
        mx = max(sc.values())
        den = sum(math.exp(x - mx) for x in sc.values())
        lse[i] = mx + math.log(den)
        for j in vis:
            w = math.exp(sc[j] - mx) / den
            for t in range(d):
                o[i][t] += w * v[j][t]
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,sk", [(1, 1), (1, 6), (3, 5), (5, 3), (4, 4), (7, 2)])
def test_forward_matches_brute_force(sq, sk, causal):
    B, H, D = 3, 2, 4
    q, k, v = _rand((B, H, sq, D), 1), _rand((B, H, sk, D), 2), _rand((B, H, sk, D), 3)
    kv_len = np.array([sk, max(0, sk - 2), 0])[:B]
    o, lse = attention_forward(q, k, v, causal, 0.7, kv_len)
    for b in range(B):
        for h in range(H):
            ob, lb = _brute(q[b, h], k[b, h], v[b, h], causal, 0.7, int(kv_len[b]))
            np.testing.assert_allclose(o[b, h], ob, rtol=1e-12, atol=1e-12)
            assert np.array_equal(np.isinf(lse[b, h]), np.isinf(lb))
            fin = np.isfinite(lb)
            np.testing.assert_allclose(lse[b, h][fin], lb[fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_padding_equals_truncation(causal):
    """kv_len = L on Sk keys gives exactly what the first L keys alone give."""
    B, H, sq, sk, D = 3, 2, 6, 9, 5
    q, k, v, do = _rand((B, H, sq, D), 4), _rand((B, H, sk, D), 5), _rand((B, H, sk, D), 6), \
        _rand((B, H, sq, D), 7)
    kv_len = np.array([9, 4, 7])
    o, lse = attention_forward(q, k, v, causal, 0.4, kv_len)
    dq, dk, dv, _ = attention_backward(q, k, v, do, causal, 0.4, kv_len)
    for b in range(B):
        L = int(kv_len[b])
        sl = slice(b, b + 1)
        o_t, lse_t = attention_forward(q[sl], k[sl, :, :L], v[sl, :, :L], causal, 0.4)
        dq_t, dk_t, dv_t, _ = attention_backward(q[sl], k[sl, :, :L], v[sl, :, :L], do[sl],
                                                 causal, 0.4)
        np.testing.assert_allclose(o[sl], o_t, rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(np.isinf(lse[sl]), np.isinf(lse_t))
        np.testing.assert_allclose(dq[sl], dq_t, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dk[sl, :, :L], dk_t, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv[sl, :, :L], dv_t, rtol=1e-12, atol=1e-12)
        assert not dk[sl, :, L:].any() and not dv[sl, :, L:].any()


@pytest.mark.parametrize("causal", [False, True])
def test_padded_rows_cannot_matter(causal):
    """Arbitrary (huge) values in K and V rows past L change nothing."""
    B, H, sq, sk, D = 2, 2, 5, 8, 4
    q, k, v, do = _rand((B, H, sq, D), 8), _rand((B, H, sk, D), 9), _rand((B, H, sk, D), 10), \
        _rand((B, H, sq, D), 11)
    kv_len = np.array([5, 3])
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(kv_len):
        k2[b, :, L:] = 1e6
        v2[b, :, L:] = -1e6
    ref = attention_forward(q, k, v, causal, 0.5, kv_len) + attention_backward(q, k, v, do, causal, 0.5, kv_len)[:3]
    got = attention_forward(q, k2, v2, causal, 0.5, kv_len) + attention_backward(q, k2, v2, do, causal, 0.5, kv_len)[:3]
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)


def test_bottom_right_alignment():
    """The last query row sees every valid key, and dropping leading query rows
    leaves the remaining rows' results unchanged (causal, Sq != Sk)."""
    B, H, sq, sk, D = 2, 2, 6, 10, 4
    q, k, v = _rand((B, H, sq, D), 12), _rand((B, H, sk, D), 13), _rand((B, H, sk, D), 14)
    kv_len = np.array([10, 7])
    o, lse = attention_forward(q, k, v, True, 0.6, kv_len)
    o_nc, lse_nc = attention_forward(q, k, v, False, 0.6, kv_len)
    np.testing.assert_allclose(o[:, :, -1], o_nc[:, :, -1], rtol=1e-13, atol=1e-13)
    for drop in (1, 3, 5):
        o2, lse2 = attention_forward(q[:, :, drop:], k, v, True, 0.6, kv_len)
        np.testing.assert_allclose(o2, o[:, :, drop:], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse2, lse[:, :, drop:], rtol=1e-13, atol=1e-13)


def test_one_token_query():
    """Sq = 1: causal equals non-causal (the query sees every valid key) and O
    is the plain softmax-weighted sum."""
    B, H, sk, D = 2, 3, 9, 6
    q, k, v = _rand((B, H, 1, D), 15), _rand((B, H, sk, D), 16), _rand((B, H, sk, D), 17)
    kv_len = np.array([9, 4])
    o_c, _ = attention_forward(q, k, v, True, 0.3, kv_len)
    o_n, _ = attention_forward(q, k, v, False, 0.3, kv_len)
    np.testing.assert_allclose(o_c, o_n, rtol=1e-14, atol=1e-14)
    for b in range(B):
        L = int(kv_len[b])
        for h in range(H):
            s = 0.3 * k[b, h, :L] @ q[b, h, 0]
            w = np.exp(s - s.max())
            np.testing.assert_allclose(o_c[b, h, 0], (w / w.sum()) @ v[b, h, :L], rtol=1e-12)


def test_empty_rows():
    """No visible key: O = 0, LSE = -inf, zero gradients (L = 0; causal Sq > L)."""
    B, H, sq, sk, D = 2, 2, 7, 5, 3
    q, k, v, do = _rand((B, H, sq, D), 18), _rand((B, H, sk, D), 19), _rand((B, H, sk, D), 20), \
        _rand((B, H, sq, D), 21)
    kv_len = np.array([0, 4])
    o, lse = attention_forward(q, k, v, True, 0.5, kv_len)
    dq, dk, dv, delta = attention_backward(q, k, v, do, True, 0.5, kv_len)
    assert not o[0].any() and np.all(np.isneginf(lse[0])) and not dq[0].any()
    assert not dk[0].any() and not dv[0].any() and not delta[0].any()
    # batch 1: L = 4, Sq = 7 -> rows 0..2 see nothing, row 3 sees key 0
    assert not o[1, :, :3].any() and np.all(np.isneginf(lse[1, :, :3])) and not dq[1, :, :3].any()
    assert np.all(np.isfinite(lse[1, :, 3:]))


@pytest.mark.parametrize("causal", [False, True])
def test_cross_gradients_finite_differences(causal):
    B, H, sq, sk, D = 2, 1, 3, 5, 3
    q, k, v, do = _rand((B, H, sq, D), 22), _rand((B, H, sk, D), 23), _rand((B, H, sk, D), 24), \
        _rand((B, H, sq, D), 25)
    kv_len = np.array([5, 3])
    dq, dk, dv, _ = attention_backward(q, k, v, do, causal, 0.8, kv_len)
    fd = fd_full(q, k, v, do, causal, 0.8, kv_len=kv_len)
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        np.testing.assert_allclose(g, fd[name], rtol=1e-6, atol=1e-7, err_msg=name)
