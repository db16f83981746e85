"""Central finite-difference gradient checker for the attention oracle.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see ``oracle/attention.py``).

The loss is L = sum(O * dO) (its gradient with respect to O is dO), so the
derivative of L with respect to each element of Q, K and V is what
``attention_backward`` must return.  This module perturbs one input element at
a time by +-h, with h = rel_step * max(1, |x|), and evaluates L with the
oracle's own forward: it checks the backward against the forward, and knows
nothing of how the backward is computed.
"""
from __future__ import annotations

import numpy as np

from .attention import loss


def fd_grad(q, k, v, do, causal: bool, scale: float, which: str, coords,
            rel_step: float = 1e-6, kv_len=None):
    """Central-difference dL/d<which> at the given flat coordinates."""
    arrays = {n: np.array(a, dtype=np.float64, copy=True)
              for n, a in (("q", q), ("k", k), ("v", v))}
    x = arrays[which].reshape(-1)
    out = np.empty(len(coords))
    for n, c in enumerate(coords):
        orig = x[c]
        h = rel_step * max(1.0, abs(orig))
        x[c] = orig + h
        lp = loss(arrays["q"], arrays["k"], arrays["v"], do, causal, scale, kv_len)
        x[c] = orig - h
        lm = loss(arrays["q"], arrays["k"], arrays["v"], do, causal, scale, kv_len)
        x[c] = orig
        out[n] = (lp - lm) / (2.0 * h)
    return out


def fd_full(q, k, v, do, causal: bool, scale: float, rel_step: float = 1e-6, kv_len=None):
    """Central differences over every element of Q, K and V (tiny shapes only)."""
    res = {}
    for which, a in (("q", q), ("k", k), ("v", v)):
        n = int(np.prod(np.shape(a)))
        res[which] = fd_grad(q, k, v, do, causal, scale, which, range(n),
                             rel_step, kv_len).reshape(np.shape(a))
    return res
