"""Plain float64 CPU oracle for scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and imports nothing from it.

What is computed.  "Meganeura: Portable GPU Training and Inference through
Vulkan and Metal" (arXiv 2608.01563) names attention as one graph node with a
local derivative rule (Section 3.1), lowered to tiled attention forward, dQ and
fused dK+dV kernels (Section 3.3), and its arithmetic contracts (Section 4.2).
The pages never write the formula, so this oracle is the textbook definition
of scaled-dot-product attention with the row log-sum-exp saved, for each
(batch, head) slice independently:

    S_ij  = s * sum_d Q_id K_jd                 (j visible from i)
    LSE_i = log sum_{j visible} exp(S_ij)       (natural log, scale included)
    P_ij  = exp(S_ij - LSE_i), 0 if j is not visible
    O_i   = sum_j P_ij V_j

and, for a loss L whose gradient with respect to O is dO,

    dV_j  = sum_i P_ij dO_i
    dP_ij = sum_d dO_id V_jd
    D_i   = sum_d dO_id O_id
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = s sum_j dS_ij K_j ,   dK_j = s sum_i dS_ij Q_i

Readings where the pages are silent: tensors are [B, H, S, D] row-major
(queries [B, H, Sq, D], keys and values [B, H, Sk, D]); batch b has L_b <= Sk
valid keys (kv_len; all Sk when absent), and key j is visible from query i iff
j < L_b and, in the causal case, j <= i + L_b - Sq (the causal diagonal is
aligned with the end of the valid keys; with Sq = Sk = L_b this is j <= i); a
query row with no visible key has O = 0, LSE = -inf and no gradient; the scale
multiplies the scores before the softmax; LSE uses the natural logarithm.

Everything is float64, one (b, h) slice at a time, with the full S x S score
matrix: no tiling, no online softmax, no reordering beyond what numpy's matmul
does inside one product.
"""
from __future__ import annotations

import numpy as np


def _visible(sq: int, sk: int, causal: bool, nvalid=None) -> np.ndarray:
    """Boolean Sq x Sk matrix, True where query i may attend to key j."""
    L = sk if nvalid is None else int(nvalid)
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    vis = j < L
    if causal:
        vis = vis & (j <= i + (L - sq))
    return vis


def _slice_softmax(q, k, causal, scale, nvalid=None):
    """Scores, row LSE and probabilities for one (b, h) slice, in float64.
    Rows with no visible key get P = 0 and LSE = -inf."""
    s = scale * (q @ k.T)
    vis = _visible(q.shape[0], k.shape[0], causal, nvalid)
    s = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1, keepdims=True)
    m = np.where(any_vis, s.max(axis=1, keepdims=True), 0.0)
    e = np.where(vis, np.exp(s - m), 0.0)
    l = e.sum(axis=1, keepdims=True)
    lse = np.where(any_vis, m + np.log(np.where(any_vis, l, 1.0)), -np.inf)
    p = e / np.where(any_vis, l, 1.0)
    return s, lse[:, 0], p


def _nvalid(kv_len, b):
    return None if kv_len is None else int(kv_len[b])


def _as64(*arrays):
    return [np.asarray(a, dtype=np.float64) for a in arrays]


def attention_forward(q, k, v, causal: bool, scale: float, kv_len=None):
    """O [B,H,Sq,D] and LSE [B,H,Sq] in float64 (kv_len: valid keys per batch)."""
    q, k, v = _as64(q, k, v)
    bsz, nh, sq, hd = q.shape
    o = np.empty((bsz, nh, sq, v.shape[-1]))
    lse = np.empty((bsz, nh, sq))
    for b in range(bsz):
        for h in range(nh):
            _, lse_bh, p = _slice_softmax(q[b, h], k[b, h], causal, scale, _nvalid(kv_len, b))
            o[b, h] = p @ v[b, h]
            lse[b, h] = lse_bh
    return o, lse


def attention_backward(q, k, v, do, causal: bool, scale: float, kv_len=None):
    """dQ, dK, dV and D = rowsum(dO * O) [B,H,Sq], in float64.

    O is the oracle's own forward output (the exact O), so D is exact too.
    """
    q, k, v, do = _as64(q, k, v, do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    delta = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            _, _, p = _slice_softmax(q[b, h], k[b, h], causal, scale, _nvalid(kv_len, b))
            o = p @ v[b, h]
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            d_i = (do[b, h] * o).sum(axis=1)
            ds = p * (dp - d_i[:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
            delta[b, h] = d_i
    return dq, dk, dv, delta


def attention_probs(q, k, causal: bool, scale: float, kv_len=None):
    """P [B,H,Sq,Sk] (float64), for pins and diagnostics on small shapes."""
    q, k = _as64(q, k)
    p = np.empty(q.shape[:3] + (k.shape[2],))
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            p[b, h] = _slice_softmax(q[b, h], k[b, h], causal, scale, _nvalid(kv_len, b))[2]
    return p


def loss(q, k, v, do, causal: bool, scale: float, kv_len=None) -> float:
    """The scalar L = sum(O * dO), whose gradient with respect to O is dO."""
    o, _ = attention_forward(q, k, v, causal, scale, kv_len)
    return float((o * np.asarray(do, dtype=np.float64)).sum())


def attention_forward_rows(q, k, v, causal: bool, scale: float, b: int, h: int, rows,
                           kv_len=None):
    """O and LSE for selected query rows of one (b, h) slice, each row on its own.

    For spot checks at sizes where the full oracle is slow: row i uses only
    its visible keys (the first min(L, i + 1 + L - Sq) when causal, else the
    first L), exactly as in ``attention_forward``.
    """
    sq = q.shape[2]
    q, k, v = _as64(q[b, h], k[b, h], v[b, h])
    L = k.shape[0] if kv_len is None else int(kv_len[b])
    outs, lses = [], []
    for i in rows:
        n_vis = max(0, min(L, i + 1 + L - sq)) if causal else L
        if n_vis == 0:
            outs.append(np.zeros(v.shape[1]))
            lses.append(-np.inf)
            continue
        s = scale * (k[:n_vis] @ q[i])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        outs.append((e / l) @ v[:n_vis])
        lses.append(m + np.log(l))
    return np.array(outs), np.array(lses)
