"""GPU parity of the strided entry points (attn_fwd_strided / attn_bwd_strided)
against the float64 oracle: Q, K, V read straight from a packed
[B, S, 3, H, D] projection or a [B, S, 2, H, D] key/value cache, O and dO in
[B, S, H, D], the gradients written into a packed [B, S, 3, H, D] buffer
(the pages' packed projection forms, Section 3.2), one K/V head shared by
all query heads; with causal masks, padded keys, one-token queries and the
query-chunk split of many queries over few keys."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_host

pytestmark = pytest.mark.gpu


def _exact(x, dt):
    x = np.asarray(x, dtype=np.float32)
    if dt == "bf16":
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    return x


def _dev(x, dt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _bhsd(t, slot=None):
    """[B,H,S,D] view of a [B,S,H,D] tensor, or of slot `slot` of [B,S,n,H,D]."""
    return (t if slot is None else t[:, :, slot]).permute(0, 2, 1, 3)


def _grads_err(host, ref):
    return {k: max_rel_err(host[k], ref[k]) for k in ref}


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,S,D,causal", [(2, 4, 130, 64, True), (2, 3, 197, 32, False),
                                            (1, 2, 256, 128, True)])
def test_packed_qkv_step(B, H, S, D, causal, dt):
    import torch
    note(f"[gpu case] strided packed QKV B{B} H{H} S{S} D{D} causal={causal} dtype={dt} "
         "-> attn_fwd_strided + attn_bwd_strided")
    rng = np.random.default_rng(S + D)
    packed = _exact(rng.standard_normal((B, S, 3, H, D)), dt)
    dO = _exact(rng.standard_normal((B, S, H, D)), dt)
    pk, dOt = _dev(packed, dt), _dev(dO, dt)
    tdt = pk.dtype
    scale = 1.0 / np.sqrt(D)
    o = torch.full((B, S, H, D), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    dpk = torch.full_like(pk, float("nan"))
    q, k, v = (_bhsd(pk, i) for i in range(3))
    afb.attn_fwd_strided(q, k, v, _bhsd(o), lse, None, causal, scale)
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.empty(afb.attn_bwd_cross_workspace_size(code, B, H, S, S, D, causal),
                     dtype=torch.uint8, device="cuda")
    afb.attn_bwd_strided(q, k, v, _bhsd(o), _bhsd(dOt), lse, _bhsd(dpk, 0), _bhsd(dpk, 1),
                         _bhsd(dpk, 2), ws, None, causal, scale)
    torch.cuda.synchronize()
    qo, ko, vo = (packed[:, :, i].transpose(0, 2, 1, 3).astype(np.float64) for i in range(3))
    ro, rl = oracle.attention_forward(qo, ko, vo, causal, scale)
    rdq, rdk, rdv, _ = oracle.attention_backward(qo, ko, vo, dO.transpose(0, 2, 1, 3), causal,
                                                 scale)
    hp = to_host(dpk)
    host = {"o": to_host(o).transpose(0, 2, 1, 3), "lse": to_host(lse),
            "dq": hp[:, :, 0].transpose(0, 2, 1, 3), "dk": hp[:, :, 1].transpose(0, 2, 1, 3),
            "dv": hp[:, :, 2].transpose(0, 2, 1, 3)}
    errs = _grads_err(host, {"o": ro, "lse": rl, "dq": rdq, "dk": rdk, "dv": rdv})
    note("  errors " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[dt], (k_, v_)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,Sq,Sk,D,causal,kvl", [
    (2, 4, 1, 300, 64, True, [300, 97]),        # one-token queries over a KV cache
    (2, 3, 5, 200, 128, True, [200, 3]),        # few queries; rows with no visible key
    (1, 2, 2048, 77, 64, False, None),          # many queries over few keys: query split
    (2, 2, 96, 160, 32, True, [160, 120]),
])
def test_kv_cache_cross(B, H, Sq, Sk, D, causal, kvl, dt):
    """Queries in [B,Sq,H,D], keys and values in a [B,Sk,2,H,D] cache."""
    import torch
    note(f"[gpu case] strided KV cache B{B} H{H} Sq{Sq} Sk{Sk} D{D} causal={causal} "
         f"kv_len={kvl} dtype={dt}")
    rng = np.random.default_rng(Sq * 7 + Sk)
    qn = _exact(rng.standard_normal((B, Sq, H, D)), dt)
    kvn = _exact(rng.standard_normal((B, Sk, 2, H, D)), dt)
    dOn = _exact(rng.standard_normal((B, Sq, H, D)), dt)
    qt, kvt, dOt = _dev(qn, dt), _dev(kvn, dt), _dev(dOn, dt)
    if kvl is not None:  # padded cache rows are never read
        for b, L in enumerate(kvl):
            kvt[b, L:] = float("nan")
    tdt = qt.dtype
    kv_len = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(D)
    o = torch.full((B, Sq, H, D), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((B, H, Sq), float("nan"), device="cuda")
    dq = torch.full((B, Sq, H, D), float("nan"), dtype=tdt, device="cuda")
    dkv = torch.full((B, Sk, 2, H, D), float("nan"), dtype=tdt, device="cuda")
    afb.attn_fwd_strided(_bhsd(qt), _bhsd(kvt, 0), _bhsd(kvt, 1), _bhsd(o), lse, kv_len, causal,
                         scale)
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.empty(afb.attn_bwd_cross_workspace_size(code, B, H, Sq, Sk, D, causal),
                     dtype=torch.uint8, device="cuda")
    afb.attn_bwd_strided(_bhsd(qt), _bhsd(kvt, 0), _bhsd(kvt, 1), _bhsd(o), _bhsd(dOt), lse,
                         _bhsd(dq), _bhsd(dkv, 0), _bhsd(dkv, 1), ws, kv_len, causal, scale)
    torch.cuda.synchronize()
    kvnp = None if kvl is None else np.array(kvl)
    qo = qn.transpose(0, 2, 1, 3).astype(np.float64)
    ko, vo = (kvn[:, :, i].transpose(0, 2, 1, 3).astype(np.float64) for i in range(2))
    ro, rl = oracle.attention_forward(qo, ko, vo, causal, scale, kvnp)
    rdq, rdk, rdv, _ = oracle.attention_backward(qo, ko, vo, dOn.transpose(0, 2, 1, 3), causal,
                                                 scale, kvnp)
    hk = to_host(dkv)
    hl = to_host(lse)
    assert np.array_equal(np.isneginf(hl), np.isneginf(rl))
    fin = np.isfinite(rl)
    errs = {"o": max_rel_err(to_host(o).transpose(0, 2, 1, 3), ro),
            "lse": max_rel_err(hl[fin], rl[fin]) if fin.any() else 0.0,
            "dq": max_rel_err(to_host(dq).transpose(0, 2, 1, 3), rdq),
            "dk": max_rel_err(hk[:, :, 0].transpose(0, 2, 1, 3), rdk),
            "dv": max_rel_err(hk[:, :, 1].transpose(0, 2, 1, 3), rdv)}
    note("  errors " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[dt], (k_, v_)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_shared_kv_head(dt):
    """One K, V head for all query heads (head stride 0 on k and v): the
    forward and per-head dK, dV whose head sum is the shared head's gradient."""
    import torch
    B, H, S, D = 2, 4, 130, 64
    note(f"[gpu case] strided shared K/V head B{B} H{H} S{S} D{D} dtype={dt}")
    rng = np.random.default_rng(11)
    qn = _exact(rng.standard_normal((B, H, S, D)), dt)
    kn, vn = (_exact(rng.standard_normal((B, 1, S, D)), dt) for _ in range(2))
    dOn = _exact(rng.standard_normal((B, H, S, D)), dt)
    qt, kt, vt, dOt = (_dev(x, dt) for x in (qn, kn, vn, dOn))
    kx, vx = kt.expand(B, H, S, D), vt.expand(B, H, S, D)   # head stride 0
    assert kx.stride(1) == 0
    o = torch.empty_like(qt)
    lse = torch.empty((B, H, S), device="cuda")
    dq, dk, dv = torch.empty_like(qt), torch.empty_like(qt), torch.empty_like(qt)
    afb.attn_fwd_strided(qt, kx, vx, o, lse, None, True, 0.125)
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.empty(afb.attn_bwd_cross_workspace_size(code, B, H, S, S, D, True),
                     dtype=torch.uint8, device="cuda")
    afb.attn_bwd_strided(qt, kx, vx, o, dOt, lse, dq, dk, dv, ws, None, True, 0.125)
    torch.cuda.synchronize()
    kb, vb = np.repeat(kn, H, axis=1), np.repeat(vn, H, axis=1)
    ro, _ = oracle.attention_forward(qn, kb, vb, True, 0.125)
    rdq, rdk, rdv, _ = oracle.attention_backward(qn, kb, vb, dOn, True, 0.125)
    errs = {"o": max_rel_err(to_host(o), ro), "dq": max_rel_err(to_host(dq), rdq),
            "dk_sum": max_rel_err(to_host(dk).astype(np.float64).sum(1), rdk.sum(1)),
            "dv_sum": max_rel_err(to_host(dv).astype(np.float64).sum(1), rdv.sum(1))}
    note("  errors " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[dt], (k_, v_)
    shared = torch.empty_like(kt).expand(B, H, S, D)
    with pytest.raises(afb.AttnError):   # a shared dK head would be written by every head
        afb.attn_bwd_strided(qt, kx, vx, o, dOt, lse, dq, shared, dv, ws, None, True, 0.125)
