"""GPU parity of the rotary-embedding / layout pass (attn_rope_copy) against
the float64 oracle, alone and composed with the attention forward and
backward on a packed [B, S, 3, H, D] projection (the pages' packed projection
form, Section 3.2, with the RoPE of their DinoVision case, Section 5.2)."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_host

pytestmark = pytest.mark.gpu

# one rounding of the rotated value to bf16 (nearest-even: 2^-9 relative),
# on top of float32 arithmetic
ROT_TOL = {"f32": 1e-6, "bf16": 4e-3}


def _dev(x, dt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _exact(x, dt):
    """The values a device tensor of dtype dt holds for x (bf16: rounded)."""
    x = np.asarray(x, dtype=np.float32)
    if dt == "bf16":
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    return x


def _tables(P, D, axial=None):
    import torch
    ang = oracle.rope_angles_axial(*axial, D) if axial else oracle.rope_angles_1d(np.arange(P), D)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    return c, s, torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_rope_copy_layouts(dt, D):
    import torch
    B, H, S = 2, 3, 37
    note(f"[gpu case] rope copy B{B} H{H} S{S} D{D} dtype={dt}")
    rng = np.random.default_rng(D)
    packed = _exact(rng.standard_normal((B, S, 3, H, D)), dt)
    c, s, ct, st = _tables(S + 5, D)
    pk = _dev(packed, dt)
    offs, pst = afb.packed_qkv(H, S, D)
    bhsd = afb.strides_bhsd(H, S, D)
    bshd = afb.strides_bshd(H, S, D)
    nan = float("nan")
    q = oracle.gather_rows(packed, offs[0], pst, (B, H, S, D)).astype(np.float64)
    # packed Q -> [B,H,S,D], rotated, table rows 5..5+S-1
    out = torch.full((B, H, S, D), nan, dtype=pk.dtype, device="cuda")
    afb.attn_rope_copy(pk, offs[0], pst, out, 0, bhsd, (B, H, S, D), ct, st, pos_offset=5)
    # [B,H,S,D] -> [B,S,H,D], transposed rotation
    out2 = torch.full((B, S, H, D), nan, dtype=pk.dtype, device="cuda")
    afb.attn_rope_copy(out, 0, bhsd, out2, 0, bshd, (B, H, S, D), ct, st, transpose=True)
    # packed V -> [B,H,S,D], plain copy; then in place rotation of that copy
    v = torch.full((B, H, S, D), nan, dtype=pk.dtype, device="cuda")
    afb.attn_rope_copy(pk, offs[2], pst, v, 0, bhsd, (B, H, S, D))
    v_copy = v.clone()
    afb.attn_rope_copy(v, 0, bhsd, v, 0, bhsd, (B, H, S, D), ct, st)
    # scatter into slot 1 of a packed buffer: the other slots stay untouched
    dst = torch.full_like(pk, 7.0)
    afb.attn_rope_copy(out, 0, bhsd, dst, offs[1], pst, (B, H, S, D))
    torch.cuda.synchronize()

    ref1 = oracle.rope(q, c, s, pos_offset=5)
    assert max_rel_err(to_host(out), ref1) <= ROT_TOL[dt]
    ref2 = oracle.rope_transpose(_exact(to_host(out), dt), c, s).transpose(0, 2, 1, 3)
    assert max_rel_err(to_host(out2), ref2) <= ROT_TOL[dt]
    vref = oracle.gather_rows(packed, offs[2], pst, (B, H, S, D))
    assert np.array_equal(to_host(v_copy), vref)                     # a copy is exact
    assert max_rel_err(to_host(v), oracle.rope(vref, c, s)) <= ROT_TOL[dt]
    d = to_host(dst)
    assert np.array_equal(d[:, :, 1].transpose(0, 2, 1, 3), to_host(out))
    assert np.all(d[:, :, 0] == 7.0) and np.all(d[:, :, 2] == 7.0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,S,D,causal,axial", [(2, 4, 130, 64, True, None),
                                                   (2, 2, 64, 64, False, (8, 8)),
                                                   (1, 2, 200, 128, True, None)])
def test_packed_qkv_rope_train_step(B, H, S, D, causal, axial, dt):
    """Packed QKV projection -> RoPE on Q, K -> attention fwd + bwd ->
    O in [B,S,H,D] and the gradient of the packed projection, against the
    oracle composed the same way (dQ = R^T dQ', dK = R^T dK')."""
    import torch
    note(f"[gpu case] packed QKV + RoPE B{B} H{H} S{S} D{D} causal={causal} axial={axial} "
         f"dtype={dt} -> attn_rope_copy + attn_fwd + attn_bwd")
    rng = np.random.default_rng(S)
    packed = _exact(rng.standard_normal((B, S, 3, H, D)), dt)
    dO = _exact(rng.standard_normal((B, S, H, D)), dt)
    c, s, ct, st = _tables(S, D, axial)
    scale = 1.0 / np.sqrt(D)
    pk, dOt = _dev(packed, dt), _dev(dO, dt)
    tdt = pk.dtype
    offs, pst = afb.packed_qkv(H, S, D)
    bhsd, bshd = afb.strides_bhsd(H, S, D), afb.strides_bshd(H, S, D)
    shp = (B, H, S, D)
    q, k, v, o, do, dq, dk, dv = (torch.empty(shp, dtype=tdt, device="cuda") for _ in range(8))
    lse = torch.empty((B, H, S), device="cuda")
    afb.attn_rope_copy(pk, offs[0], pst, q, 0, bhsd, shp, ct, st)
    afb.attn_rope_copy(pk, offs[1], pst, k, 0, bhsd, shp, ct, st)
    afb.attn_rope_copy(pk, offs[2], pst, v, 0, bhsd, shp)
    afb.attn_fwd(q, k, v, o, lse, causal, scale)
    o_bshd = torch.full((B, S, H, D), float("nan"), dtype=tdt, device="cuda")
    afb.attn_rope_copy(o, 0, bhsd, o_bshd, 0, bshd, shp)
    afb.attn_rope_copy(dOt, 0, bshd, do, 0, bhsd, shp)
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.empty(afb.attn_bwd_workspace_size(code, B, H, S, D, causal), dtype=torch.uint8,
                     device="cuda")
    afb.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal, scale)
    dpk = torch.full_like(pk, float("nan"))
    afb.attn_rope_copy(dq, 0, bhsd, dpk, offs[0], pst, shp, ct, st, transpose=True)
    afb.attn_rope_copy(dk, 0, bhsd, dpk, offs[1], pst, shp, ct, st, transpose=True)
    afb.attn_rope_copy(dv, 0, bhsd, dpk, offs[2], pst, shp)
    torch.cuda.synchronize()

    qo, ko, vo = (oracle.gather_rows(packed, offs[i], pst, shp).astype(np.float64) for i in range(3))
    rq, rk = oracle.rope(qo, c, s), oracle.rope(ko, c, s)
    do_o = dO.transpose(0, 2, 1, 3).astype(np.float64)
    ro, _ = oracle.attention_forward(rq, rk, vo, causal, scale)
    rdq, rdk, rdv, _ = oracle.attention_backward(rq, rk, vo, do_o, causal, scale)
    gq, gk = oracle.rope_transpose(rdq, c, s), oracle.rope_transpose(rdk, c, s)
    ref_dp = np.stack([gq.transpose(0, 2, 1, 3), gk.transpose(0, 2, 1, 3),
                       rdv.transpose(0, 2, 1, 3)], axis=2)
    hp = to_host(dpk)
    errs = {"o": max_rel_err(to_host(o_bshd), ro.transpose(0, 2, 1, 3)),
            "dq": max_rel_err(hp[:, :, 0], ref_dp[:, :, 0]),
            "dk": max_rel_err(hp[:, :, 1], ref_dp[:, :, 1]),
            "dv": max_rel_err(hp[:, :, 2], ref_dp[:, :, 2])}
    note("  errors " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[dt], (k_, v_)
