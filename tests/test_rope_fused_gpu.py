"""GPU parity of the fused RoPE entry points (attn_fwd_rope, attn_bwd_rope):
a packed [B, S, 3, H, D] projection (the pages' packed projection form,
Section 3.2) with RoPE on Q and K (the axial RoPE of their DinoVision case,
Section 5.2, and its 1-D form), O and dO in [B, S, H, D], the gradient
written into a packed buffer.  Checked against the float64 oracle composed
the same way (turn Q and K, attend, dQ = R^T dQ', dK = R^T dK'), against
the separate-pass path (attn_rope_copy around the strided kernels), and the
turned Q and K the forward leaves in qk_rot against attn_rope_copy's output,
bit for bit.  Every workspace layout of the backward is exercised: the
recommended one (dS path, with the dK+dV query split where the shape takes
it) and the minimum (dQ with recomputed scores)."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_host, workspace_bytes

pytestmark = pytest.mark.gpu

CASES = [  # B, H, S, D, causal, axial grid, pos_offset
    (2, 4, 130, 64, True, None, 0),      # ragged last tile
    (2, 2, 64, 64, False, (8, 8), 0),    # axial tables, non-causal
    (1, 2, 200, 128, True, None, 3),     # head_dim 128, table rows from 3
    (2, 3, 77, 32, True, None, 0),       # head_dim 32
    (1, 2, 5, 64, True, None, 1),        # fewer rows than one tile
    (1, 3, 256, 64, True, None, 0),      # few items: the dK+dV query split
]


def _exact(x, dt):
    x = np.asarray(x, dtype=np.float32)
    if dt == "bf16":
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    return x


def _dev(x, dt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _tables(rows, D, axial):
    import torch
    if axial:
        ang = oracle.rope_angles_axial(*axial, D)
        ang = np.concatenate([ang, ang[: max(0, rows - len(ang))]])[:rows]
    else:
        ang = oracle.rope_angles_1d(np.arange(rows), D)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    return c, s, torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()


def _views(pk, dpk, o_s, dOt, H, S):
    """[B,H,S,D] views of the packed projection, its gradient, O and dO."""
    q, k, v = (pk[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    dq, dk, dv = (dpk[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    return q, k, v, dq, dk, dv, o_s.permute(0, 2, 1, 3), dOt.permute(0, 2, 1, 3)


@pytest.mark.parametrize("ws_mode", ["full", "min"])
@pytest.mark.parametrize("mode", ["f32", "bf16", "f32_bf16fwd"])
@pytest.mark.parametrize("B,H,S,D,causal,axial,pos", CASES)
def test_fused_rope_step(B, H, S, D, causal, axial, pos, mode, ws_mode):
    import torch
    dt = "bf16" if mode == "bf16" else "f32"
    fast = mode == "f32_bf16fwd"
    note(f"[gpu case] fused RoPE B{B} H{H} S{S} D{D} causal={causal} axial={axial} pos={pos} "
         f"mode={mode} ws={ws_mode} -> attn_fwd_rope, attn_bwd_rope")
    rng = np.random.default_rng(1000 * S + D)
    packed = _exact(rng.standard_normal((B, S, 3, H, D)), dt)
    dO = _exact(rng.standard_normal((B, S, H, D)), dt)
    c, s, ct, st = _tables(S + pos, D, axial)
    scale = 1.0 / np.sqrt(D)
    pk, dOt = _dev(packed, dt), _dev(dO, dt)
    tdt = pk.dtype
    shp = (B, H, S, D)
    nan = float("nan")
    o_s = torch.full((B, S, H, D), nan, dtype=tdt, device="cuda")
    dpk = torch.full_like(pk, nan)
    q, k, v, dq, dk, dv, o, do = _views(pk, dpk, o_s, dOt, H, S)
    qk = torch.full((2,) + shp, nan, dtype=tdt, device="cuda")
    lse = torch.full((B, H, S), nan, device="cuda")
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.full((workspace_bytes(ws_mode, code, shp, causal) // 4,), nan, device="cuda")
    afb.attn_fwd_rope(q, k, v, o, lse, qk, ct, st, causal, scale, pos_offset=pos,
                      bf16_operands=fast)
    afb.attn_bwd_rope(qk, v, o, do, lse, dq, dk, dv, ws, ct, st, causal, scale, pos_offset=pos)
    # the separate-pass path on the same inputs
    offs, pst = afb.packed_qkv(H, S, D)
    bhsd = afb.strides_bhsd(H, S, D)
    q2, k2 = (torch.full(shp, nan, dtype=tdt, device="cuda") for _ in range(2))
    afb.attn_rope_copy(pk, offs[0], pst, q2, 0, bhsd, shp, ct, st, pos_offset=pos)
    afb.attn_rope_copy(pk, offs[1], pst, k2, 0, bhsd, shp, ct, st, pos_offset=pos)
    o2 = torch.full(shp, nan, dtype=tdt, device="cuda")
    lse2 = torch.full((B, H, S), nan, device="cuda")
    afb.attn_fwd_strided(q2, k2, v, o2, lse2, None, causal, scale, bf16_operands=fast)
    dq2, dk2, dv2 = (torch.full(shp, nan, dtype=tdt, device="cuda") for _ in range(3))
    ws2 = torch.empty(afb.attn_bwd_cross_workspace_size(code, B, H, S, S, D, causal),
                      dtype=torch.uint8, device="cuda")
    afb.attn_bwd_strided(q2, k2, v, o2, do, lse2, dq2, dk2, dv2, ws2, None, causal, scale)
    g = torch.full((2,) + shp, nan, dtype=tdt, device="cuda")
    afb.attn_rope_copy(dq2, 0, bhsd, g[0], 0, bhsd, shp, ct, st, pos_offset=pos, transpose=True)
    afb.attn_rope_copy(dk2, 0, bhsd, g[1], 0, bhsd, shp, ct, st, pos_offset=pos, transpose=True)
    torch.cuda.synchronize()

    h = {n: to_host(t) for n, t in (("qk", qk), ("o", o), ("lse", lse), ("dq", dq), ("dk", dk),
                                    ("dv", dv), ("q2", q2), ("k2", k2), ("o2", o2),
                                    ("lse2", lse2), ("g", g), ("dv2", dv2))}
    for n, x in h.items():
        assert np.all(np.isfinite(x)), f"{n}: unwritten or non-finite values"
    # turned Q and K: the same rounding as the rotation pass
    assert np.array_equal(h["qk"][0], h["q2"]), "turned Q differs from attn_rope_copy"
    assert np.array_equal(h["qk"][1], h["k2"]), "turned K differs from attn_rope_copy"
    # oracle: turn, attend, turn the gradients back
    qo, ko, vo = (oracle.gather_rows(packed, offs[i], pst, shp).astype(np.float64)
                  for i in range(3))
    rq, rk = oracle.rope(qo, c, s, pos), oracle.rope(ko, c, s, pos)
    if fast:  # the practical contract's forward operands: turned, rounded to bf16
        rq, rk, vf = (_exact(x, "bf16").astype(np.float64) for x in (h["q2"], h["k2"], vo))
    else:
        vf = vo
    ro, rl = oracle.attention_forward(rq, rk, vf, causal, scale)
    tol = TOL["bf16" if mode != "f32" else "f32"]
    errs = {"o": max_rel_err(h["o"], ro), "lse": max_rel_err(h["lse"], rl)}
    if not fast:
        rdq, rdk, rdv, _ = oracle.attention_backward(rq, rk, vo, dO.transpose(0, 2, 1, 3)
                                                     .astype(np.float64), causal, scale)
        errs["dq"] = max_rel_err(h["dq"], oracle.rope_transpose(rdq, c, s, pos))
        errs["dk"] = max_rel_err(h["dk"], oracle.rope_transpose(rdk, c, s, pos))
        errs["dv"] = max_rel_err(h["dv"], rdv)
    # the separate-pass path computes the same step (rounding order aside)
    errs["o_vs_passes"] = max_rel_err(h["o"], h["o2"])
    errs["dq_vs_passes"] = max_rel_err(h["dq"], h["g"][0])
    errs["dk_vs_passes"] = max_rel_err(h["dk"], h["g"][1])
    errs["dv_vs_passes"] = max_rel_err(h["dv"], h["dv2"])
    note("  errors " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= tol, (k_, v_)


def test_fused_rope_repeatable():
    """Two calls on the same inputs give the same bits (fixed sum orders)."""
    import torch
    B, H, S, D = 2, 4, 130, 64
    note(f"[gpu case] fused RoPE repeatability B{B} H{H} S{S} D{D}")
    rng = np.random.default_rng(7)
    pk = _dev(rng.standard_normal((B, S, 3, H, D)), "f32")
    dOt = _dev(rng.standard_normal((B, S, H, D)), "f32")
    c, s, ct, st = _tables(S, D, None)
    outs = []
    for _ in range(2):
        o_s = torch.empty((B, S, H, D), device="cuda")
        dpk = torch.empty_like(pk)
        q, k, v, dq, dk, dv, o, do = _views(pk, dpk, o_s, dOt, H, S)
        qk = torch.empty((2, B, H, S, D), device="cuda")
        lse = torch.empty((B, H, S), device="cuda")
        ws = torch.empty(afb.attn_bwd_workspace_size(afb.ATTN_F32, B, H, S, D, True),
                         dtype=torch.uint8, device="cuda")
        afb.attn_fwd_rope(q, k, v, o, lse, qk, ct, st, True, 0.125)
        afb.attn_bwd_rope(qk, v, o, do, lse, dq, dk, dv, ws, ct, st, True, 0.125)
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in (o_s, lse, dpk, qk)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fused_rope_separate_bshd_tensors(dt):
    """Q, K, V, O, dO and the gradients as separate [B, S, H, D] tensors
    (row stride H*D), a sequence that is not a multiple of the tile, and a
    table offset: the fused step against the oracle."""
    import torch
    B, H, S, D, causal, pos = 2, 3, 150, 64, True, 7
    note(f"[gpu case] fused RoPE [B,S,H,D] tensors B{B} H{H} S{S} D{D} pos={pos} dtype={dt}")
    rng = np.random.default_rng(11)
    x = {n: _exact(rng.standard_normal((B, S, H, D)), dt) for n in ("q", "k", "v", "do")}
    c, s, ct, st = _tables(S + pos, D, None)
    scale = 1.0 / np.sqrt(D)
    dev = {n: _dev(v, dt) for n, v in x.items()}
    view = lambda t: t.permute(0, 2, 1, 3)
    tdt = dev["q"].dtype
    nan = float("nan")
    o_s, dq_s, dk_s, dv_s = (torch.full((B, S, H, D), nan, dtype=tdt, device="cuda")
                             for _ in range(4))
    qk = torch.full((2, B, H, S, D), nan, dtype=tdt, device="cuda")
    lse = torch.full((B, H, S), nan, device="cuda")
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.empty(afb.attn_bwd_workspace_size(code, B, H, S, D, causal), dtype=torch.uint8,
                     device="cuda")
    afb.attn_fwd_rope(view(dev["q"]), view(dev["k"]), view(dev["v"]), view(o_s), lse, qk, ct, st,
                      causal, scale, pos_offset=pos)
    afb.attn_bwd_rope(qk, view(dev["v"]), view(o_s), view(dev["do"]), lse, view(dq_s),
                      view(dk_s), view(dv_s), ws, ct, st, causal, scale, pos_offset=pos)
    torch.cuda.synchronize()
    t = {n: x[n].transpose(0, 2, 1, 3).astype(np.float64) for n in x}
    rq, rk = oracle.rope(t["q"], c, s, pos), oracle.rope(t["k"], c, s, pos)
    ro, rl = oracle.attention_forward(rq, rk, t["v"], causal, scale)
    rdq, rdk, rdv, _ = oracle.attention_backward(rq, rk, t["v"], t["do"], causal, scale)
    got = {n: to_host(v).transpose(0, 2, 1, 3) for n, v in (("o", o_s), ("dq", dq_s),
                                                           ("dk", dk_s), ("dv", dv_s))}
    errs = {"o": max_rel_err(got["o"], ro), "lse": max_rel_err(to_host(lse), rl),
            "dq": max_rel_err(got["dq"], oracle.rope_transpose(rdq, c, s, pos)),
            "dk": max_rel_err(got["dk"], oracle.rope_transpose(rdk, c, s, pos)),
            "dv": max_rel_err(got["dv"], rdv)}
    note("  errors " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[dt], (k_, v_)


def test_fused_rope_forward_shared_kv_head():
    """Multi-query attention in the fused forward: one K, V head (head stride
    0) read by every query head; each head's turned K copy is stored for it."""
    import torch
    B, H, S, D, causal = 1, 4, 96, 64, True
    note(f"[gpu case] fused RoPE forward, shared K/V head B{B} H{H} S{S} D{D}")
    rng = np.random.default_rng(12)
    q = rng.standard_normal((B, H, S, D)).astype(np.float32)
    k1 = rng.standard_normal((B, 1, S, D)).astype(np.float32)
    v1 = rng.standard_normal((B, 1, S, D)).astype(np.float32)
    c, s, ct, st = _tables(S, D, None)
    qd = _dev(q, "f32")
    kd, vd = _dev(k1, "f32").expand(B, H, S, D), _dev(v1, "f32").expand(B, H, S, D)
    o = torch.full((B, H, S, D), float("nan"), device="cuda")
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    qk = torch.full((2, B, H, S, D), float("nan"), device="cuda")
    afb.attn_fwd_rope(qd, kd, vd, o, lse, qk, ct, st, causal, 0.125)
    torch.cuda.synchronize()
    kx = np.broadcast_to(k1, (B, H, S, D)).astype(np.float64)
    vx = np.broadcast_to(v1, (B, H, S, D)).astype(np.float64)
    rq, rk = oracle.rope(q.astype(np.float64), c, s), oracle.rope(kx, c, s)
    ro, rl = oracle.attention_forward(rq, rk, vx, causal, 0.125)
    assert max_rel_err(to_host(o), ro) <= TOL["f32"]
    assert max_rel_err(to_host(lse), rl) <= TOL["f32"]
    assert max_rel_err(to_host(qk[1]), rk) <= 1e-6
