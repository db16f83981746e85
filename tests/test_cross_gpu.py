"""GPU parity of cross-attention and padded keys (attn_fwd_cross /
attn_bwd_cross) against the float64 oracle: separate query and key lengths,
per-batch valid key counts, the causal diagonal at the end of the valid keys,
rows with no visible key (O = 0, LSE = -inf, no gradient).  Padded K and V
rows hold NaN on the device, so reading one would show in every output."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_device, to_host

pytestmark = pytest.mark.gpu

# (name, B, H, Sq, Sk, D, causal, kv_len or None)
CASES = [
    ("text_cross_77", 2, 8, 256, 77, 64, False, None),
    ("text_cross_77_padded", 2, 8, 256, 77, 64, False, [77, 50]),
    ("one_token_decode", 4, 8, 1, 512, 64, True, [512, 300, 1, 0]),
    ("more_queries_than_keys", 2, 4, 200, 130, 64, True, [130, 97]),
    ("chunked_prefill_d128", 2, 4, 96, 300, 128, True, [300, 250]),
    ("padded_self_d32", 3, 4, 197, 197, 32, True, [197, 120, 64]),
    # few-query heads (the VALU forward for Sq <= 16): rows with no visible
    # key (L = 3 < Sq = 5), every head_dim, one and sixteen queries
    ("few_queries_causal", 2, 4, 5, 300, 64, True, [300, 3]),
    ("sixteen_queries_d128", 2, 4, 16, 1000, 128, False, [1000, 777]),
    ("decode_d32_long", 3, 4, 1, 2000, 32, True, [2000, 1, 1500]),
    ("decode_d128_ragged", 2, 3, 1, 333, 128, False, None),
    ("three_queries_d32", 2, 3, 3, 70, 32, True, None),
    # many queries over few keys: the dK+dV pass splits the queries into
    # chunks and adds their partial sums (with causal rows that see nothing)
    ("long_queries_77", 1, 2, 2048, 77, 64, False, None),
    ("long_queries_causal_split", 1, 2, 1024, 200, 64, True, [150]),
    ("long_queries_d128_padded", 2, 1, 1536, 100, 128, False, [100, 61]),
]


def _ds_bytes(B, H, Sq, Sk, dt):
    """dS^T of the dS path: [B*H][ceil(Sk/128)*128][ceil(Sq/128)*128]."""
    r = lambda n: (n + 127) // 128 * 128
    b = B * H * r(Sk) * r(Sq) * (2 if dt == "bf16" else 4)
    return (b + 255) // 256 * 256


def _ws_bytes(mode, code, dt, B, H, Sq, Sk, D, causal):
    """Workspace for a mode: full (recommended), min, or split (the minimum
    and the dK, dV partials, no dS^T: the query split with dQ recomputed)."""
    rec = afb.attn_bwd_cross_workspace_size(code, B, H, Sq, Sk, D, causal)
    mn = afb.attn_bwd_cross_workspace_size_min(code, B, H, Sq, Sk, D, causal)
    if mode == "full":
        return rec
    if mode == "min":
        return mn
    return mn + (rec - mn - _ds_bytes(B, H, Sq, Sk, dt))


def _inputs(B, H, Sq, Sk, D, dt, seed=0):
    return synth.cross_inputs((B, H, Sq, D), (B, H, Sk, D), seed, dt)


def _err_lse(got, ref):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "rows without keys"
    return max_rel_err(got[fin], ref[fin]) if fin.any() else 0.0


@pytest.mark.parametrize("ws", ["full", "min", "split"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name,B,H,Sq,Sk,D,causal,kvl", CASES)
def test_cross_parity(name, B, H, Sq, Sk, D, causal, kvl, dt, ws):
    import torch
    note(f"[gpu case] cross {name} B{B} H{H} Sq{Sq} Sk{Sk} D{D} causal={causal} kv_len={kvl} "
         f"dtype={dt} workspace={ws} -> attn_fwd_cross + attn_bwd_cross")
    inp = _inputs(B, H, Sq, Sk, D, dt)
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("q", "k", "v", "do")}
    kv_len = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device="cuda")
    if kvl is not None:  # padded rows are never read: poison them
        for b, L in enumerate(kvl):
            dev["k"][b, :, L:] = float("nan")
            dev["v"][b, :, L:] = float("nan")
    tdt = dev["q"].dtype
    nan = float("nan")
    o = torch.full((B, H, Sq, D), nan, dtype=tdt, device="cuda")
    lse = torch.full((B, H, Sq), nan, device="cuda")
    dq = torch.full((B, H, Sq, D), nan, dtype=tdt, device="cuda")
    dk = torch.full((B, H, Sk, D), nan, dtype=tdt, device="cuda")
    dv = torch.full((B, H, Sk, D), nan, dtype=tdt, device="cuda")
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    wsb = torch.full((_ws_bytes(ws, code, dt, B, H, Sq, Sk, D, causal) // 4,), nan, device="cuda")
    scale = 1.0 / np.sqrt(D)
    afb.attn_fwd_cross(dev["q"], dev["k"], dev["v"], o, lse, kv_len, causal, scale)
    afb.attn_bwd_cross(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, wsb, kv_len,
                       causal, scale)
    torch.cuda.synchronize()
    host = {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    kvn = None if kvl is None else np.array(kvl)
    ro, rl = oracle.attention_forward(inp["q"], inp["k"], inp["v"], causal, scale, kvn)
    rdq, rdk, rdv, _ = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal,
                                                 scale, kvn)
    errs = {"o": max_rel_err(host["o"], ro), "lse": _err_lse(host["lse"], rl),
            "dq": max_rel_err(host["dq"], rdq), "dk": max_rel_err(host["dk"], rdk),
            "dv": max_rel_err(host["dv"], rdv)}
    note(f"  errors {name} {dt} {ws}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL[dt], (k_, v_)
    if kvl is not None:  # gradients of padded keys are exact zeros
        for b, L in enumerate(kvl):
            assert not host["dk"][b, :, L:].any() and not host["dv"][b, :, L:].any()
    empty = np.isneginf(rl)
    assert not host["o"][empty].any() and not host["dq"][empty].any()


def test_cross_equal_lengths_match_self_attention():
    """attn_fwd_cross / attn_bwd_cross with Sq = Sk and no kv_len give exactly
    what attn_fwd / attn_bwd give (the same kernels)."""
    import torch
    B, H, S, D = 2, 3, 130, 64
    note(f"[gpu case] cross vs self B{B} H{H} S{S} D{D}")
    inp = synth.make_inputs((B, H, S, D), 5, "f32")
    dev = {n: to_device(inp[n], None, "f32") for n in ("q", "k", "v", "do")}
    outs = []
    for cross in (False, True):
        o = torch.empty_like(dev["q"]); lse = torch.empty((B, H, S), device="cuda")
        g = [torch.empty_like(dev["q"]) for _ in range(3)]
        ws = torch.empty(afb.attn_bwd_workspace_size(0, B, H, S, D, True), dtype=torch.uint8,
                         device="cuda")
        if cross:
            afb.attn_fwd_cross(dev["q"], dev["k"], dev["v"], o, lse, None, True, 0.125)
            afb.attn_bwd_cross(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *g, ws, None,
                               True, 0.125)
        else:
            afb.attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, True, 0.125)
            afb.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *g, ws, True, 0.125)
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in (o, lse, *g)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("Sq,Sk,D,causal,kvl", [(1, 512, 64, True, [512, 200]),
                                               (5, 300, 128, True, [300, 4]),
                                               (16, 257, 32, False, None)])
def test_few_query_practical_contract(Sq, Sk, D, causal, kvl):
    """The practical contract (float32 tensors, bf16-rounded forward
    operands) on the few-query forward: against the oracle on the rounded
    operands at the reduced-precision gate, and visibly different from the
    strict forward."""
    import torch
    B, H = 2, 3
    note(f"[gpu case] few-query practical B{B} H{H} Sq{Sq} Sk{Sk} D{D} causal={causal} "
         f"kv_len={kvl} -> attn_fwd_cross(bf16_operands)")
    inp = _inputs(B, H, Sq, Sk, D, "f32", seed=4)
    rnd = _inputs(B, H, Sq, Sk, D, "bf16", seed=4)
    dev = {n: to_device(inp[n], None, "f32") for n in ("q", "k", "v")}
    kv_len = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device="cuda")
    o = torch.full((B, H, Sq, D), float("nan"), device="cuda")
    o_s = torch.full((B, H, Sq, D), float("nan"), device="cuda")
    lse = torch.full((B, H, Sq), float("nan"), device="cuda")
    scale = 1.0 / np.sqrt(D)
    afb.attn_fwd_cross(dev["q"], dev["k"], dev["v"], o, lse, kv_len, causal, scale,
                       bf16_operands=True)
    afb.attn_fwd_cross(dev["q"], dev["k"], dev["v"], o_s, None, kv_len, causal, scale)
    torch.cuda.synchronize()
    kvn = None if kvl is None else np.array(kvl)
    o_r, lse_r = oracle.attention_forward(rnd["q"], rnd["k"], rnd["v"], causal, scale, kvn)
    o_f, _ = oracle.attention_forward(inp["q"], inp["k"], inp["v"], causal, scale, kvn)
    ho, hl, hs = to_host(o), to_host(lse), to_host(o_s)
    e = {"o": max_rel_err(ho, o_r), "lse": _err_lse(hl, lse_r), "o_strict": max_rel_err(hs, o_f)}
    diff = np.abs(ho - hs).max() / np.abs(hs).max()
    note("  errors " + ", ".join(f"{k}={v:.2e}" for k, v in e.items()) + f"; |O - O_strict| {diff:.2e}")
    assert e["o"] <= TOL["bf16"] and e["lse"] <= TOL["bf16"] and e["o_strict"] <= TOL["f32"]
    assert diff > TOL["f32"], diff


def test_query_split_deterministic():
    """The split dK+dV pass (partials added in a fixed order) gives bitwise
    the same gradients on every run."""
    import torch
    B, H, Sq, Sk, D = 1, 2, 2048, 77, 64
    note(f"[gpu case] query split determinism B{B} H{H} Sq{Sq} Sk{Sk} D{D}")
    inp = _inputs(B, H, Sq, Sk, D, "f32", seed=2)
    dev = {n: to_device(inp[n], None, "f32") for n in ("q", "k", "v", "do")}
    ws = torch.empty(afb.attn_bwd_cross_workspace_size(0, B, H, Sq, Sk, D, False),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dev["q"])
    lse = torch.empty((B, H, Sq), device="cuda")
    afb.attn_fwd_cross(dev["q"], dev["k"], dev["v"], o, lse, None, False, 0.125)
    runs = []
    for _ in range(3):
        g = [torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])]
        afb.attn_bwd_cross(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *g, ws, None, False,
                           0.125)
        torch.cuda.synchronize()
        runs.append([to_host(t) for t in g])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert np.array_equal(a, b)
