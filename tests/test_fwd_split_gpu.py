"""GPU parity of the key-split forward (attn_fwd_ws with the workspace of
attn_fwd_workspace_size): shapes with few long heads, whose longest query
tiles are cut into key chunks merged afterwards.  Each case checks that the
split is taken (a non-zero workspace), compares O and LSE with the float64
oracle at the contract's gate, checks the unsplit forward agrees, and feeds
the split forward's O and LSE to the backward (whole-step parity).  Outputs
and workspace are NaN-prefilled."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [  # B, H, S, D, causal
    (1, 16, 1024, 128, True),   # the long-context workload
    (1, 8, 1000, 64, True),     # ragged last tile
    (1, 8, 1024, 64, False),    # non-causal long heads
    (1, 8, 1500, 32, True),     # head_dim 32, ragged
]


def _slices(B, H):
    return sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})


@pytest.mark.parametrize("mode", ["f32", "bf16", "f32_bf16fwd"])
@pytest.mark.parametrize("B,H,S,D,causal", CASES)
def test_key_split_forward(B, H, S, D, causal, mode):
    import torch
    dt = "bf16" if mode == "bf16" else "f32"
    shape = (B, H, S, D)
    scale = 1.0 / np.sqrt(D)
    code = {"f32": afb.ATTN_F32, "bf16": afb.ATTN_BF16, "f32_bf16fwd": afb.ATTN_F32_BF16FWD}[mode]
    nbytes = afb.attn_fwd_workspace_size(code, B, H, S, D, causal)
    assert nbytes > 0, "the key split should apply to this shape"
    note(f"[gpu case] key-split forward B{B} H{H} S{S} D{D} causal={causal} mode={mode} "
         f"workspace={nbytes} -> attn_fwd_ws, attn_fwd, attn_bwd")
    inp = synth.make_inputs(shape, 3, dt)
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("q", "k", "v", "do")}
    nan = float("nan")
    tdt = dev["q"].dtype
    ws = torch.full((nbytes // 4,), nan, device="cuda")
    o = torch.full(shape, nan, dtype=tdt, device="cuda")
    lse = torch.full((B, H, S), nan, device="cuda")
    o_plain = torch.full(shape, nan, dtype=tdt, device="cuda")
    lse_plain = torch.full((B, H, S), nan, device="cuda")
    o_nolse = torch.full(shape, nan, dtype=tdt, device="cuda")
    fast = mode == "f32_bf16fwd"
    afb.attn_fwd_ws(dev["q"], dev["k"], dev["v"], o, lse, ws, causal, scale, bf16_operands=fast)
    afb.attn_fwd_ws(dev["q"], dev["k"], dev["v"], o_nolse, None, ws, causal, scale,
                    bf16_operands=fast)
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o_plain, lse_plain, causal, scale,
                 bf16_operands=fast)
    dq, dk, dv = (torch.full(shape, nan, dtype=tdt, device="cuda") for _ in range(3))
    wsb = torch.full((afb.attn_bwd_workspace_size(code, B, H, S, D, causal) // 4,), nan,
                     device="cuda")
    afb.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, wsb, causal, scale)
    torch.cuda.synchronize()
    h = {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("o_plain", o_plain),
                                    ("lse_plain", lse_plain), ("o_nolse", o_nolse), ("dq", dq),
                                    ("dk", dk), ("dv", dv))}
    for n, x in h.items():
        assert np.all(np.isfinite(x)), f"{n}: unwritten or non-finite values"
    # the inference-only call stores the same O
    assert np.array_equal(h["o"], h["o_nolse"])
    # split and unsplit forwards differ only in the order chunks are summed
    tol = TOL["bf16" if mode != "f32" else "f32"]
    assert max_rel_err(h["o"], h["o_plain"]) <= tol
    assert max_rel_err(h["lse"], h["lse_plain"]) <= tol
    rnd = synth.make_inputs(shape, 3, "bf16") if fast else inp  # operands the contract uses
    worst = {}
    for b, hh in _slices(B, H):
        x = {n: rnd[n][b:b + 1, hh:hh + 1].astype(np.float64) for n in ("q", "k", "v")}
        ro, rl = oracle.attention_forward(x["q"], x["k"], x["v"], causal, scale)
        worst["o"] = max(worst.get("o", 0.0), max_rel_err(h["o"][b:b + 1, hh:hh + 1], ro))
        worst["lse"] = max(worst.get("lse", 0.0), max_rel_err(h["lse"][b:b + 1, hh:hh + 1], rl))
        if not fast:  # whole step against the oracle (the practical contract's
            # backward is strict f32 on the bf16-rounded forward: covered elsewhere)
            xd = {n: inp[n][b:b + 1, hh:hh + 1].astype(np.float64) for n in ("q", "k", "v", "do")}
            rdq, rdk, rdv, _ = oracle.attention_backward(xd["q"], xd["k"], xd["v"], xd["do"],
                                                         causal, scale)
            for n, ref in (("dq", rdq), ("dk", rdk), ("dv", rdv)):
                worst[n] = max(worst.get(n, 0.0), max_rel_err(h[n][b:b + 1, hh:hh + 1], ref))
    note("  errors " + ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for n, e in worst.items():
        assert e <= tol, (n, e)


def test_key_split_deterministic():
    """The chunk merge adds in a fixed order: repeated calls are bitwise equal."""
    import torch
    B, H, S, D = 1, 16, 1024, 128
    note(f"[gpu case] key-split determinism B{B} H{H} S{S} D{D}")
    inp = synth.make_inputs((B, H, S, D), 4, "f32")
    dev = {n: to_device(inp[n], None, "f32") for n in ("q", "k", "v")}
    ws = torch.empty(afb.attn_fwd_workspace_size(afb.ATTN_F32, B, H, S, D, True),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        o = torch.empty((B, H, S, D), device="cuda")
        lse = torch.empty((B, H, S), device="cuda")
        afb.attn_fwd_ws(dev["q"], dev["k"], dev["v"], o, lse, ws, True, 0.125)
        torch.cuda.synchronize()
        outs.append((to_host(o), to_host(lse)))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
