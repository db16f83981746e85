"""GPU parity of the pages' practical contract ("Meganeura", Section 4.2:
eligible forward matrix and attention inputs rounded locally to reduced
precision, f32 accumulation and stores, the backward kept f32), here
ATTN_F32_BF16FWD: float32 tensors, the forward's MFMA operands rounded to
bf16 inside the kernel, the strict-f32 backward fed that forward's O and
LSE; and of the inference-only forward (no LSE stored)."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, oracle_all, to_device, to_host

pytestmark = pytest.mark.gpu


def _run_practical(shape, seed, causal, scale, sigma_qkv, sigma_do, ws_mode):
    import torch
    B, H, S, D = shape
    inp = synth.make_inputs(shape, seed, "f32", sigma_qkv, sigma_do)
    dev = {n: to_device(inp[n], None, "f32") for n in ("q", "k", "v", "do")}
    nan = float("nan")
    o = torch.full((B, H, S, D), nan, device="cuda")
    o_strict = torch.full((B, H, S, D), nan, device="cuda")
    lse = torch.full((B, H, S), nan, device="cuda")
    lse_strict = torch.full((B, H, S), nan, device="cuda")
    dq, dk, dv = (torch.full((B, H, S, D), nan, device="cuda") for _ in range(3))
    wsf = afb.attn_bwd_workspace_size if ws_mode == "full" else afb.attn_bwd_workspace_size_min
    ws = torch.empty(wsf(afb.ATTN_F32_BF16FWD, B, H, S, D, causal), dtype=torch.uint8, device="cuda")
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, causal, scale, bf16_operands=True)
    afb.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, ws, causal, scale)
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o_strict, lse_strict, causal, scale)
    torch.cuda.synchronize()
    host = {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv),
                                         ("o_strict", o_strict))}
    return inp, host


@pytest.mark.parametrize("ws", ["full", "min"])
@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_practical_contract(name, ws):
    cfg = synth.CONFIGS[name]
    note(f"[gpu case] practical contract {name} shape={cfg.shape} seed=0 workspace={ws} "
         "-> attn_fwd(ATTN_F32_BF16FWD) + attn_bwd(f32)")
    inp, host = _run_practical(cfg.shape, 0, cfg.causal, cfg.scale, cfg.sigma_qkv, cfg.sigma_do, ws)
    # The forward against the oracle on the operands it multiplies: the same
    # seeded values rounded to bf16 (only P's rounding remains).
    rnd = synth.make_inputs(cfg.shape, 0, "bf16", cfg.sigma_qkv, cfg.sigma_do)
    o_r, lse_r = oracle.attention_forward(*(rnd[n].astype(np.float64) for n in ("q", "k", "v")),
                                          cfg.causal, cfg.scale)
    e_fwd = {"o": max_rel_err(host["o"], o_r), "lse": max_rel_err(host["lse"], lse_r)}
    # The whole step against the oracle on the float32 inputs, at the
    # reduced-precision gate.
    ref = oracle_all(inp, cfg.causal, cfg.scale)
    e_all = {n: max_rel_err(host[n], ref[n]) for n in ("o", "lse", "dq", "dk", "dv")}
    # The operands really are rounded: the result differs from the strict
    # forward's by more than the strict gate.
    diff = max_rel_err(host["o"], host["o_strict"])
    note(f"  practical {name} ws {ws}: fwd vs rounded-input oracle " +
         ", ".join(f"{k}={v:.2e}" for k, v in e_fwd.items()) + "; step vs f32 oracle " +
         ", ".join(f"{k}={v:.2e}" for k, v in e_all.items()) + f"; |O - O_strict| {diff:.2e}")
    for k, v in {**e_fwd, **e_all}.items():
        assert v <= TOL["bf16"], (k, v)
    assert diff > TOL["f32"], diff


@pytest.mark.parametrize("mode", ["f32", "bf16", "f32_bf16fwd"])
@pytest.mark.parametrize("S,D,causal", [(197, 64, False), (130, 128, True), (64, 32, True),
                                        (512, 64, True), (1, 64, True), (16, 128, False)])
def test_forward_without_lse(mode, S, D, causal):
    """lse = NULL stores no LSE and leaves O bit-identical."""
    import torch
    shape = (2, 3, S, D)
    note(f"[gpu case] forward without LSE mode={mode} shape={shape} causal={causal}")
    dt = "bf16" if mode == "bf16" else "f32"
    inp = synth.make_inputs(shape, 3, dt)
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("q", "k", "v")}
    o1 = torch.empty_like(dev["q"])
    o2 = torch.full_like(dev["q"], float("nan"))
    lse = torch.empty(shape[:3], device="cuda")
    scale = 1.0 / np.sqrt(D)
    fast = mode == "f32_bf16fwd"
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o1, lse, causal, scale, bf16_operands=fast)
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o2, None, causal, scale, bf16_operands=fast)
    torch.cuda.synchronize()
    a = o1.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    b = o2.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    assert np.array_equal(a, b)
