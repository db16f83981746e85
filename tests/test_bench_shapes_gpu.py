"""GPU parity at every shape the benchmark reports beyond the five workloads:
the long causal sequences (S = 2048 and 4096, head_dim 64 and 128), the
77-token text cross-attention at 4096 queries, the one-token decode cells,
and the ResNet-50 convolution layers at batch 32.  The HIP path runs the full
shape, in the launch configuration the benchmark times (recommended
workspace); the float64 oracle is evaluated on whole (batch, head) slices
where the full tensor would be too slow for it (every (b, h) slice of
attention is independent, so a slice of the GPU result must equal the
oracle on that slice).  Gates as everywhere: max |gpu - ref| / max |ref| per
output <= 1e-4 (strict f32), 2e-2 (bf16)."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_device, to_host

pytestmark = pytest.mark.gpu


def _slices(B, H):
    """(b, h) slices checked against the oracle: the first, the last and one
    in the middle."""
    picks = {(0, 0), (B - 1, H - 1), (B // 2, H // 2)}
    return sorted(picks)


def _self_attention_case(shape, dt, ws_mode, seed=0):
    import torch
    B, H, S, D = shape
    scale = 1.0 / np.sqrt(D)
    note(f"[gpu case] long sequence B{B} H{H} S{S} D{D} causal dtype={dt} workspace={ws_mode} "
         f"-> attn_fwd + attn_bwd")
    inp = synth.make_inputs(shape, seed, dt)
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("q", "k", "v", "do")}
    nan = float("nan")
    tdt = dev["q"].dtype
    o, dq, dk, dv = (torch.full(shape, nan, dtype=tdt, device="cuda") for _ in range(4))
    lse = torch.full((B, H, S), nan, device="cuda")
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    wsf = afb.attn_bwd_workspace_size if ws_mode == "full" else afb.attn_bwd_workspace_size_min
    ws = torch.full((wsf(code, B, H, S, D, True) // 4,), nan, device="cuda")
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, True, scale)
    afb.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, ws, True, scale)
    torch.cuda.synchronize()
    host = {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk),
                                       ("dv", dv))}
    for n, x in host.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values (unwritten or overflow)"
    worst = {}
    for b, h in _slices(B, H):
        x = {n: inp[n][b:b + 1, h:h + 1].astype(np.float64) for n in ("q", "k", "v", "do")}
        ro, rl = oracle.attention_forward(x["q"], x["k"], x["v"], True, scale)
        rdq, rdk, rdv, _ = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], True,
                                                     scale)
        for n, ref in (("o", ro), ("lse", rl), ("dq", rdq), ("dk", rdk), ("dv", rdv)):
            e = max_rel_err(host[n][b:b + 1, h:h + 1], ref)
            worst[n] = max(worst.get(n, 0.0), e)
    note(f"  errors B{B} H{H} S{S} D{D} {dt} {ws_mode}: " +
         ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    for n, e in worst.items():
        assert e <= TOL[dt], (n, e)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", synth.LONG_SEQ_SHAPES,
                         ids=[f"B{b}H{h}S{s}D{d}" for b, h, s, d in synth.LONG_SEQ_SHAPES])
def test_long_sequence_parity(shape, dt):
    """The benchmark's long-sequence shapes, full size, recommended workspace."""
    _self_attention_case(shape, dt, "full")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_long_sequence_minimum_workspace(dt):
    """The longest head_dim-128 shape on the minimum workspace (dQ recomputes
    the scores), the path a caller without room for the S x S workspace takes."""
    _self_attention_case(synth.LONG_SEQ_SHAPES[-1], dt, "min")


def _cross_case(wl, dt, seed=0):
    import torch
    B, H, Sq, Sk, D = wl.batch, wl.heads, wl.seq_q, wl.seq_k, wl.head_dim
    kvl = synth.key_lengths(seed, B, wl.min_keys, Sk) if wl.padded else None
    note(f"[gpu case] cross workload {wl.name} B{B} H{H} Sq{Sq} Sk{Sk} D{D} causal={wl.causal} "
         f"padded={wl.padded} dtype={dt} -> attn_fwd_cross + attn_bwd_cross")
    inp = synth.cross_inputs((B, H, Sq, D), (B, H, Sk, D), seed, dt)
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("q", "k", "v", "do")}
    kv_len = None if kvl is None else torch.tensor(kvl, dtype=torch.int32, device="cuda")
    if kvl is not None:  # padded rows are never read: poison them
        for b, L in enumerate(kvl):
            dev["k"][b, :, L:] = float("nan")
            dev["v"][b, :, L:] = float("nan")
    nan = float("nan")
    tdt = dev["q"].dtype
    o = torch.full((B, H, Sq, D), nan, dtype=tdt, device="cuda")
    lse = torch.full((B, H, Sq), nan, device="cuda")
    dq = torch.full((B, H, Sq, D), nan, dtype=tdt, device="cuda")
    dk = torch.full((B, H, Sk, D), nan, dtype=tdt, device="cuda")
    dv = torch.full((B, H, Sk, D), nan, dtype=tdt, device="cuda")
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    ws = torch.full((afb.attn_bwd_cross_workspace_size(code, B, H, Sq, Sk, D, wl.causal) // 4,),
                    nan, device="cuda")
    scale = 1.0 / np.sqrt(D)
    afb.attn_fwd_cross(dev["q"], dev["k"], dev["v"], o, lse, kv_len, wl.causal, scale)
    afb.attn_bwd_cross(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv, ws, kv_len,
                       wl.causal, scale)
    torch.cuda.synchronize()
    host = {n: to_host(t) for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk),
                                       ("dv", dv))}
    kvn = None if kvl is None else np.asarray(kvl)
    x = {n: inp[n].astype(np.float64) for n in ("q", "k", "v", "do")}
    ro, rl = oracle.attention_forward(x["q"], x["k"], x["v"], wl.causal, scale, kvn)
    rdq, rdk, rdv, _ = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], wl.causal,
                                                 scale, kvn)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(host["lse"]), np.isneginf(rl)), "rows without keys"
    errs = {"o": max_rel_err(host["o"], ro), "lse": max_rel_err(host["lse"][fin], rl[fin]),
            "dq": max_rel_err(host["dq"], rdq), "dk": max_rel_err(host["dk"], rdk),
            "dv": max_rel_err(host["dv"], rdv)}
    note(f"  errors {wl.name} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dt], (n, e)
    if kvl is not None:  # gradients of padded keys are exact zeros
        for b, L in enumerate(kvl):
            assert not host["dk"][b, :, L:].any() and not host["dv"][b, :, L:].any()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name", list(synth.CROSS_WORKLOADS))
def test_cross_workload_parity(name, dt):
    """The benchmark's cross-attention workloads at their full size: the
    77-token text cross-attention over 4096 queries, and the one-token decode
    with and without padded keys (the oracle takes every (b, h) slice)."""
    _cross_case(synth.CROSS_WORKLOADS[name], dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("layer", list(synth.CONV_LAYERS))
def test_conv_layer_parity(layer, dt):
    """The benchmark's ResNet-50 layers at batch 32: forward, data derivative
    (not for the stem, whose input is the image) and filter derivative,
    compared in full."""
    import torch
    N, H, W, C, K, R, S, st, pd = synth.CONV_LAYERS[layer]
    P, Q = oracle.out_size(H, W, R, S, st, pd)
    note(f"[gpu case] conv layer {layer} N{N} {H}x{W} C{C} K{K} {R}x{S} stride {st} pad {pd} "
         f"dtype={dt} -> conv2d_fwd, bwd_data, bwd_filter")
    inp = synth.conv_inputs((N, H, W, C), (K, R, S, C), (N, P, Q, K), 0, dt)
    x, w, dy = (to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("x", "w", "dy"))
    nan = float("nan")
    y = torch.full((N, P, Q, K), nan, dtype=x.dtype, device="cuda")
    dx = torch.full((N, H, W, C), nan, dtype=x.dtype, device="cuda")
    dw = torch.full((K, R, S, C), nan, dtype=x.dtype, device="cuda")
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    wsb = afb.conv2d_bwd_filter_workspace_size(code, (N, H, W, C), (K, R, S, C), st, pd)
    ws = torch.full((max(wsb, 4) // 4,), nan, device="cuda") if wsb else None
    has_dx = not layer.startswith("stem")
    afb.conv2d_fwd(x, w, y, st, pd)
    if has_dx:
        afb.conv2d_bwd_data(dy, w, dx, st, pd)
    afb.conv2d_bwd_filter(x, dy, dw, ws, st, pd)
    torch.cuda.synchronize()
    x64, w64, dy64 = (inp[n].astype(np.float64) for n in ("x", "w", "dy"))
    errs = {"y": max_rel_err(to_host(y), oracle.conv2d_forward(x64, w64, st, pd)),
            "dw": max_rel_err(to_host(dw),
                              oracle.conv2d_backward_filter(x64, dy64, w64.shape, st, pd))}
    if has_dx:
        errs["dx"] = max_rel_err(to_host(dx),
                                 oracle.conv2d_backward_data(dy64, w64, x64.shape, st, pd))
    note(f"  errors {layer} {dt}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dt], (n, e)
