"""Run the HIP path and the float64 oracle on the same seeded inputs and
compare them.  Test infrastructure (imports the oracle)."""
from __future__ import annotations

import sys

import numpy as np

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str) -> None:
    """Name the case on the real stderr, flushed, before a GPU step."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def max_rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over one tensor (normwise-max)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def to_device(x_f32: np.ndarray, bits, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x_f32))
    return t.cuda()


def to_host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def workspace_bytes(ws_mode: str, code: int, shape, causal: bool) -> int:
    """Backward workspace for a mode: "full" the recommended size (dS^T, so dQ
    is a GEMM, plus the dK, dV partials of the query split where the shape
    takes it); "min" the minimum (dQ recomputes the scores, no split);
    "ds_only" the minimum plus dS^T; "split_only" the recommended size less
    dS^T (the query split with dQ recomputed)."""
    B, H, S, D = shape
    rec = afb.attn_bwd_workspace_size(code, B, H, S, D, causal)
    mn = afb.attn_bwd_workspace_size_min(code, B, H, S, D, causal)
    sp = (S + 127) // 128 * 128
    ds = (B * H * sp * sp * (2 if code == afb.ATTN_BF16 else 4) + 255) // 256 * 256
    return {"full": rec, "min": mn, "ds_only": mn + ds, "split_only": rec - ds}[ws_mode]


def gpu_fwd_bwd(inp: dict, shape, dtype: str, causal: bool, scale: float, guard: int = 0,
                fill=float("nan"), ws_mode: str = "full"):
    """Run attn_fwd then attn_bwd (fed the GPU's own O and LSE).

    Outputs are prefilled with `fill` so an unwritten element shows; with
    guard > 0 every output gets `guard` extra trailing elements that must stay
    untouched.  Returns host arrays and the device tensors.
    """
    import torch
    B, H, S, D = shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dtype) for n in ("q", "k", "v", "do")}

    def out(shape_, dt):
        n = int(np.prod(shape_))
        buf = torch.full((n + guard,), fill, dtype=dt, device="cuda")
        return buf, buf[:n].view(shape_)

    bufs = {}
    for name in ("o", "dq", "dk", "dv"):
        bufs[name] = out((B, H, S, D), tdt)
    bufs["lse"] = out((B, H, S), torch.float32)
    code = afb.ATTN_BF16 if dtype == "bf16" else afb.ATTN_F32
    ws_bytes = workspace_bytes(ws_mode, code, shape, causal)
    ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    t = {k_: v_[1] for k_, v_ in bufs.items()}
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], t["o"], t["lse"], causal, scale)
    afb.attn_bwd(dev["q"], dev["k"], dev["v"], t["o"], dev["do"], t["lse"],
                 t["dq"], t["dk"], t["dv"], ws, causal, scale)
    # The prep stage on its own (attn_bwd runs it, except where dK+dV forms D
    # itself: bf16 on the dS path), into a fresh minimum workspace: D and
    # LSE*log2(e) of every row.
    wsp = torch.full((workspace_bytes("min", code, shape, causal) // 4,), float("nan"),
                     dtype=torch.float32, device="cuda")
    afb.attn_bwd_prep(t["o"], dev["do"], t["lse"], wsp)
    torch.cuda.synchronize()
    host = {k_: to_host(v_) for k_, v_ in t.items()}
    host["delta"] = wsp[: B * H * S].cpu().numpy().reshape(B, H, S)
    host["lse2"] = wsp[B * H * S: 2 * B * H * S].cpu().numpy().reshape(B, H, S)
    if guard:
        for name, (buf, _) in bufs.items():
            tail = buf[buf.numel() - guard:].float().cpu().numpy()
            host[name + "_guard_ok"] = bool(np.all(np.isnan(tail))) if np.isnan(fill) \
                else bool(np.all(tail == fill))
    return host, dev, t


def oracle_all(inp: dict, causal: bool, scale: float) -> dict:
    q, k, v, do = (inp[n].astype(np.float64) for n in ("q", "k", "v", "do"))
    o, lse = oracle.attention_forward(q, k, v, causal, scale)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, causal, scale)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "delta": delta}


def compare(host: dict, ref: dict, names=("o", "lse", "dq", "dk", "dv")) -> dict:
    return {n: max_rel_err(host[n], ref[n]) for n in names}


def run_case(shape, seed: int, dtype: str, causal: bool, scale: float, sigma_qkv=1.0,
             sigma_do=1.0, guard: int = 0, ws_mode: str = "full"):
    note(f"[gpu case] shape={shape} seed={seed} dtype={dtype} causal={causal} "
         f"workspace={ws_mode} -> attn_fwd + attn_bwd")
    inp = synth.make_inputs(shape, seed, dtype, sigma_qkv, sigma_do)
    host, dev, outs = gpu_fwd_bwd(inp, shape, dtype, causal, scale, guard=guard, ws_mode=ws_mode)
    ref = oracle_all(inp, causal, scale)
    return compare(host, ref), host, ref, inp, dev, outs
