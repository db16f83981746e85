"""GPU parity: the HIP path against the float64 oracle, element by element, on
the same seeded inputs.  Gate per output tensor X in {O, LSE, dQ, dK, dV}:
max|X_gpu - X_ref| / max|X_ref| <= 1e-4 (strict f32) or 2e-2 (bf16).  The
backward is fed the GPU forward's own O and LSE (the pipeline is gated)."""
import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
from parity_util import TOL, compare, gpu_fwd_bwd, max_rel_err, note, run_case, workspace_bytes

pytestmark = pytest.mark.gpu

CFG_CASES = [(name, dt, seed, ws) for name in synth.CONFIGS for dt in ("f32", "bf16")
             for seed in (0, 1, 2) for ws in ("full", "min")]


@pytest.mark.parametrize("name,dtype,seed,ws", CFG_CASES)
def test_config_parity(name, dtype, seed, ws):
    """The five measured workloads at full size, three seeds, both contracts,
    both backward paths (dS + GEMM with the recommended workspace; recompute
    with the minimum one)."""
    cfg = synth.CONFIGS[name]
    errs, host, ref, *_ = run_case(cfg.shape, seed, dtype, cfg.causal, cfg.scale,
                                   cfg.sigma_qkv, cfg.sigma_do, ws_mode=ws)
    note(f"  errors {name} {dtype} seed {seed} ws {ws}: " +
         ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[dtype], (k, v)
    # D and LSE*log2(e) as the prep stage writes them to the workspace
    assert max_rel_err(host["delta"], ref["delta"]) <= TOL[dtype]
    assert max_rel_err(host["lse2"], ref["lse"] * np.log2(np.e)) <= TOL[dtype]


MICRO = [(S, D, causal) for S in (1, 5, 16, 17, 33, 67, 130, 197) for D in (32, 64, 128)
         for causal in (True, False)]


@pytest.mark.parametrize("ws", ["full", "min"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,D,causal", MICRO)
def test_ragged_micro_shapes(S, D, causal, dtype, ws):
    """Sequence lengths that end mid-tile, every head_dim, guard bands after
    every output, NaN-prefilled outputs and workspace, both backward paths."""
    shape = (2, 3, S, D)
    scale = 1.0 / np.sqrt(D)
    errs, host, ref, inp, *_ = run_case(shape, 7, dtype, causal, scale, guard=64, ws_mode=ws)
    if S == 1:
        # One key: P = 1, so O = V and dV = dO, while dQ and dK are exactly 0
        # (dS = P (dP - D) with dP = D); the oracle's float64 dQ, dK are
        # rounding noise there, so the relative metric does not apply.
        # Bound |dQ|, |dK| by the rounding of dP - D instead.
        q, k, v, do = (inp[n].astype(np.float64) for n in ("q", "k", "v", "do"))
        bound = TOL[dtype] * scale * D * np.abs(do).max() * np.abs(v).max() \
            * max(np.abs(k).max(), np.abs(q).max())
        assert np.abs(host["dq"]).max() <= bound and np.abs(host["dk"]).max() <= bound
        errs = {n: errs[n] for n in ("o", "lse", "dv")}
    for k_, v_ in errs.items():
        assert v_ <= TOL[dtype], (k_, v_)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert host[name + "_guard_ok"], name


@pytest.mark.parametrize("ws", ["full", "min"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic_and_inputs_untouched(dtype, ws):
    import torch
    shape = (2, 4, 197, 64)
    inp = synth.make_inputs(shape, 3, dtype)
    note(f"[gpu case] determinism shape={shape} dtype={dtype} workspace={ws}")
    h1, dev, _ = gpu_fwd_bwd(inp, shape, dtype, True, 0.125, ws_mode=ws)
    before = {k: v.clone() for k, v in dev.items()}
    h2, dev2, _ = gpu_fwd_bwd(inp, shape, dtype, True, 0.125, ws_mode=ws)
    for n in ("o", "lse", "dq", "dk", "dv", "delta", "lse2"):
        assert np.array_equal(h1[n], h2[n]), n
    for n, t in dev.items():
        assert torch.equal(t, before[n]), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_gradient_invariants_on_gpu(dtype, causal):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold for any inputs."""
    shape = (2, 2, 256, 64)
    inp = synth.make_inputs(shape, 5, dtype)
    note(f"[gpu case] invariants shape={shape} dtype={dtype} causal={causal}")
    h, *_ = gpu_fwd_bwd(inp, shape, dtype, causal, 0.125)
    dk_sum = h["dk"].astype(np.float64).sum(axis=2)
    scale_k = np.abs(h["dk"]).max() * np.sqrt(256)
    assert np.abs(dk_sum).max() <= 10 * TOL[dtype] * scale_k
    dv_sum = h["dv"].astype(np.float64).sum(axis=2)
    do_sum = inp["do"].astype(np.float64).sum(axis=2)
    assert max_rel_err(dv_sum, do_sum) <= 10 * TOL[dtype]


def test_backward_alone_on_oracle_forward():
    """Diagnostic split: the backward fed the oracle's O and LSE (rounded to
    the storage type) must meet the gate on its own."""
    import torch
    import attention_forward_backward_amd as afb
    from parity_util import oracle_all, to_host
    for dtype in ("f32", "bf16"):
        cfg = synth.CONFIGS["decoder_step"]
        shape = (2, 12, 512, 64)
        inp = synth.make_inputs(shape, 0, dtype)
        ref = oracle_all(inp, True, cfg.scale)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        note(f"[gpu case] backward-only shape={shape} dtype={dtype}")
        dev = {}
        for n in ("q", "k", "v", "do"):
            if dtype == "bf16":
                dev[n] = torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
            else:
                dev[n] = torch.from_numpy(inp[n]).cuda()
        o = torch.from_numpy(ref["o"]).to(tdt).cuda()
        lse = torch.from_numpy(ref["lse"]).float().cuda()
        outs = [torch.full(shape, float("nan"), dtype=tdt, device="cuda") for _ in range(3)]
        ws = torch.empty(afb.attn_bwd_workspace_size(int(dtype == "bf16"), *shape, True),
                         dtype=torch.uint8, device="cuda")
        afb.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *outs, ws, True, cfg.scale)
        torch.cuda.synchronize()
        for t, n in zip(outs, ("dq", "dk", "dv")):
            assert max_rel_err(to_host(t), ref[n]) <= TOL[dtype], (dtype, n)


@pytest.mark.parametrize("ws", ["full", "min"])
def test_split_stages_match_fused_call(ws):
    """attn_bwd_prep, attn_bwd_dkdv, attn_bwd_dq in turn give bitwise the same
    as attn_bwd."""
    import torch
    import attention_forward_backward_amd as afb
    shape = (1, 4, 130, 64)
    inp = synth.make_inputs(shape, 2, "f32")
    note(f"[gpu case] split stages shape={shape} workspace={ws}")
    h, dev, outs = gpu_fwd_bwd(inp, shape, "f32", True, 0.125, ws_mode=ws)
    dq = torch.empty_like(outs["dq"])
    dk = torch.empty_like(outs["dk"])
    dv = torch.empty_like(outs["dv"])
    wsf = afb.attn_bwd_workspace_size if ws == "full" else afb.attn_bwd_workspace_size_min
    wsb = torch.empty(wsf(0, *shape, True), dtype=torch.uint8, device="cuda")
    afb.attn_bwd_prep(outs["o"], dev["do"], outs["lse"], wsb)
    afb.attn_bwd_dkdv(dev["q"], dev["k"], dev["v"], dev["do"], dk, dv, wsb, True, 0.125)
    afb.attn_bwd_dq(dev["q"], dev["k"], dev["v"], dev["do"], dq, wsb, True, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(dq, outs["dq"]) and torch.equal(dk, outs["dk"]) and torch.equal(dv, outs["dv"])


@pytest.mark.parametrize("causal", [True, False])
def test_split_stages_bf16(causal):
    """bf16 with the recommended workspace: attn_bwd forms D inside dK+dV (no
    prep launch), while the three stage entry points run the prep pass and
    the dK+dV kernel that reads D from the workspace; both against the
    oracle, and against each other to the rounding of D."""
    import torch
    import attention_forward_backward_amd as afb
    from parity_util import oracle_all, to_host
    shape = (2, 3, 197, 64)
    inp = synth.make_inputs(shape, 5, "bf16")
    note(f"[gpu case] bf16 split stages shape={shape} causal={causal}")
    h, dev, outs = gpu_fwd_bwd(inp, shape, "bf16", causal, 0.125, ws_mode="full")
    ref = oracle_all(inp, causal, 0.125)
    dq, dk, dv = (torch.empty_like(outs[n]) for n in ("dq", "dk", "dv"))
    wsb = torch.empty(afb.attn_bwd_workspace_size(afb.ATTN_BF16, *shape, causal),
                      dtype=torch.uint8, device="cuda")
    afb.attn_bwd_prep(outs["o"], dev["do"], outs["lse"], wsb)
    afb.attn_bwd_dkdv(dev["q"], dev["k"], dev["v"], dev["do"], dk, dv, wsb, causal, 0.125)
    afb.attn_bwd_dq(dev["q"], dev["k"], dev["v"], dev["do"], dq, wsb, causal, 0.125)
    torch.cuda.synchronize()
    for t, n in zip((dq, dk, dv), ("dq", "dk", "dv")):
        staged = to_host(t)
        assert max_rel_err(staged, ref[n]) <= TOL["bf16"], ("staged", n)
        assert max_rel_err(h[n], ref[n]) <= TOL["bf16"], ("fused", n)
        assert max_rel_err(staged, h[n]) <= TOL["bf16"], ("staged vs fused", n)


def test_paths_agree():
    """The dS + GEMM path and the recompute path give the same gradients to
    within rounding (they sum the same terms in a different order)."""
    shape = (2, 3, 197, 64)
    for dtype in ("f32", "bf16"):
        inp = synth.make_inputs(shape, 4, dtype)
        note(f"[gpu case] paths agree shape={shape} dtype={dtype}")
        hf, *_ = gpu_fwd_bwd(inp, shape, dtype, True, 0.125, ws_mode="full")
        hm, *_ = gpu_fwd_bwd(inp, shape, dtype, True, 0.125, ws_mode="min")
        for n in ("o", "lse", "dk", "dv"):
            assert np.array_equal(hf[n], hm[n]), n
        assert max_rel_err(hf["dq"], hm["dq"]) <= TOL[dtype]


@pytest.mark.parametrize("shape,dtype", [((1, 16, 1024, 128), "f32"), ((1, 4, 1024, 64), "bf16")])
@pytest.mark.parametrize("ws", ["full", "ds_only", "split_only"])
def test_few_long_heads_workspace_paths(shape, dtype, ws):
    """Few long causal heads take the query-chunk split of dK+dV (with f32
    tensors the long-context workload itself; with bf16 below 256 (key tile,
    head) items): every workspace layout that selects or skips the split and
    the dS path gives the oracle's result within the contract's gate."""
    B, H, S, D = shape
    code = afb.ATTN_BF16 if dtype == "bf16" else afb.ATTN_F32
    rec = afb.attn_bwd_workspace_size(code, B, H, S, D, True)
    assert rec > workspace_bytes("ds_only", code, shape, True)  # the split's partials are there
    errs, host, *_ = run_case(shape, 0, dtype, True, 1.0 / np.sqrt(D), guard=64, ws_mode=ws)
    for name, e in errs.items():
        assert e <= TOL[dtype], f"{name}: {e:.3e} > {TOL[dtype]} (workspace {ws})"
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert host[name + "_guard_ok"], f"{name}: guard band written"
