"""The allocation-free backward (attn_bwd_noalloc, include/attn.h) against the
backward with a caller-owned workspace (attn_bwd) and against the float64
oracle: two calls in a row on one GPU, the second on a smaller input, each
called through the C ABI with raw device pointers.  The library's scratch
array keeps the first call's contents, so the second call also shows that
nothing left in it leaks into a result."""
import ctypes

import numpy as np
import pytest

import attention_forward_backward_amd as afb
from attention_forward_backward_amd import synth
import oracle
from parity_util import TOL, max_rel_err, note, to_device, to_host

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20  # ATTN_BWD_NOALLOC_MAX_BYTES


def _run_pair(shape, dt, causal, seed):
    """Forward, then the backward twice: attn_bwd_noalloc and attn_bwd with
    a workspace of the size the scratch array gives (the same layout)."""
    import torch
    B, H, S, D = shape
    scale = 1.0 / np.sqrt(D)
    inp = synth.make_inputs(shape, seed, dt)
    dev = {n: to_device(inp[n], inp.get(n + "_bits"), dt) for n in ("q", "k", "v", "do")}
    nan = float("nan")
    tdt = dev["q"].dtype
    o = torch.full(shape, nan, dtype=tdt, device="cuda")
    lse = torch.full((B, H, S), nan, device="cuda")
    afb.attn_fwd(dev["q"], dev["k"], dev["v"], o, lse, causal, scale)
    code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
    grads = {}
    for mode in ("noalloc", "workspace"):
        dq, dk, dv = (torch.full(shape, nan, dtype=tdt, device="cuda") for _ in range(3))
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        note(f"[gpu case] {mode} backward shape={shape} dtype={dt} causal={causal} seed={seed}")
        if mode == "noalloc":
            rc = afb.lib().attn_bwd_noalloc(code, dev["q"].data_ptr(), dev["k"].data_ptr(),
                                            dev["v"].data_ptr(), o.data_ptr(),
                                            dev["do"].data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                            dk.data_ptr(), dv.data_ptr(), B, H, S, D,
                                            int(causal), float(scale), stream)
        else:
            nbytes = min(afb.attn_bwd_workspace_size(code, B, H, S, D, causal), SCRATCH_BYTES)
            ws = torch.full((nbytes // 4,), nan, device="cuda")
            rc = afb.lib().attn_bwd(code, dev["q"].data_ptr(), dev["k"].data_ptr(),
                                    dev["v"].data_ptr(), o.data_ptr(), dev["do"].data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    ws.data_ptr(), nbytes, B, H, S, D, int(causal),
                                    float(scale), stream)
        assert rc == 0, afb.STATUS.get(rc, rc)
        torch.cuda.synchronize()
        grads[mode] = {n: to_host(t) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    return inp, grads, scale


@pytest.mark.parametrize("first,second", [
    (((8, 12, 512, 64), "f32", True), ((2, 3, 197, 64), "bf16", False)),
    (((8, 12, 512, 64), "bf16", True), ((1, 2, 130, 128), "f32", True)),
])
def test_noalloc_matches_workspace_backward(first, second):
    for seed, (shape, dt, causal) in enumerate((first, second)):
        inp, grads, scale = _run_pair(shape, dt, causal, seed)
        for n in ("dq", "dk", "dv"):
            assert np.all(np.isfinite(grads["noalloc"][n])), n
            # the same kernels on the same workspace layout: bitwise equal
            assert np.array_equal(grads["noalloc"][n], grads["workspace"][n]), n
        # and within the contract's gate of the oracle (first, middle and
        # last (b, h) slices)
        B, H = shape[:2]
        for b, h in sorted({(0, 0), (B // 2, H // 2), (B - 1, H - 1)}):
            x = {n: inp[n][b:b + 1, h:h + 1].astype(np.float64) for n in ("q", "k", "v", "do")}
            rdq, rdk, rdv, _ = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal,
                                                         scale)
            for n, ref in (("dq", rdq), ("dk", rdk), ("dv", rdv)):
                e = max_rel_err(grads["noalloc"][n][b:b + 1, h:h + 1], ref)
                assert e <= TOL[dt], (shape, dt, n, e)
