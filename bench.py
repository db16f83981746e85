#!/usr/bin/env python3
"""Benchmark: attention forward+backward throughput on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
attn_fwd (O, LSE) followed by attn_bwd (dQ, dK, dV), with every input already
resident in device memory.  The workload is the decoder training-step
attention, B=8 H=12 S=512 D=64 causal, scale 1/8, in both arithmetic
contracts (strict f32 is the headline `value`; bf16 is reported alongside).

Throughput counts credited FLOP = 14*D per visible (query, key) pair
(forward 4*D: QK^T, PV; backward 10*D: QK^T, dO V^T, P^T dO, dS K, dS^T Q),
with S(S+1)/2 visible pairs per head when causal.  Recomputation the kernels
do on top of that is not credited.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (f32 / bf16-MFMA) at B8 H12 S512 D64 causal, 1 GPU"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}  # MI355X dense MFMA: f32, bf16


def mfma_dtype(dt: str, kname: str) -> str:
    """MFMA operand type of one entry point under a contract (f32_bf16fwd: the
    forward multiplies bf16 operands, the backward is strict f32)."""
    if dt == "bf16" or (dt == "f32_bf16fwd" and kname == "attn_fwd"):
        return "bf16"
    return "f32"
PEAK_HBM_GBS = 8000.0
# MFMA FLOP per visible pair that each compute kernel executes (its own
# contractions; the dQ stage is the dS*K GEMM with the recommended workspace)
KERNEL_FLOP_PER_PAIR_D = {"attn_fwd": 4, "attn_bwd_dkdv": 8, "attn_bwd_dq": 2}
KERNEL_SYMBOL = {"attn_fwd": "fwd_kernel", "attn_bwd_prep": "bwd_prep_kernel",
                 "attn_bwd_dkdv": "bwd_dkdv_kernel", "attn_bwd_dq": "bwd_dq_gemm_kernel"}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    # The GPU reaches its sustained clock only after some tens of milliseconds
    # of continuous load; a short warm-up times the clock ramp instead of the
    # kernels (measured on MI355X at B8 H12 S512 D64 f32: 10 warm-up steps
    # give 159.7 us/step, 300 give 141.5, and 2000 timed steps after those
    # 141.2).  300 steps are about 45 ms of f32 work.
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--config", default="decoder_step")
    p.add_argument("--dtypes", default="f32,bf16,f32_bf16fwd",
                   help="first one is the headline value; f32_bf16fwd = float32 tensors, "
                        "bf16-rounded forward operands, strict-f32 backward")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time for the oracle baseline sample")
    p.add_argument("--workspace", choices=("full", "min"), default="full",
                   help="backward workspace: full (dS stored, dQ as a GEMM) or min (dQ recomputes)")
    p.add_argument("--only-step", action="store_true",
                   help="time only the full step (used under a profiler)")
    p.add_argument("--no-cross", action="store_true",
                   help="skip the cross-attention and one-token workloads")
    p.add_argument("--no-rope", action="store_true",
                   help="skip the packed-QKV + RoPE layout pass measurement")
    p.add_argument("--no-graph", action="store_true",
                   help="time the configs, cross and RoPE sections from eager calls only, no HIP graphs "
                        "(for counter runs under a profiler)")
    p.add_argument("--rope-only", action="store_true",
                   help="run only the packed-QKV + RoPE measurement (used under a profiler)")
    p.add_argument("--cross-only", action="store_true",
                   help="run only the cross-attention and one-token workloads (prints their "
                        "section alone; used under a profiler)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip timing the five self-attention workloads (configs key)")
    p.add_argument("--configs-only", action="store_true",
                   help="time only the five self-attention workloads")
    p.add_argument("--no-long-seq", action="store_true",
                   help="skip the longer-sequence shapes (long_seq key)")
    p.add_argument("--long-seq-only", action="store_true",
                   help="time only the longer-sequence shapes")
    p.add_argument("--no-conv", action="store_true",
                   help="skip timing the convolution entry points (conv key)")
    p.add_argument("--conv-only", action="store_true",
                   help="time only the convolution entry points")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="instead of the benchmark, run 5 plain device-to-device copies of "
                        "BYTES bytes (the reference kernel for scaling HBM byte counters)")
    return p.parse_args()


def copy_calibration(nbytes: int) -> None:
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": x.numel() * 4, "launches": 5}), flush=True)


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "attention_forward_backward_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, dtype: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(f"{kernel}/{workload}/{dtype}")
    if not e or e.get("sources") != src_hash:
        return None
    return e.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the attention "
              "path here is single-GPU (every (batch, head) slice is independent, so a "
              "multi-GPU split would give each GPU its own slices).", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_forward_backward_amd as afb
    from attention_forward_backward_amd import synth

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    afb.lib()  # fail loudly if the HIP library is missing

    cfg = synth.CONFIGS[args.config]
    B, H, S, D = cfg.shape
    flops = cfg.flops
    dtypes = [d.strip() for d in args.dtypes.split(",") if d.strip()]
    stream = torch.cuda.current_stream()
    src_hash = kernel_sources_hash()
    workload = f"{cfg.name} B{B} H{H} S{S} D{D} {'causal' if cfg.causal else 'non-causal'}"

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.cross_only:
        print(json.dumps({"cross": cross_section(dtypes, args, stream, log)}), flush=True)
        return
    if args.rope_only:
        print(json.dumps({"rope_packed": rope_section(cfg, dtypes, args, stream, log)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"configs": configs_section(args, log)}), flush=True)
        return
    if args.conv_only:
        print(json.dumps({"conv": conv_section(args, log)}), flush=True)
        return
    if args.long_seq_only:
        print(json.dumps({"long_seq": scaling_section(args, log)}), flush=True)
        return

    results = {}
    for dt in dtypes:
        log(f"[bench] {workload} dtype={dt}: generating inputs")
        inp = synth.config_inputs(cfg, args.seed, "bf16" if dt == "bf16" else "f32")
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        code = {"bf16": afb.ATTN_BF16, "f32": afb.ATTN_F32, "f32_bf16fwd": afb.ATTN_F32_BF16FWD}[dt]
        fast_fwd = dt == "f32_bf16fwd"

        def dev(n):
            if dt == "bf16":
                return torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(inp[n]).cuda()

        q, k, v, do = (dev(n) for n in ("q", "k", "v", "do"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        wsf = afb.attn_bwd_workspace_size if args.workspace == "full" else \
            afb.attn_bwd_workspace_size_min
        ws = torch.empty(wsf(code, B, H, S, D, cfg.causal), dtype=torch.uint8, device="cuda")
        sc = cfg.scale

        def fwd():
            afb.attn_fwd(q, k, v, o, lse, cfg.causal, sc, stream, bf16_operands=fast_fwd)

        def bwd_prep():
            afb.attn_bwd_prep(o, do, lse, ws, stream)

        def bwd_dkdv():
            afb.attn_bwd_dkdv(q, k, v, do, dk, dv, ws, cfg.causal, sc, stream)

        def bwd_dq():
            afb.attn_bwd_dq(q, k, v, do, dq, ws, cfg.causal, sc, stream)

        def bwd():
            afb.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, cfg.causal, sc, stream)

        def step():
            fwd()
            bwd()

        def timed(fn, steps, warmup):
            return timed_events(fn, steps, warmup, stream)  # ms per call

        log(f"[bench] {dt}: {args.warmup} warmup + {args.steps} timed steps (fwd+bwd)")
        ms_step = timed(step, args.steps, args.warmup)
        res = {"ms_per_step": ms_step,
               "value": flops["fwd_bwd"] / (ms_step * 1e-3) / 1e12}
        # The spread of single steps: the same K steps again right after the
        # headline bracket, with an event after each (kept out of the
        # headline bracket so its K steps run back to back).
        _, res["timed_steps"] = timed_events_samples(step, args.steps, 0, stream)
        if not args.only_step:
            res["step_samples"] = step_samples(step, stream)
            ms = {"fwd": timed(fwd, args.steps, 3), "bwd": timed(bwd, args.steps, 3)}
            ms_dq = timed(bwd_dq, args.steps, 3)
            if dt == "bf16" and args.workspace == "full":
                # attn_bwd runs no prep pass here: its dK+dV kernel forms D
                # itself, a variant the split-stage call (which reads D from
                # the workspace) does not launch, so that kernel is timed as
                # the whole backward less the dQ GEMM
                kern = {"attn_fwd": ms["fwd"], "attn_bwd_dkdv": ms["bwd"] - ms_dq,
                        "attn_bwd_dq": ms_dq}
                res["kernels_note"] = ("no prep pass in the step; attn_bwd_dkdv (D formed in "
                                       "dK+dV) = attn_bwd - attn_bwd_dq")
            else:
                kern = {"attn_fwd": ms["fwd"], "attn_bwd_prep": timed(bwd_prep, args.steps, 3),
                        "attn_bwd_dkdv": timed(bwd_dkdv, args.steps, 3),
                        "attn_bwd_dq": ms_dq}
            res["phases"] = {
                ph: {"ms": ms[ph], "tflops": flops[ph] / (ms[ph] * 1e-3) / 1e12,
                     "frac_of_mfma_peak": round(
                         flops[ph] / (ms[ph] * 1e-3) / 1e12 /
                         PEAK_TFLOPS[mfma_dtype(dt, "attn_fwd" if ph == "fwd" else "attn_bwd_dkdv")],
                         4)}
                for ph in ("fwd", "bwd")}
            res["kernels"] = {}
            esz = 2 if dt == "bf16" else 4
            for kname, kms in kern.items():
                if kname == "attn_bwd_prep":
                    # memory-bound: O and dO read, LSE read, D and LSE*log2(e) written
                    kb = 2 * B * H * S * D * esz + 3 * B * H * S * 4
                    res["kernels"][kname] = {
                        "symbol": KERNEL_SYMBOL[kname], "avg_us": kms * 1e3,
                        "bytes_per_launch": kb, "gbs": kb / (kms * 1e-3) / 1e9}
                    continue
                kf = KERNEL_FLOP_PER_PAIR_D[kname] * D * cfg.pairs
                res["kernels"][kname] = {
                    "symbol": KERNEL_SYMBOL[kname], "avg_us": kms * 1e3,
                    "flop_per_launch": kf, "tflops": kf / (kms * 1e-3) / 1e12}
            dom = max((kk for kk in kern if kk != "attn_bwd_prep"), key=kern.get)
            dk_ = res["kernels"][dom]
            achieved = dk_["tflops"]
            peak = PEAK_TFLOPS[mfma_dtype(dt, dom)]
            res["roofline"] = {
                "kernel": dom, "bound": "mfma", "achieved": round(achieved, 3),
                "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": load_traffic(dom, cfg.name, dt, src_hash),
                "flop_per_launch": dk_["flop_per_launch"],
                "avg_launch_us": round(dk_["avg_us"], 3)}
            # against the peak of the backward's MFMA type (most of the step)
            res["step_frac_of_mfma_peak"] = round(
                res["value"] / PEAK_TFLOPS[mfma_dtype(dt, "attn_bwd_dkdv")], 4)
        results[dt] = res
        log(f"[bench] {dt}: {ms_step * 1e3:.1f} us/step, {res['value']:.2f} TFLOP/s")
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()

    head = dtypes[0]
    line = {
        "metric": METRIC,
        "value": round(results[head]["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(results[head]["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head,
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals, seed %d)" % args.seed,
        "config": {"workload": workload, "batch": B, "heads": H, "seq_len": S,
                   "head_dim": D, "causal": cfg.causal, "scale": cfg.scale,
                   "credited_gflop_per_step": flops["fwd_bwd"] / 1e9,
                   "flop_convention": "14*D per visible pair, causal pairs S(S+1)/2",
                   "backward_workspace": args.workspace},
        "kernel_sources": src_hash,
    }
    for key in ("timed_steps", "roofline", "phases", "kernels", "kernels_note",
                "step_frac_of_mfma_peak", "step_samples"):
        if key in results[head]:
            line[key] = results[head][key]
    for dt in dtypes[1:]:
        line[dt] = {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                    for kk, vv in results[dt].items()}

    if not args.no_cross and not args.only_step:
        line["cross"] = cross_section(dtypes, args, stream, log)
    if not args.no_rope and not args.only_step:
        line["rope_packed"] = rope_section(cfg, dtypes, args, stream, log)

    if not args.no_configs and not args.only_step:
        line["configs"] = configs_section(args, log)
    if not args.no_long_seq and not args.only_step:
        line["long_seq"] = scaling_section(args, log)
    if not args.no_conv and not args.only_step:
        line["conv"] = conv_section(args, log)

    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: timing the float64 oracle on the host")
        line["cpu_baseline"] = cpu_baseline(cfg, args.seed, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def visible_pairs(w, kv_len) -> int:
    """Visible (query, key) pairs of a cross workload: query i sees key j iff
    j < L_b and, when causal, j <= i + L_b - Sq."""
    total = 0
    for L in kv_len:
        L = int(L)
        if w.causal:
            per = sum(max(0, min(L, i + 1 + L - w.seq_q)) for i in range(w.seq_q))
        else:
            per = w.seq_q * L
        total += per
    return total * w.heads


def timed_events_samples(fn, steps, warmup, stream):
    """timed_events, plus the time of each call inside the same bracket (an
    event recorded after every call): (ms per call, {median, quartiles,
    minimum, maximum} of the single calls in us)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e3
    stats = {"median_us": round(float(np.median(per)), 2),
             "p25_us": round(float(np.percentile(per, 25)), 2),
             "p75_us": round(float(np.percentile(per, 75)), 2),
             "min_us": round(float(per.min()), 2), "max_us": round(float(per.max()), 2),
             "samples": int(steps)}
    return ev[0].elapsed_time(ev[-1]) / steps, stats


def timed_events(fn, steps, warmup, stream):
    """ms per call of fn: warmup calls, then steps calls between two events
    on `stream`, synchronised on both sides."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_samples(step, stream, n: int = 50, flush_bytes: int = 512 << 20) -> dict:
    """Distribution of single-step times (HIP events around each step, one
    synchronisation per sample): "warm" back to back, as in repeated
    training steps (the working set stays in the 256 MB Infinity Cache), and
    "flushed" with a 512 MB buffer written between samples, so the step
    starts from HBM.  Median, quartiles, minimum and maximum in us."""
    import torch
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    out = {}
    for mode in ("warm", "flushed"):
        t = []
        for _ in range(n):
            if mode == "flushed":
                scratch.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3)
        q = np.percentile(t, [0, 25, 50, 75, 100])
        out[mode] = {"median_us": round(float(q[2]), 2), "p25_us": round(float(q[1]), 2),
                     "p75_us": round(float(q[3]), 2), "min_us": round(float(q[0]), 2),
                     "max_us": round(float(q[4]), 2), "samples": n}
    del scratch
    return out


def timed_graph(fn, per_graph=20, replays=30):
    """ms per call of fn from replays of a HIP graph of per_graph calls (no
    host launch cost between calls); fn launches on the current stream."""
    import torch
    for _ in range(per_graph):
        fn()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(per_graph):
            fn()
    for _ in range(3):
        gr.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    del gr
    return e0.elapsed_time(e1) / (replays * per_graph)


def configs_section(args, log) -> dict:
    """fwd, bwd and fwd+bwd of every self-attention workload (tiny, small
    decoder, decoder step, long context, ragged encoder) in each of its
    contracts (the forward with the key split where attn_fwd_workspace_size
    gives it a workspace), GPU time from HIP-graph replays (eager calls with
    --no-graph):
    credited TFLOP/s, its fraction of the contract's dense MFMA peak and of
    the attainable roofline min(peak, FLOP per compulsory byte x 8 TB/s), and
    the compulsory HBM bytes (every input read once, every output written
    once) per second."""
    import torch
    import attention_forward_backward_amd as afb
    from attention_forward_backward_amd import synth

    out = {}
    for name, cfg in synth.CONFIGS.items():
        B, H, S, D = cfg.shape
        T, L = B * H * S * D, B * H * S
        rec = {"shape": f"B{B} H{H} S{S} D{D} {'causal' if cfg.causal else 'non-causal'}",
               "visible_pairs": cfg.pairs}
        for dt in cfg.dtypes:
            inp = synth.config_inputs(cfg, args.seed, dt)

            def dev(n):
                if dt == "bf16":
                    return torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
                return torch.from_numpy(inp[n]).cuda()

            q, k, v, do = (dev(n) for n in ("q", "k", "v", "do"))
            o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
            lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
            code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
            ws = torch.empty(afb.attn_bwd_workspace_size(code, B, H, S, D, cfg.causal),
                             dtype=torch.uint8, device="cuda")
            # the key-split forward where the shape takes it (few long heads)
            fws_bytes = afb.attn_fwd_workspace_size(code, B, H, S, D, cfg.causal)
            fws = torch.empty(fws_bytes, dtype=torch.uint8, device="cuda") if fws_bytes else None

            def fwd():
                afb.attn_fwd_ws(q, k, v, o, lse, fws, cfg.causal, cfg.scale, None)

            def bwd():
                afb.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, cfg.causal, cfg.scale, None)

            def step():
                fwd()
                bwd()

            log(f"[bench] configs {name} {rec['shape']} dtype={dt}")
            step()
            if args.no_graph:
                tm = lambda fn: timed_events(fn, args.steps, 3, torch.cuda.current_stream())
            else:
                tm = timed_graph
            ms = {"fwd": tm(fwd), "bwd": tm(bwd), "fwd_bwd": tm(step)}
            esz = 2 if dt == "bf16" else 4
            nbytes = {"fwd": 4 * T * esz + 4 * L, "bwd": 8 * T * esz + 4 * L}
            nbytes["fwd_bwd"] = nbytes["fwd"] + nbytes["bwd"]
            peak = PEAK_TFLOPS["bf16" if dt == "bf16" else "f32"]
            r = {}
            for ph in ("fwd", "bwd", "fwd_bwd"):
                tf = cfg.flops[ph] / (ms[ph] * 1e-3) / 1e12
                # attainable: min(MFMA peak, arithmetic intensity x HBM peak)
                attain = min(peak, cfg.flops[ph] / nbytes[ph] * PEAK_HBM_GBS / 1e3)
                r[ph] = {"us": round(ms[ph] * 1e3, 2), "tflops": round(tf, 3),
                         "frac_of_mfma_peak": round(tf / peak, 4),
                         "attainable_tflops": round(attain, 1),
                         "frac_of_attainable": round(tf / attain, 4),
                         "compulsory_bytes": nbytes[ph],
                         "gbs": round(nbytes[ph] / (ms[ph] * 1e-3) / 1e9, 1)}
            r["forward_key_split"] = bool(fws_bytes)
            rec[dt] = r
            del q, k, v, do, o, dq, dk, dv, lse, ws, fws
            torch.cuda.empty_cache()
        out[name] = rec
    return out




def scaling_section(args, log) -> dict:
    """fwd+bwd of causal self-attention at longer sequences, both contracts,
    GPU time from HIP-graph replays (recommended workspace): credited
    TFLOP/s (14 D per visible pair) and its fraction of the MFMA peak."""
    import torch
    import attention_forward_backward_amd as afb
    from attention_forward_backward_amd import synth

    out = {}
    for (B, H, S, D) in synth.LONG_SEQ_SHAPES:
        name = f"B{B} H{H} S{S} D{D} causal"
        pairs = B * H * S * (S + 1) // 2
        rec = {"visible_pairs": pairs}
        for dt in ("f32", "bf16"):
            inp = synth.make_inputs((B, H, S, D), args.seed, dt)

            def dev(n):
                if dt == "bf16":
                    return torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
                return torch.from_numpy(inp[n]).cuda()

            q, k, v, do = (dev(n) for n in ("q", "k", "v", "do"))
            o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
            lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
            code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
            ws = torch.empty(afb.attn_bwd_workspace_size(code, B, H, S, D, True),
                             dtype=torch.uint8, device="cuda")
            sc = 1.0 / math.sqrt(D)

            def fwd():
                afb.attn_fwd(q, k, v, o, lse, True, sc, None)

            def step():
                fwd()
                afb.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, True, sc, None)

            log(f"[bench] scaling {name} dtype={dt}")
            step()
            ms_f, ms_s = timed_graph(fwd, 10, 10), timed_graph(step, 10, 10)
            peak = PEAK_TFLOPS["bf16" if dt == "bf16" else "f32"]
            tf_f = 4 * D * pairs / (ms_f * 1e-3) / 1e12
            tf_s = 14 * D * pairs / (ms_s * 1e-3) / 1e12
            rec[dt] = {"fwd_us": round(ms_f * 1e3, 1), "fwd_tflops": round(tf_f, 1),
                       "fwd_frac_of_mfma_peak": round(tf_f / peak, 4),
                       "fwd_bwd_us": round(ms_s * 1e3, 1), "fwd_bwd_tflops": round(tf_s, 1),
                       "fwd_bwd_frac_of_mfma_peak": round(tf_s / peak, 4)}
            del q, k, v, do, o, dq, dk, dv, lse, ws
            torch.cuda.empty_cache()
        out[name] = rec
    return out




def conv_section(args, log) -> dict:
    """Forward, data derivative and filter derivative of three ResNet-50
    convolutions (include/conv.h), strict f32 and bf16: time per call from
    HIP events over back-to-back calls, TFLOP/s (2 N P Q K R S C per call)
    and its fraction of the contract's dense MFMA peak."""
    import torch
    import attention_forward_backward_amd as afb
    from attention_forward_backward_amd import synth

    stream = torch.cuda.current_stream()
    out = {}
    for name, (N, H, W, C, K, R, S, st, pd) in synth.CONV_LAYERS.items():
        P, Q = afb.conv2d_out_size(H, W, R, S, st, pd)
        flop = 2 * N * P * Q * K * R * S * C
        rec = {"shape": f"N{N} {H}x{W} C{C} K{K} {R}x{S} stride {st[0]} pad {pd[0]}",
               "flop_per_call": flop}
        for dt in ("f32", "bf16"):
            inp = synth.conv_inputs((N, H, W, C), (K, R, S, C), (N, P, Q, K), args.seed, dt)

            def dev(n):
                if dt == "bf16":
                    return torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
                return torch.from_numpy(inp[n]).cuda()

            x, w, dy = dev("x"), dev("w"), dev("dy")
            y, dx, dw = torch.empty_like(dy), torch.empty_like(x), torch.empty_like(w)
            code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
            wsb = afb.conv2d_bwd_filter_workspace_size(code, x.shape, w.shape, st, pd)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
            calls = {"fwd": lambda: afb.conv2d_fwd(x, w, y, st, pd),
                     "bwd_data": lambda: afb.conv2d_bwd_data(dy, w, dx, st, pd),
                     "bwd_filter": lambda: afb.conv2d_bwd_filter(x, dy, dw, ws, st, pd)}
            log(f"[bench] conv {name} {rec['shape']} dtype={dt}")
            peak = PEAK_TFLOPS["bf16" if dt == "bf16" else "f32"]
            r = {}
            if name.startswith("stem"):
                del calls["bwd_data"]
            for op, fn in calls.items():
                ms = timed_events(fn, 20, 3, stream)
                tf = flop / (ms * 1e-3) / 1e12
                r[op] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 2),
                         "frac_of_mfma_peak": round(tf / peak, 4)}
            rec[dt] = r
            del x, w, dy, y, dx, dw, ws
            torch.cuda.empty_cache()
        out[name] = rec
    return out


def cross_section(dtypes, args, stream, log) -> dict:
    """fwd and fwd+bwd time of the cross-attention and one-token workloads
    (attn_fwd_cross / attn_bwd_cross), per arithmetic contract: from replays
    of a HIP graph (fwd_us, fwd_bwd_us: GPU time, the one-token calls are
    shorter than a Python launch) and from eager calls (*_eager)."""
    import torch
    import attention_forward_backward_amd as afb
    from attention_forward_backward_amd import synth

    def timed(fn, steps, warmup):
        return timed_events(fn, steps, warmup, stream)

    out = {}
    for wname, w in synth.CROSS_WORKLOADS.items():
        B, H, Sq, Sk, D = w.batch, w.heads, w.seq_q, w.seq_k, w.head_dim
        kvl = synth.key_lengths(args.seed, B, w.min_keys, Sk) if w.padded else None
        pairs = visible_pairs(w, kvl if kvl is not None else [Sk] * B)
        rec = {"shape": f"B{B} H{H} Sq{Sq} Sk{Sk} D{D} {'causal' if w.causal else 'non-causal'}",
               "kv_len": None if kvl is None else kvl.tolist(), "visible_pairs": pairs}
        for dt in dtypes:
            sd = "bf16" if dt == "bf16" else "f32"
            inp = synth.cross_inputs((B, H, Sq, D), (B, H, Sk, D), args.seed, sd)

            def dev(n):
                if dt == "bf16":
                    return torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda()
                return torch.from_numpy(inp[n]).cuda()

            q, k, v, do = (dev(n) for n in ("q", "k", "v", "do"))
            kv = None if kvl is None else torch.from_numpy(kvl).cuda()
            o, dq = torch.empty_like(q), torch.empty_like(q)
            dk, dv = torch.empty_like(k), torch.empty_like(v)
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
            code = {"bf16": afb.ATTN_BF16, "f32": afb.ATTN_F32,
                    "f32_bf16fwd": afb.ATTN_F32_BF16FWD}[dt]
            ws = torch.empty(afb.attn_bwd_cross_workspace_size(code, B, H, Sq, Sk, D, w.causal),
                             dtype=torch.uint8, device="cuda")
            fast = dt == "f32_bf16fwd"

            # stream=None: the current stream (the capture stream in a graph)
            def fwd():
                afb.attn_fwd_cross(q, k, v, o, lse, kv, w.causal, w.scale, None,
                                   bf16_operands=fast)

            def step():
                fwd()
                afb.attn_bwd_cross(q, k, v, o, do, lse, dq, dk, dv, ws, kv, w.causal, w.scale,
                                   None)

            log(f"[bench] cross {wname} {rec['shape']} dtype={dt}")
            ms_fe = timed(fwd, args.steps, args.warmup)
            ms_se = timed(step, args.steps, args.warmup)
            ms_f = ms_fe if args.no_graph else timed_graph(fwd)
            ms_s = ms_se if args.no_graph else timed_graph(step)
            # forward's algorithmic HBM bytes: Q and O, the valid K and V
            # rows, the LSE
            esz = 2 if dt == "bf16" else 4
            nkeys = int(sum(kvl)) if kvl is not None else B * Sk
            fbytes = (2 * B * H * Sq * D + 2 * H * nkeys * D) * esz + B * H * Sq * 4
            gbs = fbytes / (ms_f * 1e-3) / 1e9
            rec[dt] = {"fwd_us": round(ms_f * 1e3, 2), "fwd_bwd_us": round(ms_s * 1e3, 2),
                       "fwd_us_eager": round(ms_fe * 1e3, 2),
                       "fwd_bwd_us_eager": round(ms_se * 1e3, 2),
                       "fwd_tflops": round(4 * D * pairs / (ms_f * 1e-3) / 1e12, 3),
                       "fwd_bwd_tflops": round(14 * D * pairs / (ms_s * 1e-3) / 1e12, 3),
                       "fwd_bytes": fbytes, "fwd_gbs": round(gbs, 1),
                       "fwd_frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
            del q, k, v, do, o, dq, dk, dv, lse, ws
        out[wname] = rec
    torch.cuda.empty_cache()
    return out


def eager_time(fn, steps: int) -> float:
    """ms per call of fn over `steps` eager calls after as many warm-up calls."""
    import torch
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_time(fn, per_graph=20, replays=30) -> float:
    """ms per call of fn from replays of a HIP graph of per_graph calls."""
    import torch
    for _ in range(per_graph):
        fn()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(per_graph):
            fn()
    for _ in range(3):
        gr.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    del gr
    return e0.elapsed_time(e1) / (replays * per_graph)


def rope_section(cfg, dtypes, args, stream, log) -> dict:
    """The workload's step on a packed [B, S, 3, H, D] projection with 1-D
    RoPE on Q and K, O and dO in [B, S, H, D], three ways:
    fused (attn_fwd_rope + attn_bwd_rope: Q and K tiles turned inside the
    forward kernel, dQ and dK turned back in the kernels that store them);
    with separate passes (attn_rope_copy turns Q and K into
    [B, H, S, D] before the strided kernels and takes dQ, dK back through the
    transposed rotation after them); and the packed step without RoPE.  A
    rotation pass reads and writes one [B, H, S, D] tensor (plus table rows):
    HBM-bound.  Timed from HIP graph replays."""
    import torch
    import attention_forward_backward_amd as afb
    from attention_forward_backward_amd import synth
    B, H, S, D = cfg.shape
    shp = (B, H, S, D)
    # 1-D rotary angles p * 10000^(-2i/D) (the input tables of the pass)
    ang = np.arange(S)[:, None] * 10000.0 ** (-2.0 * np.arange(D // 2) / D)
    ct = torch.from_numpy(np.cos(ang).astype(np.float32)).cuda()
    st = torch.from_numpy(np.sin(ang).astype(np.float32)).cuda()
    offs, pst = afb.packed_qkv(H, S, D)
    bhsd, bshd = afb.strides_bhsd(H, S, D), afb.strides_bshd(H, S, D)
    out = {"layout": "packed [B,S,3,H,D] QKV, dO and O in [B,S,H,D]", "rope": "1-D, base 10000"}
    for dt in dtypes:
        if dt == "f32_bf16fwd":
            continue
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        pk = torch.from_numpy(synth.normal_f32(args.seed, 0, (B, S, 3, H, D))).cuda().to(tdt)
        dOt = torch.from_numpy(synth.normal_f32(args.seed, 3, (B, S, H, D))).cuda().to(tdt)
        q, k, dq, dk = (torch.empty(shp, dtype=tdt, device="cuda") for _ in range(4))
        o_s = torch.empty((B, S, H, D), dtype=tdt, device="cuda")
        dpk = torch.empty_like(pk)
        lse = torch.empty((B, H, S), device="cuda")
        code = afb.ATTN_BF16 if dt == "bf16" else afb.ATTN_F32
        ws = torch.empty(afb.attn_bwd_cross_workspace_size(code, B, H, S, S, D, cfg.causal),
                         dtype=torch.uint8, device="cuda")

        # the strided kernels read V straight from the packed projection and
        # dO from [B,S,H,D], and write O to [B,S,H,D] and dV into the packed
        # gradient; only the rotated Q, K and the gradients through the
        # rotation (dQ, dK) take a pass
        v_view = pk[:, :, 2].permute(0, 2, 1, 3)
        o_view = o_s.permute(0, 2, 1, 3)
        do_view = dOt.permute(0, 2, 1, 3)
        dv_view = dpk[:, :, 2].permute(0, 2, 1, 3)

        def prologue():
            afb.attn_rope_copy(pk, offs[0], pst, q, 0, bhsd, shp, ct, st)
            afb.attn_rope_copy(pk, offs[1], pst, k, 0, bhsd, shp, ct, st)

        def epilogue():
            afb.attn_rope_copy(dq, 0, bhsd, dpk, offs[0], pst, shp, ct, st, transpose=True)
            afb.attn_rope_copy(dk, 0, bhsd, dpk, offs[1], pst, shp, ct, st, transpose=True)

        def step():
            prologue()
            afb.attn_fwd_strided(q, k, v_view, o_view, lse, None, cfg.causal, cfg.scale)
            afb.attn_bwd_strided(q, k, v_view, o_view, do_view, lse, dq, dk, dv_view, ws, None,
                                 cfg.causal, cfg.scale)
            epilogue()

        # the same step without RoPE: every tensor read and written in place
        q_view, k_view = pk[:, :, 0].permute(0, 2, 1, 3), pk[:, :, 1].permute(0, 2, 1, 3)
        dq_view, dk_view = dpk[:, :, 0].permute(0, 2, 1, 3), dpk[:, :, 1].permute(0, 2, 1, 3)

        qk = torch.empty((2,) + shp, dtype=tdt, device="cuda")
        dq_view0, dk_view0 = dpk[:, :, 0].permute(0, 2, 1, 3), dpk[:, :, 1].permute(0, 2, 1, 3)
        q_raw, k_raw = pk[:, :, 0].permute(0, 2, 1, 3), pk[:, :, 1].permute(0, 2, 1, 3)

        def step_fused():
            afb.attn_fwd_rope(q_raw, k_raw, v_view, o_view, lse, qk, ct, st, cfg.causal,
                              cfg.scale)
            afb.attn_bwd_rope(qk, v_view, o_view, do_view, lse, dq_view0, dk_view0, dv_view, ws,
                              ct, st, cfg.causal, cfg.scale)

        def fwd_fused():
            afb.attn_fwd_rope(q_raw, k_raw, v_view, o_view, lse, qk, ct, st, cfg.causal,
                              cfg.scale)

        def step_plain():
            afb.attn_fwd_strided(q_view, k_view, v_view, o_view, lse, None, cfg.causal, cfg.scale)
            afb.attn_bwd_strided(q_view, k_view, v_view, o_view, do_view, lse, dq_view, dk_view,
                                 dv_view, ws, None, cfg.causal, cfg.scale)

        log(f"[bench] packed QKV + RoPE {shp} dtype={dt}")
        esz = 2 if dt == "bf16" else 4
        tb = B * H * S * D * esz
        rot = lambda: afb.attn_rope_copy(pk, offs[0], pst, q, 0, bhsd, shp, ct, st)
        tf = (lambda fn: eager_time(fn, args.steps)) if args.no_graph else graph_time
        ms_rot = tf(rot)
        bytes_rot = 2 * tb + 2 * S * (D // 2) * 4
        ms_pro, ms_epi, ms_step = tf(prologue), tf(epilogue), tf(step)
        ms_plain = tf(step_plain)
        ms_fused, ms_ffwd = tf(step_fused), tf(fwd_fused)
        gbs = bytes_rot / (ms_rot * 1e-3) / 1e9
        out[dt] = {"fused_step_us": round(ms_fused * 1e3, 2),
                   "fused_fwd_us": round(ms_ffwd * 1e3, 2),
                   "packed_step_no_rope_us": round(ms_plain * 1e3, 2),
                   "fused_overhead_frac": round(ms_fused / ms_plain - 1.0, 4),
                   "passes_step_us": round(ms_step * 1e3, 2),
                   "rotate_us": round(ms_rot * 1e3, 2), "rotate_bytes": bytes_rot,
                   "rotate_gbs": round(gbs, 1), "rotate_frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                   "prologue_us": round(ms_pro * 1e3, 2), "epilogue_us": round(ms_epi * 1e3, 2)}
        del pk, dOt, q, k, dq, dk, o_s, dpk, lse, ws, qk
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo; 'unknown' if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, seed: int, target_s: float) -> dict:
    """The float64 oracle, as it stands, timed on this host's cores over whole
    passes of the workload: once with its BLAS held to one thread and once
    with every thread the BLAS library starts, each leg until about
    target_s / 2 seconds have passed.  `value` is the all-core leg."""
    import oracle
    from attention_forward_backward_amd import synth
    from threadpoolctl import threadpool_info, threadpool_limits

    inp = synth.config_inputs(cfg, seed, "f32")
    q, k, v, do = (inp[n].astype(np.float64) for n in ("q", "k", "v", "do"))

    def leg(limit_s: float) -> tuple:
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.attention_forward(q, k, v, cfg.causal, cfg.scale)
            oracle.attention_backward(q, k, v, do, cfg.causal, cfg.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= limit_s or el / reps * (reps + 1) > 2.5 * limit_s:
                break
        return reps, el / reps

    with threadpool_limits(limits=1):
        reps1, per1 = leg(target_s / 2)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    repsn, pern = leg(target_s / 2)
    flop = cfg.flops["fwd_bwd"]
    return {"value": flop / pern / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "logical_cpus": os.cpu_count(),
            "single_thread": {"value": flop / per1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "s_per_pass": round(per1, 3), "passes": reps1},
            "sample": f"{repsn} full pass(es) of the {cfg.name} workload (fwd+bwd, float64, "
                      f"numpy oracle) with {threads} BLAS threads, {pern:.2f} s per pass; "
                      f"single-thread leg {reps1} pass(es), {per1:.2f} s per pass"}


if __name__ == "__main__":
    main()
