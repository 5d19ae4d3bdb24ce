#!/usr/bin/env python
"""Benchmark: one d20-shaped GPT block training step (forward + backward) on
one MI355X, B=4, T=2048, width 1280, 10 heads x 128, RMSNorm, RoPE, QK-norm.

Prints one JSON line: tokens/s of the step, the roofline of the dominant
kernel (timed with hipEvents on the library's stream during a traced pass of
the same steps), and the float64 CPU oracle timed on a bounded sample of the
same workload.  Inputs are seeded synthetic tensors resident in HBM before
the timed region starts.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

METRIC = "train tokens/s (fwd+bwd) on 1 GPU, d20 shape; % bf16 MFMA peak"
PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12        # MI355X HBM3E, B/s
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_PROFILE = os.path.join(HERE, "profiles", "hbm_traffic_d20_block_fwd_bwd.md")
CSRC = os.path.join(HERE, "decoder_only_gpt_bf16_amd", "csrc")

# call site -> (kernels as named in the counter summary, their source files);
# sites that share a GEMM instance with others have no entry
SITE_KERNEL = {
    "attn_fwd": (["attn_fwd_mfma<128, true>"], "attention"),
    "attn_bwd_dkdv": (["attn_bwd_dkdv_mfma<128>"], "attention"),
    "attn_bwd_dq": (["attn_bwd_dq_mfma<128>"], "attention"),
    "qkv_gemm": (["gemm_mfma<false, false, 6, 256, 256, 8, 2, 0>"], "gemm"),
    "fc_gemm_gelu": (["gemm_mfma<false, false, 1, 256, 320, 8, 4, 0>"], "gemm"),
    "proj_dgrad_gelu": (["gemm_mfma<false, true, 2, 256, 320, 8, 4, 0>"], "gemm"),
    "wgrad_group": (["gemm_group_dp<true, true, 3, 256, 320, 8, 4, 0>"], "gemm"),
    # rocprofv3 prints the bf16 instances of the norm kernels this way
    "norm1_fwd": (["norm_fwd_k<bool _Accum, int, E, true, 3>"], "norm"),
    "norm2_fwd": (["norm_fwd_k<bool _Accum, int, E, false, 3>"], "norm"),
    # the two backward norms are one instance at one shape
    "norm1_bwd": (["norm_bwd_k<bool _Accum, int, E, false, 3>"], "norm"),
    "norm2_bwd": (["norm_bwd_k<bool _Accum, int, E, false, 3>"], "norm"),
}
SOURCES = {"attention": ["attention.hip", "common.h", "kernels.h"], "gemm": ["gemm.hip", "common.h", "kernels.h"],
           "xent": ["xent.hip", "common.h", "kernels.h"], "norm": ["norm.hip", "common.h", "kernels.h"]}
# the LM heads: one counter summary per head (their kernels are shared, with
# other shapes), call site -> kernels as for the block
HEAD_PROFILES = {name: os.path.join(HERE, "profiles", f"hbm_traffic_{name}.md")
                 for name in ("gpt2_124m_step_head", "d20_val_bpb_head")}
HEAD_SITE_KERNEL = {
    "xent_stats_gemm": (["gemm_mfma<false, false, 4, 256, 256, 8, 2, 0>"], "gemm"),
    "xent_grad_gemm": (["gemm_mfma<false, false, 5, 256, 256, 8, 2, 0>"], "gemm"),
    "xent_dh_gemm": (["gemm_mfma<false, true, 3, 256, 192, 8, 4, 0>"], "gemm"),
    "xent_finish": (["xent_finish_k"], "xent"),
    "xent_dh_convert": (["_ZN12_GLOBAL__N_18f32_to_kIDF16bEEvlPKfPT_"], "xent"),
}


def block_flops(B, T, C, H):
    """Useful FLOPs of one block fwd+bwd: 6 * 12 C^2 per token for the
    Linear layers, causal attention counted on the lower triangle."""
    D = C // H
    N = B * T
    lin = 6 * 12 * C * C * N
    attn_fwd = 2 * B * H * D * T * T        # QK^T and PV, each 2*B*H*D*T^2/2
    return lin + 3 * attn_fwd                 # backward = 2x forward


def site_work(name, B, T, C, H):
    """(bound, algorithmic work per launch) of a block call site."""
    N, D = B * T, C // H
    g = lambda m, n, k: 2.0 * m * n * k  # noqa: E731
    half = B * H * D * T * T                 # one causal T x T x D product (2*T^2*D/2 per head)
    flops = {
        "qkv_gemm": g(N, 3 * C, C), "qkv_dgrad": g(N, C, 3 * C), "qkv_wgrad": g(3 * C, C, N),
        "out_gemm": g(N, C, C), "out_dgrad": g(N, C, C), "out_wgrad": g(C, C, N),
        "fc_gemm_gelu": g(N, 4 * C, C), "fc_dgrad": g(N, C, 4 * C), "fc_wgrad": g(4 * C, C, N),
        "proj_gemm": g(N, C, 4 * C), "proj_dgrad_gelu": g(N, 4 * C, C), "proj_wgrad": g(C, 4 * C, N),
        "attn_fwd": 2 * half, "attn_bwd_dkdv": 3 * half, "attn_bwd_dq": 1 * half,
        # the four weight gradients as one grouped launch
        "wgrad_group": g(3 * C, C, N) + g(C, C, N) + g(4 * C, C, N) + g(C, 4 * C, N),
    }
    if name in flops:
        return "mfma", flops[name]
    s = 2  # bf16
    bytes_ = {
        "norm1_fwd": N * C * 2 * s + 8 * N, "norm2_fwd": N * C * 2 * s + 8 * N,
        "norm1_bwd": N * C * 4 * s, "norm2_bwd": N * C * 4 * s,
        "qk_rope_norm": 2 * N * 2 * C * s, "qk_bwd": 3 * N * 2 * C * s,
        "attn_delta": 2 * N * C * s + 4 * N * H,
    }
    if name in bytes_:
        return "hbm", bytes_[name]
    return None, None


def source_hash(family):
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES[family]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(site, profile=TRAFFIC_PROFILE, table=None):
    """HBM bytes per launch of a call site's kernel (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated) from a committed counter summary, or None when the
    site's kernel is not uniquely named there or its sources changed since
    the counters were taken."""
    table = SITE_KERNEL if table is None else table
    if site not in table or not os.path.exists(profile):
        return None
    kernels, fam = table[site]
    want = source_hash(fam)
    found = {}
    with open(profile) as fh:
        for line in fh:
            cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
            if len(cells) == 6 and cells[0] in kernels:
                if cells[5] != want:
                    return None
                found[cells[0]] = int(cells[4])
    return sum(found.values()) if len(found) == len(kernels) else None


def cpu_baseline(w, run_s=4.0, runs=3):
    """The float64 oracle on whole sequences of the workload, one at a time
    (sequence b of the same seeded batch): `runs` runs of at least run_s
    seconds each on the BLAS thread pool as configured, whose median is the
    value; then, with one BLAS thread, one sequence of the GPT-2 and d20
    blocks and one whole tiny-model step (loss and every gradient)."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = len(os.sched_getaffinity(0))
    import oracle as O
    from decoder_only_gpt_bf16_amd import synth

    def block_seqs(wl, min_s):
        x, dy, p = synth.make_block_inputs(wl)
        cfg = synth.oracle_cfg(wl.cfg)
        n, dt = 0, 0.0
        t0 = time.perf_counter()
        while n == 0 or dt < min_s:
            b = n % wl.B
            y, cache = O.block_fwd(cfg, x[b:b + 1], p)
            O.block_bwd(cfg, dy[b:b + 1], cache, p)
            n += 1
            dt = time.perf_counter() - t0
        return n, dt

    rates, total_n, total_s = [], 0, 0.0
    for _ in range(runs):
        n, dt = block_seqs(w, run_s)
        rates.append(n * w.T / dt)
        total_n += n
        total_s += dt
    rates.sort()
    out = {"value": rates[len(rates) // 2], "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "runs": [round(r, 1) for r in rates],
           "sample": f"median of {runs} runs of >= {run_s:.0f} s, {total_n} sequences (B=1, T={w.T} each) of the "
                     f"d20 block fwd+bwd in float64 NumPy, {total_s:.1f} s in all"}
    if threadpool_limits is not None:
        single = {}
        with threadpool_limits(1):
            for name in ("gpt2_block", "d20_block"):
                wl = synth.BY_NAME[name]
                n, dt = block_seqs(wl, 0.0)
                single[name] = {"tokens_per_s": round(n * wl.T / dt, 1), "seconds": round(dt, 2),
                                "sample": f"one sequence (T={wl.T}) fwd+bwd"}
            wl = synth.TINY
            ids, y, P, _ = synth.make_model_inputs(wl)
            cfg = synth.oracle_cfg(wl.cfg)
            t0 = time.perf_counter()
            O.model_fwd_bwd(cfg, ids, y, P)
            dt = time.perf_counter() - t0
            single[wl.name] = {"tokens_per_s": round(wl.B * wl.T / dt, 1), "seconds": round(dt, 4),
                               "sample": f"one whole step (B={wl.B}, T={wl.T})"}
        out["single_thread"] = single
    return out


def time_steps(fn, steps, warmup, per_step=None):
    """Mean ms per step of `steps` calls bracketed by synchronizations
    (hipEvents on the current stream, the library's stream).  per_step (a
    list) receives each step's own event-timed ms as well."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)] if per_step is not None else None
    a.record()
    for i in range(steps):
        if ev:
            ev[i].record()
        fn()
    if ev:
        ev[steps].record()
    b.record()
    torch.cuda.synchronize()
    if ev:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return a.elapsed_time(b) / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="only the headline workload (no other configs, LM head or clock sample)")
    ap.add_argument("--extra", action="store_true", help="also time the whole d20 training step (20 blocks + head)")
    ap.add_argument("--adamw", action="store_true",
                    help="also time the AdamW step over the d20 model's parameter set (HBM-bound)")
    ap.add_argument("--window", type=int, default=0,
                    help="also time the d20 block with sliding-window attention of this many keys")
    ap.add_argument("--fp8", action="store_true",
                    help="also time FP8 quantization, FP8 GEMMs at the d20 Linear shapes and the FP8 d20 block step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 4 device copies of 256 MiB (known HBM bytes) to scale the HBM counters")
    ap.add_argument("--head-only", choices=sorted(HEAD_PROFILES),
                    help="time only this LM head (for profiling it alone) and print its figures")
    ap.add_argument("--config-only", choices=["gpt2_block", "gpt2_124m_step", "d20_val_bpb"],
                    help="time only this other configuration (for profiling it alone) and print its figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (data-parallel sharding "
              "would sit above it); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_only_gpt_bf16_amd import binding as B
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import BlockRunner

    if args.copy_calibration:
        # each copy reads 256 MiB and writes 256 MiB of HBM
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.head_only:
        print(json.dumps({"lm_head": lm_head_workloads(args, only=args.head_only)}), flush=True)
        return
    if args.config_only:
        print(json.dumps({"configs": config_workloads(args, only=args.config_only)}), flush=True)
        return

    w = synth.D20_BLOCK
    cfg = w.cfg
    x, dy, p = synth.make_block_inputs(w)
    r = BlockRunner(cfg, w.B, w.T, x, dy, p)
    torch.cuda.synchronize()
    per = []
    ms = time_steps(r.step, args.steps, args.warmup, per)
    per.sort()
    flops = block_flops(w.B, w.T, cfg.n_embd, cfg.n_head)
    tok_s = w.B * w.T / (ms * 1e-3)

    # traced pass over the same number of steps: per call-site kernel times
    B.gpt_trace_begin(64 * args.steps)
    for _ in range(args.steps):
        r.step()
    torch.cuda.synchronize()
    trace = B.gpt_trace_end()
    sites = {}
    for name, (n, us) in trace.items():
        bound, work = site_work(name, w.B, w.T, cfg.n_embd, cfg.n_head)
        avg = us / n
        e = {"launches_per_step": n / args.steps, "avg_us": round(avg, 2), "share": 0.0}
        if bound:
            e["bound"] = bound
            e["frac"] = (work / (avg * 1e-6)) / (PEAK_BF16 if bound == "mfma" else PEAK_HBM)
            e["algorithmic"] = work
        tr = measured_traffic(name)
        if tr is not None:
            e["traffic"] = tr
        sites[name] = e
    total_us = sum(us for _, us in trace.values())
    for name, (n, us) in trace.items():
        sites[name]["share"] = round(us / total_us, 4)
    dom = max((k for k in trace if site_work(k, w.B, w.T, cfg.n_embd, cfg.n_head)[0]), key=lambda k: trace[k][1])
    bound, work = site_work(dom, w.B, w.T, cfg.n_embd, cfg.n_head)
    n, us = trace[dom]
    avg_s = us / n * 1e-6
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": work / avg_s / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": work / avg_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom)
    roof["kernel"] = dom
    roof["avg_us"] = round(us / n, 2)
    roof["work_per_launch"] = work

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "d20 block fwd+bwd (RMSNorm, RoPE, QK-norm, GELU MLP)", "batch": w.B, "seq_len": w.T,
                   "n_embd": cfg.n_embd, "n_head": cfg.n_head, "head_dim": cfg.head_dim},
        "mfma_frac": round(flops / (ms * 1e-3) / PEAK_BF16, 4),
        "step_ms_median": round(per[len(per) // 2], 4), "step_ms_min": round(per[0], 4),
        "flop_per_step": flops,
        "roofline": roof,
        "kernels": sites,
    }
    if not args.quick:
        out["gpu_clock_mhz"] = clock_during(r.step)
        del r
        torch.cuda.empty_cache()
        out["configs"] = config_workloads(args)
        out["lm_head"] = lm_head_workloads(args)
    if args.extra or args.adamw or args.window or args.fp8:
        out["extra"] = extra_workloads(args) if args.extra else {}
        if args.adamw:
            out["extra"]["adamw_d20_model"] = adamw_workload(args)
        if args.window:
            out["extra"][f"d20_block_window{args.window}"] = window_workload(args, args.window)
        if args.fp8:
            out["extra"]["fp8_d20_linears"] = fp8_workload(args)
            out["extra"]["fp8_d20_block"] = fp8_block_workload(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


def window_workload(args, window):
    """The d20 block fwd+bwd with sliding-window attention: query i attends
    to keys i - window + 1 .. i.  Useful attention work is 12 D FLOP per
    visible (query, key) pair and (batch, head): Q K^T and P V forward (4 D),
    dV, dP, dK and dQ backward (8 D); with a window that covers the sequence
    this is the causal block's 6 B H D T^2."""
    import torch
    from decoder_only_gpt_bf16_amd import binding as B
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import BlockRunner
    w = synth.scaled(synth.D20_BLOCK, window=window)
    cfg = w.cfg
    x, dy, p = synth.make_block_inputs(w)
    r = BlockRunner(cfg, w.B, w.T, x, dy, p)
    ms = time_steps(r.step, args.steps, args.warmup)
    B.gpt_trace_begin(64 * args.steps)
    for _ in range(args.steps):
        r.step()
    torch.cuda.synchronize()
    trace = B.gpt_trace_end()
    T, C, H = w.T, cfg.n_embd, cfg.n_head
    D = C // H
    pairs = sum(min(i + 1, window) for i in range(T))   # visible (query, key) pairs per (b, h)
    attn = 12.0 * w.B * H * D * pairs                    # 4 D (fwd) + 8 D (bwd) FLOP per pair
    flops = 72.0 * C * C * w.B * T + attn
    del r
    torch.cuda.empty_cache()
    return {"window": window, "ms": ms, "tokens_per_s": w.B * T / (ms * 1e-3),
            "mfma_frac": flops / (ms * 1e-3) / PEAK_BF16,
            "attn_us": {k: round(v[1] / v[0], 2) for k, v in trace.items() if k.startswith("attn")}}


PEAK_FP8 = 5.0e15        # MI355X dense fp8 MFMA


def fp8_block_workload(args):
    """The d20 block fwd+bwd with its four Linear layers as FP8 GEMMs
    (gpt_config.fp8: activations and weights E4M3, gradients E5M2, dynamic
    per-tensor scales), the same useful FLOPs as the bf16 step; priced
    against the bf16 peak like the headline (the FP8 share is its GEMMs)."""
    import torch
    from decoder_only_gpt_bf16_amd import binding as B
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import BlockRunner
    w = synth.scaled(synth.D20_BLOCK, fp8=True)
    cfg = w.cfg
    x, dy, p = synth.make_block_inputs(w)
    r = BlockRunner(cfg, w.B, w.T, x, dy, p)
    per = []
    ms = time_steps(r.step, args.steps, args.warmup, per)
    B.gpt_trace_begin(128 * args.steps)
    for _ in range(args.steps):
        r.step()
    torch.cuda.synchronize()
    trace = B.gpt_trace_end()
    f = block_flops(w.B, w.T, cfg.n_embd, cfg.n_head)
    del r
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1), "ms": round(ms, 4),
            "ms_median": round(sorted(per)[len(per) // 2], 4), "bf16_peak_frac": round(f / (ms * 1e-3) / PEAK_BF16, 4),
            "sites_us": {k: round(v[1] / v[0], 2) for k, v in trace.items()},
            "launches_per_step": {k: v[0] / args.steps for k, v in trace.items()}}


def fp8_workload(args):
    """FP8 GEMMs at the d20 block's Linear shapes (tokens 8192, C 1280), codes
    from quantizing bf16 activations and weights on the GPU; and the quantizer's
    HBM rate (2 bytes read twice and 1 byte written per element)."""
    import torch
    from decoder_only_gpt_bf16_amd import binding as B
    gen = torch.Generator(device="cuda").manual_seed(99)
    Nt, C = 8192, 1280
    shapes = {"qkv": (Nt, 3 * C, C), "fc": (Nt, 4 * C, C), "proj": (Nt, C, 4 * C), "out": (Nt, C, C)}
    res = {}
    ws = torch.empty(B.gpt_fp8_workspace_bytes(Nt * 4 * C), dtype=torch.uint8, device="cuda")
    for name, (M, N, K) in shapes.items():
        x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
        w = (0.02 * torch.randn((N, K), generator=gen, device="cuda")).to(torch.bfloat16)
        qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sa = torch.zeros(4, device="cuda")
        sb = torch.zeros(4, device="cuda")
        B.gpt_fp8_quantize(w, B.FP8_E4M3, qb, sb, ws)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        qms = time_steps(lambda: B.gpt_fp8_quantize(x, B.FP8_E4M3, qa, sa, ws), args.steps, args.warmup)
        gms = time_steps(lambda: B.gpt_fp8_gemm(qa, B.FP8_E4M3, sa, qb, B.FP8_E4M3, sb, out), args.steps, args.warmup)
        flop = 2.0 * M * N * K
        res[name] = {"M": M, "N": N, "K": K, "gemm_us": gms * 1e3, "tflops": flop / (gms * 1e-3) / 1e12,
                     "fp8_peak_frac": flop / (gms * 1e-3) / PEAK_FP8, "quant_us": qms * 1e3,
                     "quant_GBps": 5.0 * M * K / (qms * 1e-3) / 1e9}
        del x, w, qa, qb, out
    torch.cuda.empty_cache()
    return res


def adamw_workload(args):
    """AdamW + global-norm clip over the d20 model's parameters: 20 blocks of
    (w_qkv, w_o, w_fc, w_proj), token embedding and untied head [32768, 1280],
    fp32 state with a bf16 copy of every parameter.  Per element the step moves
    34 bytes (gradient read twice, for the norm and the update; param, m, v
    read and written; bf16 copy written)."""
    import torch
    from decoder_only_gpt_bf16_amd import binding as B
    from decoder_only_gpt_bf16_amd import synth
    cfg = synth.D20_BLOCK.cfg
    shapes = [s for _ in range(20) for _, s in synth.block_param_shapes(cfg)] + [(32768, cfg.n_embd)] * 2
    gen = torch.Generator(device="cuda").manual_seed(1234)
    ts = []
    for shp in shapes:
        ts.append({"param": 0.02 * torch.randn(shp, generator=gen, device="cuda"),
                   "grad": 1e-4 * torch.randn(shp, generator=gen, device="cuda"),
                   "m": torch.zeros(shp, device="cuda"), "v": torch.zeros(shp, device="cuda"),
                   "param_bf16": torch.empty(shp, dtype=torch.bfloat16, device="cuda"), "decay": True})
    n = sum(t["param"].numel() for t in ts)
    ws = torch.empty(B.gpt_adamw_workspace_bytes(ts), dtype=torch.uint8, device="cuda")
    norm = torch.zeros(4, device="cuda")
    it = [0]

    def step():
        it[0] += 1
        B.gpt_adamw_step(ts, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=it[0],
                         max_norm=1.0, grad_norm=norm, ws=ws)

    ms = time_steps(step, max(3, args.steps // 2), 2)
    byts = 34.0 * n
    res = {"params": n, "tensors": len(ts), "ms": ms, "bytes_per_step": byts,
           "achieved_GBps": byts / (ms * 1e-3) / 1e9, "hbm_frac": byts / (ms * 1e-3) / PEAK_HBM}
    del ts, ws
    torch.cuda.empty_cache()
    return res


def config_workloads(args, only=None):
    """The other configurations at their full sizes: the GPT-2 124M block
    fwd+bwd (B 8, T 1024), the 12-layer GPT-2 124M training step (B 16,
    T 1024, tied head V 50304) and the 20-layer d20 val-bpb evaluation (B 8,
    T 2048, untied head V 32768, forward only).  Useful FLOPs: 6 per
    parameter-FLOP of the Linear layers and the head, causal attention on the
    lower triangle."""
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import BlockRunner
    res = {}
    want = lambda w: only is None or w.name == only  # noqa: E731
    w = synth.GPT2_BLOCK
    if want(w):
        x, dy, p = synth.make_block_inputs(w)
        r = BlockRunner(w.cfg, w.B, w.T, x, dy, p)
        per = []
        ms = time_steps(r.step, args.steps, args.warmup, per)
        f = block_flops(w.B, w.T, w.cfg.n_embd, w.cfg.n_head)
        res[w.name] = {"tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1), "ms": round(ms, 4),
                       "ms_median": round(sorted(per)[len(per) // 2], 4),
                       "mfma_frac": round(f / (ms * 1e-3) / PEAK_BF16, 4), "flop_per_step": f}
        del r
    w = synth.GPT2_STEP
    if want(w):
        res.update(_gpt2_step(args, w))
    w = synth.D20_EVAL
    if want(w):
        res.update(_d20_eval(args, w))
    return res


def _gpt2_step(args, w):
    import torch
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import ModelRunner
    res = {}
    ids, y, P, tb = synth.make_model_inputs(w)
    m = ModelRunner(w.cfg, w.B, w.T, P, tb)
    m.set_batch(ids, y)
    per = []
    ms = time_steps(m.train_step, 5, 2, per)
    C, L, V, N = w.cfg.n_embd, w.cfg.n_layer, w.cfg.vocab_size, w.B * w.T
    f = L * block_flops(w.B, w.T, C, w.cfg.n_head) + 6.0 * N * C * V
    res[w.name] = {"tokens_per_s": round(N / (ms * 1e-3), 1), "ms": round(ms, 3),
                   "ms_median": round(sorted(per)[len(per) // 2], 3), "mfma_frac": round(f / (ms * 1e-3) / PEAK_BF16, 4),
                   "flop_per_step": f, "loss": m.loss.item()}
    del m, P
    torch.cuda.empty_cache()
    return res


def _d20_eval(args, w):
    import torch
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import ModelRunner
    res = {}
    ids, y, P, tb = synth.make_model_inputs(w)
    m = ModelRunner(w.cfg, w.B, w.T, P, tb, train=False)
    m.set_batch(ids, y)
    per = []
    ms = time_steps(m.eval_step, 5, 2, per)
    C, L, V, N, T = w.cfg.n_embd, w.cfg.n_layer, w.cfg.vocab_size, w.B * w.T, w.T
    f = L * (2 * 12 * C * C * N + 2 * w.B * w.cfg.n_head * (C // w.cfg.n_head) * T * T) + 2.0 * N * C * V
    m.sum_nats.zero_()
    m.sum_bytes.zero_()
    m.eval_step()
    res[w.name] = {"tokens_per_s": round(N / (ms * 1e-3), 1), "ms": round(ms, 3),
                   "ms_median": round(sorted(per)[len(per) // 2], 3), "mfma_frac": round(f / (ms * 1e-3) / PEAK_BF16, 4),
                   "flop_per_step": f, "bpb": m.sum_nats.item() / (math.log(2) * m.sum_bytes.item())}
    del m, P
    torch.cuda.empty_cache()
    return res


# LM-head call sites: algorithmic work per launch (N tokens, C width, Vc
# columns of the launch's vocabulary chunk)
def head_site_work(name, N, C, Vc, P):
    if name in ("xent_stats_gemm", "xent_grad_gemm", "xent_dh_gemm", "xent_dw_gemm"):
        return "mfma", 2.0 * N * C * Vc
    if name == "xent_finish":
        # per row: P (max, sum exp) partials read, target logit read; lse, nats written
        return "hbm", N * (8.0 * P + 12.0)
    if name == "xent_dh_convert":
        return "hbm", N * C * (4.0 + 2.0)
    return None, None


def lm_head_workloads(args, only=None):
    """The vocabulary-chunked LM head with softmax cross-entropy at the two
    full-size heads: the GPT-2 124M step (N 16384, C 768, tied V 50304:
    forward + backward: statistics, logit gradient, dh and dW per chunk of
    8192 columns) and the d20 evaluation (N 16384, C 1280, V 32768: forward
    only).  The softmax statistics ride in the logit GEMM's epilogue, so no
    logit chunk is written to HBM; each call site is timed with hipEvents on
    the library's stream and priced against MFMA (its GEMM FLOPs) or HBM
    (the bytes it must move)."""
    import numpy as np
    import torch
    from decoder_only_gpt_bf16_amd import binding as B
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import upload_i32, workspace
    res = {}
    gen = torch.Generator(device="cuda").manual_seed(7)
    for name, w, grad in (("gpt2_124m_step_head", synth.GPT2_STEP, True), ("d20_val_bpb_head", synth.D20_EVAL, False)):
        if only is not None and name != only:
            continue
        cfg, N = w.cfg, w.B * w.T
        C, V = cfg.n_embd, cfg.vocab_size
        c = B.make_config(cfg)
        ws = workspace(c, w.B, w.T)
        h = torch.randn((N, C), generator=gen, device="cuda").to(torch.bfloat16)
        W = (0.02 * torch.randn((V, C), generator=gen, device="cuda")).to(torch.bfloat16)
        tgt = upload_i32(np.random.default_rng(5).integers(0, V, N))
        loss = torch.zeros(1, device="cuda")
        nats = torch.zeros(N, device="cuda")
        dh = torch.empty((N, C), dtype=torch.bfloat16, device="cuda") if grad else None
        dW = torch.empty((V, C), dtype=torch.float32, device="cuda") if grad else None
        call = lambda: B.lm_head_xent_fwd_bwd(c, N, h, W, tgt, 1.0 / N, loss, nats, dh, dW, 0, ws)  # noqa: E731
        steps = max(5, args.steps // 5)
        ms = time_steps(call, steps, 2)
        B.gpt_trace_begin(64 * steps)
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        trace = B.gpt_trace_end()
        Vc = min(V, 8192)
        nchunk = -(-V // Vc)
        P = sum(4 * -(-min(Vc, V - i * Vc) // 256) for i in range(nchunk))
        sites = {}
        for site, (n, us) in trace.items():
            avg = us / n
            e = {"launches_per_call": n / steps, "avg_us": round(avg, 2)}
            bound, work = head_site_work(site, N, C, Vc, P)
            if bound:
                e["bound"] = bound
                e["frac"] = round(work / (avg * 1e-6) / (PEAK_BF16 if bound == "mfma" else PEAK_HBM), 4)
                tr = measured_traffic(site, HEAD_PROFILES[name], HEAD_SITE_KERNEL)
                if tr is not None:
                    e["traffic"] = tr
            sites[site] = e
        flops = (6.0 if grad else 2.0) * N * C * V
        res[name] = {"N": N, "C": C, "V": V, "fwd_bwd": grad, "ms": round(ms, 4),
                     "mfma_frac": round(flops / (ms * 1e-3) / PEAK_BF16, 4),
                     # bytes a separate softmax-xent pass over bf16 logit chunks would
                     # read (and write, for the gradient); none of it exists here
                     "unfused_chunk_bytes": (3 if grad else 1) * 2.0 * N * V,
                     "sites": sites}
        del h, W, dh, dW, ws
        torch.cuda.empty_cache()
    return res


def clock_during(fn, seconds=1.5):
    """Shader clock (MHz) sampled from amd-smi while fn runs back to back on
    the GPU; None when amd-smi is not usable."""
    import subprocess
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                out = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True,
                                     timeout=5).stdout
                samples.append(_gfx_clock(json.loads(out)))
            except Exception:
                samples.append(None)
                return

    t = threading.Thread(target=sample, daemon=True)
    t0 = time.time()
    t.start()
    while time.time() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stop.set()
    t.join(timeout=10)
    vals = [v for v in samples if v]
    return {"mhz": vals, "source": "amd-smi metric -c, sampled during back-to-back steps"} if vals else None


def _gfx_clock(js):
    """Mean current GFX clock (MHz) over the first GPU's XCDs (amd-smi's
    gfx_0 .. gfx_7 entries), or None."""
    vals = []

    def walk(o):
        if isinstance(o, dict):
            for k, v in o.items():
                if k.lower().startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict):
                    try:
                        vals.append(float(v["clk"]["value"]))
                    except (KeyError, TypeError, ValueError):
                        pass
                else:
                    walk(v)
        elif isinstance(o, list) and o:
            walk(o[0])
    walk(js)
    return sum(vals) / len(vals) if vals else None


def extra_workloads(args):
    """The whole d20 training step at the block's shape: 20 blocks, untied
    head (V 32768), B 4, T 2048, fwd + bwd with the vocabulary-chunked loss."""
    import torch
    from decoder_only_gpt_bf16_amd import synth
    from decoder_only_gpt_bf16_amd.model import ModelRunner
    res = {}
    w = dataclasses.replace(synth.D20_EVAL, name="d20_train_step", B=4, kind="step")
    ids, y, P, tb = synth.make_model_inputs(w)
    m = ModelRunner(w.cfg, w.B, w.T, P, tb)
    m.set_batch(ids, y)
    ms = time_steps(m.train_step, max(3, args.steps // 4), 2)
    C, L, V, N = w.cfg.n_embd, w.cfg.n_layer, w.cfg.vocab_size, w.B * w.T
    f = L * block_flops(w.B, w.T, C, w.cfg.n_head) + 6.0 * N * C * V
    res[w.name] = {"tokens_per_s": N / (ms * 1e-3), "ms": ms, "mfma_frac": f / (ms * 1e-3) / PEAK_BF16,
                   "loss": m.loss.item()}
    del m, P
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
