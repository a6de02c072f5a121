#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's Transformer-block share on one MI355X.

A step is one call of the path's entry point over one batch of synthetic
input already resident in HBM.  The default workload is the full pre-LN block
at the 175B layer shape (h=12288, 96 heads of 128, F=49152, 8 sequences of
2048 tokens) with all 8 tensor-parallel ranks' shares run in turn on this GPU
(tp_block_shard: LayerNorm, per-rank QKV projection, causal attention, W_o
partial, partial sum + residual, LayerNorm, per-rank MLP shard, partial sum +
residual).  Throughput is matrix TFLOP/s of the whole step (ranks run one
after another, so this is also the per-shard rate).

Besides the one JSON line the run reports, in the same line:
  roofline      the dominant kernel (the column-parallel GEMM with the fused
                GeLU epilogue, at its in-block shape) timed per launch with
                HIP events on the stream it runs on, against the bf16 MFMA peak;
  cpu_baseline  the fp64 oracle timed on the host on a bounded sample of the
                same workload.

Modes for profiler runs: --mode kernel launches only the dominant kernel,
--mode copy only a plain device copy of a known size (counter calibration).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s per TP shard (bf16) and % of MI355X dense bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gelu_h12288_f6144_traffic.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "transformer_tensor_shard_amd", "csrc", "gemm_bf16.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken on another kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_bf16.hip sha256[:16]") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def event_time(fn, reps, stream):
    """Average ms of fn() over reps launches, bracketed by HIP events."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return sum(ts) / len(ts), ts


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="block_bf16_h12288_tp8")
    ap.add_argument("--mode", default="step", choices=["step", "kernel", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768,
                    help="tokens of sequence 0 the oracle computes for the CPU baseline")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share: the tensor-parallel ranks are emulated one "
              "after another on a single MI355X, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import workloads as wl
    import transformer_tensor_shard_amd as tts

    if args.workload not in wl.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; one of {sorted(wl.WORKLOADS)}")
    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    tts.lib()

    if args.mode == "copy":
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy of {COPY_BYTES} bytes x {args.warmup + args.steps} done")
        return

    if args.mode == "kernel":
        # only the dominant kernel's operands: the token activations and rank
        # 0's column-parallel weight, at the shape the step uses
        if w.kind == "block":
            X_cpu = wl.block_input(w)
            A_cpu = wl.block_rank_weights(w, 0)[2]
        elif w.kind == "mlp":
            X_cpu, A_cpu, _ = wl.mlp_inputs(w)
        else:
            X_cpu, A_cpu, _ = wl.attn_inputs(w)
        X_k, A_k = X_cpu.to(dev), A_cpu.to(dev)
        y_k = torch.empty(X_k.shape[0], A_k.shape[1], dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup + args.steps):
            tts.tp_linear(X_k, A_k, gelu=True, out=y_k)
        torch.cuda.synchronize()
        log(f"kernel mode: {args.warmup + args.steps} launches of the GeLU GEMM "
            f"[{X_k.shape[0]}x{X_k.shape[1]}]x[{A_k.shape[0]}x{A_k.shape[1]}] done")
        return

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    log(f"generating {w.name} inputs on the host")
    if w.kind == "block":
        x_cpu = wl.block_input(w)
        w_cpu = [wl.block_rank_weights(w, r) for r in range(w.P)]
        x = x_cpu.to(dev)
        Wqkv = [t[0].to(dev) for t in w_cpu]
        Wo = [t[1].to(dev) for t in w_cpu]
        A = [t[2].to(dev) for t in w_cpu]
        B = [t[3].to(dev) for t in w_cpu]
        M, h, f = w.M, w.h, w.f
        out = torch.empty(M, h, dtype=torch.float32, device=dev)
        ws = torch.empty(tts.tp_block_shard_workspace(w.b, w.s, h, w.H, w.d, w.F, w.P),
                         dtype=torch.uint8, device=dev)

        def step():
            tts.tp_block_shard(x, Wqkv, Wo, A, B, w.b, w.s, w.H, w.d, out=out, ws=ws)
        X_k, A_k = x, A[0]
    elif w.kind == "mlp":
        X_cpu, A_cpu, B_cpu = wl.mlp_inputs(w)
        x, A0, B0 = X_cpu.to(dev), A_cpu.to(dev), B_cpu.to(dev)
        M, h, f = w.M, w.h, A_cpu.shape[1]
        out = torch.empty(M, h, dtype=torch.float32, device=dev)
        ws = torch.empty(tts.tp_mlp_shard_workspace(M, f, x.dtype), dtype=torch.uint8, device=dev)

        def step():
            tts.tp_mlp_shard(x, A0, B0, out=out, ws=ws)
        X_k, A_k = x, A0
    else:
        X_cpu, Wqkv_cpu, Wo_cpu = wl.attn_inputs(w)
        x, Wqkv0, Wo0 = X_cpu.to(dev), Wqkv_cpu.to(dev), Wo_cpu.to(dev)
        M, h = w.M, w.h
        f = w.F // w.P if w.F else 3 * w.Hl * w.d
        out = torch.empty(M, h, dtype=torch.float32, device=dev)
        ws = torch.empty(tts.tp_attn_shard_workspace(w.b, w.s, w.Hl, w.d), dtype=torch.uint8,
                         device=dev)

        def step():
            tts.tp_attn_shard(x, Wqkv0, Wo0, w.b, w.s, w.Hl, w.d, True, out=out, ws=ws)
        X_k, A_k = x, Wqkv0
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    # dominant kernel: column GEMM + fused GeLU, bf16 out, at [M,h] x [h,f]
    kf = A_k.shape[1]
    y_k = torch.empty(M, kf, dtype=torch.bfloat16, device=dev)

    def kernel():
        tts.tp_linear(X_k, A_k, gelu=True, out=y_k)

    # ---------------------------------------------------------------- timing
    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} step(s)")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.time()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.time() - wall0
    ms = start.elapsed_time(end) / args.steps
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {tflops:.1f} TFLOP/s (wall {wall:.2f} s)")

    kern_ms, kern_all = event_time(kernel, max(args.steps, 5), stream)
    kern_flops = 2 * M * h * kf
    kern_tflops = kern_flops / (kern_ms * 1e-3) / 1e12
    traffic = measured_traffic()
    log(f"dominant kernel: {kern_ms:.3f} ms/launch, {kern_tflops:.1f} TFLOP/s")

    components = {}
    if w.kind == "block":
        xn = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
        part = torch.empty(M, h, dtype=torch.float32, device=dev)
        parts = torch.empty(w.P, M, h, dtype=torch.float32, device=dev)
        aws = torch.empty(tts.tp_attn_shard_workspace(w.b, w.s, w.Hl, w.d), dtype=torch.uint8,
                          device=dev)
        mws = torch.empty(tts.tp_mlp_shard_workspace(M, f), dtype=torch.uint8, device=dev)
        att = w.attn_flops_rank()
        qkv_buf = torch.empty(M, 3 * w.Hl * w.d, dtype=torch.bfloat16, device=dev)
        o_buf = torch.empty(M, w.Hl * w.d, dtype=torch.bfloat16, device=dev)
        items = {
            "layernorm": (lambda: tts.tp_layernorm(x, out=xn), None, 2 * M * h * 2),
            "attn_shard_rank": (lambda: tts.tp_attn_shard(x, Wqkv[0], Wo[0], w.b, w.s, w.Hl,
                                                          w.d, True, out=part, ws=aws),
                                att["total"], None),
            "qkv_gemm": (lambda: tts.tp_linear(x, Wqkv[0], out=qkv_buf), att["qkv"], None),
            "attention_core": (lambda: tts.tp_attention_core(qkv_buf, w.b, w.s, w.Hl, w.d, True,
                                                             out=o_buf), att["core"], None),
            "wo_gemm": (lambda: tts.tp_linear(o_buf, Wo[0], out=part), att["wo"], None),
            "mlp_shard_rank": (lambda: tts.tp_mlp_shard(xn, A[0], B[0], out=part, ws=mws),
                               w.mlp_flops_rank(), None),
            "partial_sum": (lambda: tts.tp_partial_sum(parts, None, x, out=part), None,
                            (w.P * 4 + 2 + 4) * M * h),
        }
        for name, (fn, fl, by) in items.items():
            fn()
            t, _ = event_time(fn, 3, stream)
            c = {"ms": round(t, 4)}
            if fl:
                c["tflops"] = round(fl / (t * 1e-3) / 1e12, 1)
                c["pct_peak"] = round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)
            if by:
                c["gbs"] = round(by / (t * 1e-3) / 1e9, 1)
                c["pct_hbm"] = round(100 * by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)
            components[name] = c
            log(f"component {name}: {c}")

    # ---------------------------------------------------------------- oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_rows, locals())

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "tokens": w.M, "h": w.h,
                   "heads": w.H, "head_dim": w.d if w.H else None, "ffn": w.F, "tp": w.P,
                   "ranks_emulated": w.P if w.all_ranks else 1, "flops_per_step": flops,
                   "parallelism": "tp%d emulated on 1 GPU" % w.P},
        "roofline": {
            "kernel": "gemm_bf16_kernel<bf16 out, GeLU> [%dx%d]x[%dx%d]" % (M, h, h, kf),
            "bound": "mfma",
            "achieved": round(kern_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": kern_flops,
            "avg_launch_ms": round(kern_ms, 4),
            "launches_timed": len(kern_all),
        },
        "cpu_baseline": cpu,
        "components": components,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(w, rows_req, env):
    """The fp64 oracle, as it stands, on the first tokens of sequence 0."""
    import numpy as np
    import oracle
    from synth import workloads as wl

    if w.kind == "block":
        R = min(rows_req, w.s)
        rows = np.arange(R)
        log(f"oracle: block rows 0..{R - 1} of sequence 0 (all {w.P} ranks)")
        x_cpu, w_cpu = env["x_cpu"], env["w_cpu"]
        t0 = time.time()
        oracle.block_rows(x_cpu, w.b, w.s, [t[0] for t in w_cpu], [t[1] for t in w_cpu],
                          [t[2] for t in w_cpu], [t[3] for t in w_cpu], w.H, w.d, rows=rows)
        dt = time.time() - t0
        HD = w.Hl * w.d
        fl = w.P * (2 * R * w.h * 3 * HD + 4 * HD * R * (R + 1) // 2 + 2 * R * HD * w.h
                    + 4 * R * w.h * w.f)
        sample = (f"tokens 0..{R - 1} of sequence 0 through the whole block, all {w.P} ranks "
                  f"(LN, QKV, causal attention, W_o, partial sums, MLP); {fl / 1e12:.3f} TFLOP")
    elif w.kind == "mlp":
        R = min(rows_req, w.M)
        X_cpu, A_cpu, B_cpu = env["X_cpu"], env["A_cpu"], env["B_cpu"]
        log(f"oracle: MLP shard rows 0..{R - 1}")
        t0 = time.time()
        oracle.mlp_shard(X_cpu[:R], A_cpu, B_cpu)
        dt = time.time() - t0
        fl = 4 * R * w.h * A_cpu.shape[1]
        sample = f"rows 0..{R - 1} of the MLP shard; {fl / 1e12:.3f} TFLOP"
    else:
        R = min(rows_req, w.s)
        X_cpu, Wqkv_cpu, Wo_cpu = env["X_cpu"], env["Wqkv_cpu"], env["Wo_cpu"]
        log(f"oracle: attention shard rows 0..{R - 1} of sequence 0")
        t0 = time.time()
        oracle.attn_shard_rows(X_cpu, w.b, w.s, Wqkv_cpu, Wo_cpu, w.Hl, w.d, True,
                               np.arange(R))
        dt = time.time() - t0
        HD = w.Hl * w.d
        fl = 2 * R * w.h * 3 * HD + 4 * HD * R * (R + 1) // 2 + 2 * R * HD * w.h
        sample = f"tokens 0..{R - 1} of sequence 0 of the attention shard; {fl / 1e12:.3f} TFLOP"
    log(f"oracle: {dt:.1f} s")
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s",
            "cores": max(oracle.num_threads(), blas_threads()), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2),
            "note": "fp64; matmuls via the host BLAS, other steps plain C loops"}


if __name__ == "__main__":
    main()
