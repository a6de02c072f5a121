#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's Transformer-block share on one MI355X.

A step is one call of the path's entry point over one batch of synthetic
input already resident in HBM.  The default workload is the full pre-LN block
at the 175B layer shape (h=12288, 96 heads of 128, F=49152, 8 sequences of
2048 tokens) with all 8 tensor-parallel ranks' shares run in turn on this GPU
(tp_block_shard: LayerNorm, per-rank QKV projection, causal attention, W_o
partial, partial sum + residual fused with the second LayerNorm, per-rank MLP
shard, partial sum + residual; each step one launch over all ranks).
Throughput is matrix TFLOP/s of the whole step; all ranks' shares run on this
one GPU, so this is also the per-shard rate.

Besides the one JSON line the run reports, in the same line:
  roofline      the dominant kernel (the column-parallel GEMM with the fused
                GeLU epilogue, launched as the step launches it: for the block,
                one grouped launch over all 8 ranks) timed per launch with HIP
                events on the stream it runs on, against the bf16 MFMA peak;
  cpu_baseline  the fp64 oracle timed on the host on a bounded sample of the
                same workload;
  calibration   the throughput of a register-only MFMA loop on this GPU (the
                matrix cores' ceiling under the current clock and power
                limits) and of the vendor GEMM at the dominant kernel's shape;
  training      (block workload) rank 0's MLP-share and attention-share
                backward at the same shape, timed with HIP events.

--workload mlp_bwd_bf16_h12288_tp8 measures that backward as its own step
(dY, dB_i, dA_i, da_i and the dX_i partial of one rank at the 175B layer
shape), with the weight-gradient product X^T·dY as its dominant kernel;
--workload attn_bwd_bf16_h12288_tp8 the attention share's backward (dO,
dW_o,i, the attention-core backward, dW_qkv,i, dX_i) with its grouped
weight-gradient launch as its dominant kernel; --workload vocab_bf16_h12288_tp8
the vocab-parallel ends of all 8 ranks (embedding lookup and partial sum, the
stable cross-entropy) with the grouped logits GEMM as its dominant kernel;
--workload kvsplit_bf16_h4096_tp4 the K/V-split attention of 4 ranks, HBM bound
as a whole: each of its steps is timed on its own with the 256 MB last-level
cache flushed before it (a 1 GiB write outside the events), and so are the
HBM-bound components of every workload (LayerNorm, partial sums, embedding).

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
# committed counter summaries of each workload's dominant kernel (HBM bytes per launch)
TRAFFIC_FILES = {
    "block_bf16_h12288_tp8": os.path.join(ROOT, "profiles", "gemm_gelu_h12288_f6144_traffic.txt"),
    "mlp_bwd_bf16_h12288_tp8": os.path.join(ROOT, "profiles",
                                            "gemm_tn_wgrad_h12288_f6144_traffic.txt"),
    "attn_bwd_bf16_h12288_tp8": os.path.join(ROOT, "profiles",
                                             "gemm_tn_wgrad_attn_h12288_hd1536_traffic.txt"),
    "vocab_bf16_h12288_tp8": os.path.join(ROOT, "profiles", "gemm_ce_h12288_v51200_traffic.txt"),
}
TRAFFIC_FILE = TRAFFIC_FILES["block_bf16_h12288_tp8"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "transformer_tensor_shard_amd", "csrc", "gemm_bf16.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_counters(path=TRAFFIC_FILE, source_hash=None):
    """The committed counter summary of the dominant kernel as {key: float}
    (HBM bytes per launch, shader clock, MFMA-busy fraction), or None when it
    is missing or was taken on another kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("gemm_bf16_hip_sha256_16") != (source_hash or kernel_source_hash()):
        return None
    out = {}
    for k, v in kv.items():
        try:
            out[k] = float(v)
        except ValueError:
            pass
    return out


def measured_traffic(path=TRAFFIC_FILE, source_hash=None):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken on another kernel source."""
    c = measured_counters(path, source_hash)
    return c.get("hbm_bytes_per_launch") if c else None


class CacheFlush:
    """Writes a 1 GiB device buffer: run between the timed launches of an
    HBM-bound kernel (outside their events), it evicts the 256 MB last-level
    cache, so that no launch reads what the one before left there."""
    BYTES = 1 << 30

    def __init__(self, torch, dev):
        self.buf = torch.empty(self.BYTES // 4, dtype=torch.float32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(float(self.n & 1))


def component_time(fn, stream, flush=None):
    """Average ms of fn() alone: after a warm-up of about 0.05 s, over enough
    launches for about 0.1 s (3 to 500); with `flush`, the cache is flushed
    before every launch (outside the timing)."""
    import torch
    t1, _ = event_time(fn, 1, stream, flush)
    n = int(min(500, max(3, 0.05e3 / max(t1, 1e-3))))
    event_time(fn, n, stream, flush)
    return event_time(fn, int(min(500, max(3, 0.1e3 / max(t1, 1e-3)))), stream, flush)


def event_time(fn, reps, stream, flush=None):
    """Average ms of fn() over reps launches, bracketed by HIP events (and
    preceded by `flush()`, outside the events, when given)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        if flush is not None:
            flush()
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


def hbm_copy_calibration(torch, dev, stream):
    """A plain device copy of COPY_BYTES measured in this run: the practical
    HBM ceiling for a kernel that reads and writes."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms, _ = event_time(lambda: dst.copy_(src), 5, stream)
    return {"gbs": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1), "bytes": 2 * COPY_BYTES,
            "kernel": "torch copy_ of a 1 GiB f32 buffer"}


def calibration(tts, torch, X, W, stream, trans_a=False):
    """Two reference points measured on this GPU in this run, for reading the
    roofline fraction: the throughput of a register-only MFMA loop (the
    matrix cores' ceiling under the current clock and power limits), and the
    vendor GEMM (torch.mm, i.e. hipBLASLt) at the dominant kernel's per-rank
    shape and layout (X^T·W when trans_a)."""
    out = torch.empty(256 * 512, dtype=torch.float32, device=X.device)
    for _ in range(3):
        tts.tp_probe_mfma(256, 200, out=out)
    probe_flops = 256 * 8 * 32 * 200 * 16384
    ms, _ = event_time(lambda: tts.tp_probe_mfma(256, 200, out=out), 5, stream)
    Xop = X.t() if trans_a else X
    Y = torch.empty(Xop.shape[0], W.shape[1], dtype=torch.bfloat16, device=X.device)
    for _ in range(2):
        torch.mm(Xop, W, out=Y)
    ms_mm, _ = event_time(lambda: torch.mm(Xop, W, out=Y), 5, stream)
    mm_flops = 2 * Xop.shape[0] * Xop.shape[1] * W.shape[1]
    return {
        "mfma_only": {"tflops": round(probe_flops / (ms * 1e-3) / 1e12, 1),
                      "frac_of_peak": round(probe_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "kernel": "tp_probe_mfma: register-only MFMA 16x16x32 bf16, 2 waves/SIMD"},
        "vendor_gemm": {"tflops": round(mm_flops / (ms_mm * 1e-3) / 1e12, 1),
                        "kernel": "torch.mm bf16 %s[%dx%d]x[%dx%d] (hipBLASLt)" % (
                            "transposed A " if trans_a else "", Xop.shape[0], Xop.shape[1],
                            W.shape[0], W.shape[1])},
    }


def dominant_operands_cpu(w, wl):
    """Host copies of the dominant kernel's operands: the activations and the
    weight(s) of the column-parallel product the step spends the most time in."""
    if w.kind == "block":
        return wl.block_input(w), [wl.block_rank_weights(w, r)[2] for r in range(w.P)]
    if w.kind == "mlp":
        X, A, _ = wl.mlp_inputs(w)
        return X, [A]
    if w.kind == "mlp_bwd":
        # the weight-gradient products Y'^T·dZ and X^T·dY; the values of the
        # activations dY and Y' do not change their cost
        X, _, _, _, dZ = wl.mlp_bwd_inputs(w)
        dY = wl.normal((w.M, w.f), 1.0, w.seed, "preact", w.dtype)
        Yp = wl.normal((w.M, w.f), 1.0, w.seed, "partials", w.dtype)
        return X, [dY, Yp, dZ]
    if w.kind == "vocab":
        # the cross-entropy logits of all ranks: H and the ranks' tables
        _, targets, H, E = wl.vocab_inputs(w)
        Vr = w.V // w.P
        return H, [targets] + [E[r * Vr:(r + 1) * Vr].contiguous() for r in range(w.P)]
    if w.kind == "kvsplit":
        return wl.kvsplit_inputs(w), []
    if w.kind == "attn_bwd":
        # the weight-gradient products X^T·dqkv and O^T·dZ (values of the
        # activations dqkv and O do not change their cost)
        X, _, _, dZ = wl.attn_bwd_inputs(w)
        HD = w.Hl * w.d
        dqkv = wl.normal((w.M, 3 * HD), 1.0, w.seed, "preact", w.dtype)
        O = wl.normal((w.M, HD), 1.0, w.seed, "partials", w.dtype)
        return X, [dqkv, O, dZ]
    X, Wqkv, _ = wl.attn_inputs(w)
    return X, [Wqkv]


def dominant_kernel(w, tts, torch, X, Ws, dev):
    """(launch, algorithmic FLOPs per launch, name) of the step's dominant
    kernel, launched exactly as the step launches it: for the block, the
    column-parallel GEMM with the GeLU epilogue of all P ranks in one grouped
    launch; for the MLP shard its GeLU GEMM; for the attention shard its QKV
    projection."""
    M, K = X.shape
    if w.kind == "kvsplit":
        # the whole call: the partial-score GEMMs, the sum-and-softmax rows,
        # the e·V GEMMs and the normalisation; HBM bound (kvsplit_bytes)
        O = torch.empty(M, w.H * w.d, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(tts.tp_attention_kv_split_workspace(w.b, w.s, w.H, w.P, w.d),
                         dtype=torch.uint8, device=dev)

        def launch():
            tts.tp_attention_kv_split(X, w.b, w.s, w.H, w.P, w.d, True, out=O, ws=ws)
        name = ("tp_attention_kv_split: %d sequences x %d heads, s=%d, d=%d split over %d ranks "
                "(partial-score GEMMs, kv_softmax_kernel, e·V GEMMs, kv_normalize_kernel)"
                % (w.b, w.H, w.s, w.d, w.P))
        return launch, w.flops(), name
    if w.kind == "vocab":
        # the grouped logits GEMM of all ranks with the cross-entropy-statistics
        # epilogue, as tp_vocab_parallel_ce launches it (its per-rank statistics
        # and combine launches, a few tens of microseconds, are included)
        targets, Es = Ws[0], Ws[1:]
        ws = torch.empty(tts.tp_vocab_parallel_ce_workspace(M, Es[0].shape[0], len(Es)),
                         dtype=torch.uint8, device=dev)
        loss = torch.empty(M, dtype=torch.float32, device=dev)
        mean = torch.empty(1, dtype=torch.float32, device=dev)

        def launch():
            tts.tp_vocab_parallel_ce(X, Es, targets, loss=loss, loss_mean=mean, ws=ws)
        V = sum(E.shape[0] for E in Es)
        # the statistics epilogue takes the input-gradient layout's width rule,
        # 384 or 256 columns (it has no 192-column kernel)
        cols = tts.tp_gemm_tile_cols([(M, Es[0].shape[0])] * len(Es), K, trans_b=True)
        cols = 256 if cols == 192 else cols
        name = ("%s<NT, epi=ce_stats> (256x%d tiles) grouped over %d ranks, each [%dx%d]x[%dx%d]^T "
                "(+ statistics combine)" % ("gemm_bf16_w384_kernel" if cols == 384 else "gemm_bf16_kernel",
                                            cols, len(Es), M, K, Es[0].shape[0], K))
        return launch, 2 * M * K * V, name
    N = Ws[0].shape[1]
    if w.kind == "mlp_bwd":
        # dB_i = Y'^T·dZ [f, h] and dA_i = X^T·dY [h, f] in one grouped launch
        dY, Yp, dZ = Ws
        f, h = dY.shape[1], K
        dA = torch.empty(h, f, dtype=torch.float32, device=dev)
        dB = torch.empty(f, h, dtype=torch.float32, device=dev)

        def launch():
            tts.tp_matmul_grouped([Yp, X], [dZ, dY], trans_a=True, outs=[dB, dA])
        name = ("gemm_bf16_kernel<TN, f32 out> grouped: Y'^T·dZ [%dx%d]x[%dx%d] and "
                "X^T·dY [%dx%d]x[%dx%d]" % (f, M, M, h, h, M, M, f))
        return launch, 2 * (2 * M * h * f), name
    if w.kind == "attn_bwd":
        # dW_qkv,i = X^T·dqkv and dW_o,i = O^T·dZ in one grouped launch, with
        # the spare memory the backward gives it (its dO buffer, dead by then),
        # which lets the launch split its last wave of tiles over K
        dqkv, O, dZ = Ws
        h, n3, HD = K, dqkv.shape[1], O.shape[1]
        dWqkv = torch.empty(h, n3, dtype=torch.float32, device=dev)
        dWo = torch.empty(HD, h, dtype=torch.float32, device=dev)
        spare = torch.empty(M * HD * 2, dtype=torch.uint8, device=dev)

        def launch():
            tts.tp_matmul_grouped([X, O], [dqkv, dZ], trans_a=True, outs=[dWqkv, dWo], ws=spare)
        name = ("gemm_bf16_kernel<TN, f32 out> grouped: X^T·dqkv [%dx%d]x[%dx%d] and "
                "O^T·dZ [%dx%d]x[%dx%d] (+ the last wave's split-K sum)"
                % (h, M, M, n3, HD, M, M, h))
        return launch, 2 * M * h * n3 + 2 * M * HD * h, name
    gelu = w.kind != "attn"
    outs = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in Ws]
    if len(Ws) > 1:
        def launch():
            tts.tp_linear_batched([X] * len(Ws), Ws, gelu=gelu, outs=outs)
    else:
        def launch():
            tts.tp_linear(X, Ws[0], gelu=gelu, out=outs[0])
    cols = tts.tp_gemm_tile_cols([(M, N)] * len(Ws), K, epilogue="gelu" if gelu else "none")
    kern = "gemm_bf16_w384_kernel" if cols == 384 else "gemm_bf16_kernel"
    name = "%s<bf16 out, %s> (256x%d tiles) %s[%dx%d]x[%dx%d]" % (
        kern, "GeLU" if gelu else "no epilogue", cols,
        ("grouped over %d ranks, each " % len(Ws)) if len(Ws) > 1 else "", M, K, K, N)
    return launch, 2 * M * N * K * len(Ws), name


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 20 and about 0.25 s of steps, at most 2000)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: at least 3 and about 0.1 s of steps)")
    ap.add_argument("--workload", default="block_bf16_h12288_tp8")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the MLP-backward measurement added to the block line")
    ap.add_argument("--mode", default="step", choices=["step", "kernel", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="tokens the oracle computes for the CPU baseline (default: sized for "
                         "10-30 s on 16 host threads, or the whole workload where that is less)")
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

    if args.mode in ("copy", "kernel"):
        args.warmup = 1 if args.warmup is None else args.warmup
        args.steps = 3 if args.steps is None else args.steps
    if args.mode == "copy":
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy of {COPY_BYTES} bytes x {args.warmup + args.steps} done")
        return

    if args.mode == "kernel":
        # only the dominant kernel's operands, at the shape the step uses
        X_cpu, W_cpu = dominant_operands_cpu(w, wl)
        X_k = X_cpu.to(dev)
        W_k = [t.to(dev) for t in W_cpu]
        del X_cpu, W_cpu
        kernel, kern_flops, kern_name = dominant_kernel(w, tts, torch, X_k, W_k, dev)
        for _ in range(args.warmup + args.steps):
            kernel()
        torch.cuda.synchronize()
        log(f"kernel mode: {args.warmup + args.steps} launches of {kern_name} done")
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

        # the dominant kernel (the grouped GeLU GEMM) is timed inside every
        # timed step, by events the library records around its launch
        kev = []            # one pair per timed step, made once the step count is known

        def step(i=None):
            tts.tp_block_shard(x, Wqkv, Wo, A, B, w.b, w.s, w.H, w.d, out=out, ws=ws,
                               gelu_gemm_events=None if i is None else kev[i])
        X_k, W_k = x, A
    elif w.kind == "mlp":
        X_cpu, A_cpu, B_cpu = wl.mlp_inputs(w)
        x, A0, B0 = X_cpu.to(dev), A_cpu.to(dev), B_cpu.to(dev)
        M, h, f = w.M, w.h, A_cpu.shape[1]
        out = torch.empty(M, h, dtype=torch.float32, device=dev)
        ws = torch.empty(tts.tp_mlp_shard_workspace(M, f, x.dtype), dtype=torch.uint8, device=dev)

        def step(i=None):
            tts.tp_mlp_shard(x, A0, B0, out=out, ws=ws)
        X_k, W_k = x, [A0]
    elif w.kind == "mlp_bwd":
        X_cpu, A_cpu, B_cpu, a_cpu, dZ_cpu = wl.mlp_bwd_inputs(w)
        x, A0, B0, a0, dZ = (t.to(dev) for t in (X_cpu, A_cpu, B_cpu, a_cpu, dZ_cpu))
        M, h, f = w.M, w.h, w.f
        # the saved activations come from the training forward, outside the timed step
        _, Y0, Yp0 = tts.tp_mlp_shard_train_fwd(x, A0, B0, a0)
        bwd_out = dict(dX_out=torch.empty(M, h, dtype=torch.float32, device=dev),
                       dA_out=torch.empty(h, f, dtype=torch.float32, device=dev),
                       dB_out=torch.empty(f, h, dtype=torch.float32, device=dev),
                       da_out=torch.empty(f, dtype=torch.float32, device=dev),
                       ws=torch.empty(tts.tp_mlp_shard_backward_workspace(M, f),
                                      dtype=torch.uint8, device=dev))

        def step(i=None):
            tts.tp_mlp_shard_backward(x, A0, B0, Y0, Yp0, dZ, **bwd_out)
        dY0 = tts.tp_matmul(dZ, B0, trans_b=True, epilogue="gelu_bwd", aux=Y0,
                            out_dtype=torch.bfloat16)
        X_k, W_k = x, [dY0, Yp0, dZ]
    elif w.kind == "vocab":
        tokens_cpu, targets_cpu, H_cpu, E_cpu = wl.vocab_inputs(w)
        Vr = w.V // w.P
        tokens, targets, x = tokens_cpu.to(dev), targets_cpu.to(dev), H_cpu.to(dev)
        Es = [E_cpu[r * Vr:(r + 1) * Vr].contiguous().to(dev) for r in range(w.P)]
        M, h = w.M, w.h
        # bf16 partials: each token's row comes from exactly one rank and the
        # others contribute zeros, so the sum over ranks is exact in bf16 (the
        # model's activation dtype) and bit-identical to an f32 sum
        parts = torch.empty(w.P, M, h, dtype=torch.bfloat16, device=dev)
        emb = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
        loss = torch.empty(M, dtype=torch.float32, device=dev)
        mean = torch.empty(1, dtype=torch.float32, device=dev)
        ce_ws = torch.empty(tts.tp_vocab_parallel_ce_workspace(M, Vr, w.P), dtype=torch.uint8,
                            device=dev)

        def step(i=None):
            for r in range(w.P):
                tts.tp_vocab_embedding_shard(tokens, Es[r], r * Vr, out=parts[r])
            tts.tp_partial_sum(parts, out=emb)
            tts.tp_vocab_parallel_ce(x, Es, targets, loss=loss, loss_mean=mean, ws=ce_ws)
        X_k, W_k = x, [targets] + Es
    elif w.kind == "kvsplit":
        qkv_cpu = wl.kvsplit_inputs(w)
        qkv = qkv_cpu.to(dev)
        M, h = w.M, w.h
        O = torch.empty(M, w.H * w.d, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(tts.tp_attention_kv_split_workspace(w.b, w.s, w.H, w.P, w.d),
                         dtype=torch.uint8, device=dev)

        def step(i=None):
            tts.tp_attention_kv_split(qkv, w.b, w.s, w.H, w.P, w.d, True, out=O, ws=ws)
        X_k, W_k = qkv, []
    elif w.kind == "attn_bwd":
        X_cpu, Wqkv_cpu, Wo_cpu, dZ_cpu = wl.attn_bwd_inputs(w)
        x, Wqkv0, Wo0, dZ = (t.to(dev) for t in (X_cpu, Wqkv_cpu, Wo_cpu, dZ_cpu))
        M, h, HD = w.M, w.h, w.Hl * w.d
        f = 3 * HD
        # the saved activations come from the training forward, outside the timed step
        _, qkv0, O0, lse0 = tts.tp_attn_shard_train_fwd(x, Wqkv0, Wo0, w.b, w.s, w.Hl, w.d)
        bwd_out = dict(dX_out=torch.empty(M, h, dtype=torch.float32, device=dev),
                       dWqkv_out=torch.empty(h, 3 * HD, dtype=torch.float32, device=dev),
                       dWo_out=torch.empty(HD, h, dtype=torch.float32, device=dev),
                       ws=torch.empty(tts.tp_attn_shard_backward_workspace(w.b, w.s, w.Hl, w.d),
                                      dtype=torch.uint8, device=dev))

        def step(i=None):
            tts.tp_attn_shard_backward(x, Wqkv0, Wo0, qkv0, O0, lse0, dZ, w.b, w.s, w.Hl, w.d,
                                       **bwd_out)
        dO0 = tts.tp_matmul(dZ, Wo0, trans_b=True, out_dtype=torch.bfloat16)
        dqkv0 = tts.tp_attention_core_backward(qkv0, O0, dO0, lse0, w.b, w.s, w.Hl, w.d)
        X_k, W_k = x, [dqkv0, O0, dZ]
    else:
        X_cpu, Wqkv_cpu, Wo_cpu = wl.attn_inputs(w)
        x, Wqkv0, Wo0 = X_cpu.to(dev), Wqkv_cpu.to(dev), Wo_cpu.to(dev)
        M, h = w.M, w.h
        f = w.F // w.P if w.F else 3 * w.Hl * w.d
        out = torch.empty(M, h, dtype=torch.float32, device=dev)
        ws = torch.empty(tts.tp_attn_shard_workspace(w.b, w.s, w.Hl, w.d), dtype=torch.uint8,
                         device=dev)

        def step(i=None):
            tts.tp_attn_shard(x, Wqkv0, Wo0, w.b, w.s, w.Hl, w.d, True, out=out, ws=ws)
        X_k, W_k = x, [Wqkv0]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    kernel, kern_flops, kern_name = dominant_kernel(w, tts, torch, X_k, W_k, dev)
    # HBM-bound kernels and steps are timed with the last-level cache flushed
    # before each launch; the K/V split is HBM bound as a whole
    flush = CacheFlush(torch, dev)
    hbm_bound = w.kind == "kvsplit"

    # ---------------------------------------------------------------- timing
    # Short steps get more of both by default, so that the clocks have settled
    # and the mean covers a quarter second: the warm-up runs at least 3 steps
    # and 0.1 s, the timed region at least 20 steps and 0.25 s (at most 2000).
    auto_warm = args.warmup is None
    n_warm = 3 if auto_warm else args.warmup
    torch.cuda.synchronize()
    tw = time.time()
    done = 0
    while done < n_warm or (auto_warm and time.time() - tw < 0.1):
        step()
        done += 1
        if auto_warm:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    est = (time.time() - tw) / max(done, 1)
    args.warmup = done
    if args.steps is None:
        args.steps = int(min(2000, max(20, 0.25 / max(est, 1e-6))))
    log(f"warmup {args.warmup} step(s), {1000 * est:.3f} ms each")
    if w.kind == "block":
        kev.extend((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps))
    log(f"timing {args.steps} step(s)")
    torch.cuda.synchronize()
    wall0 = time.time()
    if hbm_bound:
        # each step bracketed by its own events, the last-level cache flushed
        # before it (outside the events): the mean of the steps' own times
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (a, b) in enumerate(evs):
            flush()
            a.record(stream)
            step(i)
            b.record(stream)
        torch.cuda.synchronize()
        per_step = sorted(a.elapsed_time(b) for a, b in evs)
        ms = sum(per_step) / args.steps
    else:
        # one event after every step: the whole region gives the mean, the
        # differences the per-step spread
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            step(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = evs[0].elapsed_time(evs[-1]) / args.steps
        per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    wall = time.time() - wall0
    step_stats = {"min": round(per_step[0], 4),
                  "median": round(per_step[len(per_step) // 2] if len(per_step) % 2
                                  else 0.5 * (per_step[len(per_step) // 2 - 1]
                                              + per_step[len(per_step) // 2]), 4),
                  "p90": round(per_step[min(len(per_step) - 1,
                                            int(math.ceil(0.9 * len(per_step))) - 1)], 4)}
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {tflops:.1f} TFLOP/s (wall {wall:.2f} s)")

    # the dominant kernel: its own launches inside the timed steps where the
    # step's entry point records them (the block), else separate launches
    iso_ms, iso_all = event_time(kernel, max(args.steps, 5), stream, flush if hbm_bound else None)
    if w.kind == "block":
        kern_all = [a.elapsed_time(b) for a, b in kev]
        kern_ms = sum(kern_all) / len(kern_all)
        kern_where = "inside the timed steps (events recorded by tp_block_shard_timed)"
    else:
        kern_ms, kern_all = iso_ms, iso_all
        kern_where = "separate launches after the timed steps"
    kern_tflops = kern_flops / (kern_ms * 1e-3) / 1e12
    counters = measured_counters(TRAFFIC_FILES[w.name]) if w.name in TRAFFIC_FILES else None
    traffic = counters.get("hbm_bytes_per_launch") if counters else None
    clock = counters.get("shader_clock_ghz") if counters else None
    log(f"dominant kernel: {kern_ms:.3f} ms/launch, {kern_tflops:.1f} TFLOP/s ({kern_where}; "
        f"separate launches {iso_ms:.3f} ms)")
    if w.kind == "kvsplit":
        calib = {"hbm_copy": hbm_copy_calibration(torch, dev, stream)}
    elif w.kind == "vocab":
        calib = calibration(tts, torch, X_k, W_k[1].t(), stream)
    else:
        calib = calibration(tts, torch, X_k, W_k[0], stream, trans_a=w.kind.endswith("_bwd"))
    log(f"calibration: {calib}")

    components = {}
    if w.kind == "block":
        P, HD = w.P, w.Hl * w.d
        xn = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
        x1 = torch.empty(M, h, dtype=torch.float32, device=dev)
        parts = torch.empty(P, M, h, dtype=torch.float32, device=dev)
        qkv_all = torch.empty(P * M, 3 * HD, dtype=torch.bfloat16, device=dev)
        o_all = torch.empty(P * M, HD, dtype=torch.bfloat16, device=dev)
        y_all = torch.empty(P * M, f, dtype=torch.bfloat16, device=dev)
        qkv_r = [qkv_all[r * M:(r + 1) * M] for r in range(P)]
        o_r = [o_all[r * M:(r + 1) * M] for r in range(P)]
        y_r = [y_all[r * M:(r + 1) * M] for r in range(P)]
        att = w.attn_flops_rank()
        # the launches tp_block_shard makes, one by one (all ranks per launch);
        # every rank's Q|K|V rows follow the previous rank's, so the attention
        # of all ranks is the attention of P*b sequences
        items = {
            "layernorm": (lambda: tts.tp_layernorm(x, out=xn), None, 2 * M * h * 2),
            "qkv_gemm_all_ranks": (lambda: tts.tp_linear_batched([x] * P, Wqkv, outs=qkv_r),
                                   P * att["qkv"], None),
            "attention_core_all_ranks": (lambda: tts.tp_attention_core(
                qkv_all, P * w.b, w.s, w.Hl, w.d, True, out=o_all), P * att["core"], None),
            "wo_gemm_all_ranks": (lambda: tts.tp_linear_batched(o_r, Wo, outs=list(parts)),
                                  P * att["wo"], None),
            "mlp_gelu_gemm_all_ranks": (lambda: tts.tp_linear_batched([xn] * P, A, gelu=True,
                                                                      outs=y_r),
                                        P * w.mlp_flops_rank() // 2, None),
            "mlp_row_gemm_all_ranks": (lambda: tts.tp_linear_batched(y_r, B, outs=list(parts)),
                                       P * w.mlp_flops_rank() // 2, None),
            "partial_sum_residual": (lambda: tts.tp_partial_sum(parts, None, x1, out=x1), None,
                                     (P * 4 + 4 + 4) * M * h),
        }
        for name, (fn, fl, by) in items.items():
            fn()
            t, _ = component_time(fn, stream, flush if by and not fl else None)
            c = {"ms": round(t, 4)}
            if fl:
                c["tflops"] = round(fl / (t * 1e-3) / 1e12, 1)
                c["pct_peak"] = round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)
            if by:
                c["gbs"] = round(by / (t * 1e-3) / 1e9, 1)
                c["pct_hbm"] = round(100 * by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)
            components[name] = c
            log(f"component {name}: {c}")
        del qkv_all, o_all, y_all, parts
    if w.kind in ("mlp", "attn"):
        # the launches of one shard call, one by one
        if w.kind == "mlp":
            Yc = torch.empty(M, f, dtype=torch.bfloat16, device=dev)
            items = {
                "gelu_gemm": (lambda: tts.tp_linear(x, A0, gelu=True, out=Yc), 2 * M * h * f),
                "row_gemm_f32_partial": (lambda: tts.tp_linear(Yc, B0, out=out), 2 * M * h * f),
            }
        else:
            HD = w.Hl * w.d
            att = w.attn_flops_rank()
            qkv_c = torch.empty(M, 3 * HD, dtype=torch.bfloat16, device=dev)
            o_c = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
            items = {
                "qkv_gemm": (lambda: tts.tp_linear(x, Wqkv0, out=qkv_c), att["qkv"]),
                "attention_core": (lambda: tts.tp_attention_core(qkv_c, w.b, w.s, w.Hl, w.d, True,
                                                                 out=o_c), att["core"]),
                "wo_gemm_f32_partial": (lambda: tts.tp_linear(o_c, Wo0, out=out), att["wo"]),
            }
        for name, (fn, fl) in items.items():
            fn()
            t, _ = component_time(fn, stream)
            c = {"ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 1),
                 "pct_peak": round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)}
            components[name] = c
            log(f"component {name}: {c}")
        del items
    if w.kind == "mlp_bwd":
        fl1 = 2 * M * h * f
        dYc = torch.empty(M, f, dtype=torch.bfloat16, device=dev)
        items = {
            "dY_gemm_nt_gelu_bwd": (lambda: tts.tp_matmul(dZ, B0, trans_b=True,
                                                          epilogue="gelu_bwd", aux=Y0, out=dYc),
                                    fl1, None),
            "dB_dA_gemm_tn_grouped": (lambda: tts.tp_matmul_grouped(
                [Yp0, x], [dZ, dYc], trans_a=True, outs=[bwd_out["dB_out"], bwd_out["dA_out"]]),
                2 * fl1, None),
            "dX_gemm_nt": (lambda: tts.tp_matmul(dYc, A0, trans_b=True, out=bwd_out["dX_out"]),
                           fl1, None),
        }
        for name, (fn, fl, by) in items.items():
            fn()
            t, _ = component_time(fn, stream, flush if by and not fl else None)
            c = {"ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 1),
                 "pct_peak": round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)}
            components[name] = c
            log(f"component {name}: {c}")
        del dYc

    if w.kind == "attn_bwd":
        Dws = torch.empty(w.b * w.Hl * w.s, dtype=torch.float32, device=dev)
        dqkv_c = torch.empty(M, 3 * HD, dtype=torch.bfloat16, device=dev)
        dO_c = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
        fl = w.attn_bwd_flops_rank()
        items = {
            "dO_gemm_nt": (lambda: tts.tp_matmul(dZ, Wo0, trans_b=True, out=dO_c), fl["wo"] // 2),
            "attention_core_backward": (lambda: tts.tp_attention_core_backward(
                qkv0, O0, dO_c, lse0, w.b, w.s, w.Hl, w.d, dqkv=dqkv_c, D_ws=Dws), fl["core"]),
            "dWqkv_dWo_gemm_tn_grouped": (lambda: tts.tp_matmul_grouped(
                [x, O0], [dqkv_c, dZ], trans_a=True,
                outs=[bwd_out["dWqkv_out"], bwd_out["dWo_out"]], ws=dO_c),
                (fl["qkv"] + fl["wo"]) // 2),
            "dX_gemm_nt": (lambda: tts.tp_matmul(dqkv_c, Wqkv0, trans_b=True,
                                                 out=bwd_out["dX_out"]), fl["qkv"] // 2),
        }
        for name, (fn, flc) in items.items():
            fn()
            t, _ = component_time(fn, stream)
            c = {"ms": round(t, 4), "tflops": round(flc / (t * 1e-3) / 1e12, 1),
                 "pct_peak": round(100 * flc / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)}
            components[name] = c
            log(f"component {name}: {c}")
        del Dws, dqkv_c, dO_c

    if w.kind == "vocab":
        Vr = w.V // w.P
        items = {
            "embedding_all_ranks": (lambda: [tts.tp_vocab_embedding_shard(
                tokens, Es[r], r * Vr, out=parts[r]) for r in range(w.P)], None,
                w.P * M * h * 2 + w.M * h * 2),
            "embedding_partial_sum": (lambda: tts.tp_partial_sum(parts, out=emb), None,
                                      (w.P + 1) * M * h * 2),
            "cross_entropy_all_ranks": (lambda: tts.tp_vocab_parallel_ce(
                x, Es, targets, loss=loss, loss_mean=mean, ws=ce_ws), w.flops(), None),
        }
        for name, (fn, fl, by) in items.items():
            fn()
            t, _ = component_time(fn, stream, flush if by and not fl else None)
            c = {"ms": round(t, 4)}
            if fl:
                c["tflops"] = round(fl / (t * 1e-3) / 1e12, 1)
                c["pct_peak"] = round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)
            if by:
                c["gbs"] = round(by / (t * 1e-3) / 1e9, 1)
                c["pct_hbm"] = round(100 * by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)
            components[name] = c
            log(f"component {name}: {c}")

    shards = None
    if w.kind == "block":
        shards = rank0_shards(w, tts, torch, x, A[0], B[0], Wqkv[0], Wo[0], dev, stream)

    training = None
    if w.kind == "block" and not args.no_training:
        training = mlp_backward_rank0(w, wl, tts, torch, x, A[0], B[0], dev, stream)
        training.update(attn_backward_rank0(w, wl, tts, torch, x, Wqkv[0], Wo[0], dev, stream))

    # ---------------------------------------------------------------- oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_rows, locals())
        if cpu["value"] > 0:
            # labelled as extrapolated: the oracle's rate on the sample applied to
            # one whole step's FLOPs, not a timed run of the whole step
            cpu["extrapolated_step_s"] = round(flops / (cpu["value"] * 1e12), 1)

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "tokens": w.M, "h": w.h,
                   "heads": w.H, "head_dim": w.d if w.H else None, "ffn": w.F, "tp": w.P,
                   "ranks_emulated": w.P if w.all_ranks else 1, "flops_per_step": flops,
                   "vocab": w.V or None,
                   "parallelism": "tp%d emulated on 1 GPU" % w.P},
        "roofline": {
            "kernel": kern_name,
            "bound": "mfma",
            "achieved": round(kern_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": kern_flops,
            "frac_of_mfma_only": (round(kern_tflops / calib["mfma_only"]["tflops"], 4)
                                  if "mfma_only" in calib else None),
            # the peak rescaled to the shader clock this kernel runs at under
            # the power limit (GRBM_GUI_ACTIVE over its duration, from the
            # committed counter run of the same launch)
            "clock_ghz": clock,
            "peak_at_clock": round(PEAK_BF16_TFLOPS * clock / 2.4, 1) if clock else None,
            "frac_at_clock": round(kern_tflops / (PEAK_BF16_TFLOPS * clock / 2.4), 4)
            if clock else None,
            "avg_launch_ms": round(kern_ms, 4),
            "launches_timed": len(kern_all),
            "timed": kern_where,
            "isolated_launch_ms": round(iso_ms, 4),
        },
        "cpu_baseline": cpu,
        "calibration": calib,
        "components": components,
    }
    if w.kind == "kvsplit":
        # HBM bound by construction: the exchange materialises every rank's
        # partial scores
        by = w.kvsplit_bytes()
        gbs = by / (kern_ms * 1e-3) / 1e9
        result["roofline"] = {
            "kernel": kern_name, "bound": "hbm", "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": None, "algorithmic_bytes_per_launch": by,
            "frac_of_copy": round(gbs / calib["hbm_copy"]["gbs"], 4),
            "avg_launch_ms": round(kern_ms, 4), "launches_timed": len(kern_all),
            "cache": "1 GiB written before every timed step and launch (outside the "
                     "events), evicting the 256 MB last-level cache"}
    if shards is not None:
        result["rank0_shards"] = shards
    if training is not None:
        result["training"] = training
    print(json.dumps(result), flush=True)


def rank0_shards(w, tts, torch, x, A0, B0, Wqkv0, Wo0, dev, stream):
    """One rank's shares at the block's shape, each as a single call on rank 0's
    slices (no grouped launch over ranks): tp_mlp_shard (the 175B-layer MLP
    shard, [16384 x 12288] x [12288 x 6144] then x [6144 x 12288]) and
    tp_attn_shard (8 sequences of 2048, 12 local heads of 128), timed with HIP
    events after a warm-up of their own, like the components."""
    M, h, f = w.M, w.h, w.f
    out = torch.empty(M, h, dtype=torch.float32, device=dev)
    ws_m = torch.empty(tts.tp_mlp_shard_workspace(M, f, x.dtype), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(tts.tp_attn_shard_workspace(w.b, w.s, w.Hl, w.d), dtype=torch.uint8,
                       device=dev)
    att = w.attn_flops_rank()
    items = {
        "mlp_shard_rank0": (lambda: tts.tp_mlp_shard(x, A0, B0, out=out, ws=ws_m),
                            w.mlp_flops_rank(),
                            "tp_mlp_shard, rank 0 of tp=8: %d tokens, h=%d, f=%d" % (M, h, f)),
        "attn_shard_rank0": (lambda: tts.tp_attn_shard(x, Wqkv0, Wo0, w.b, w.s, w.Hl, w.d, True,
                                                       out=out, ws=ws_a),
                             att["total"],
                             "tp_attn_shard, rank 0 of tp=8: %d sequences of %d, %d local heads "
                             "of %d, causal" % (w.b, w.s, w.Hl, w.d)),
    }
    res = {}
    for name, (fn, fl, what) in items.items():
        fn()
        t, _ = component_time(fn, stream)
        res[name] = {"ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 1),
                     "pct_peak": round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "flops": fl, "what": what}
        log(f"shard {name}: {res[name]}")
    del out, ws_m, ws_a
    return res


def mlp_backward_rank0(w, wl, tts, torch, x, A0, B0, dev, stream):
    """Rank 0's MLP-share backward at the block's shape (the same X, A_0, B_0;
    upstream gradient dZ ~ N(0,1) from the block's seed): its training forward
    once, then the backward timed with HIP events."""
    M, h, f = w.M, w.h, w.f
    dZ = wl.normal((M, h), 1.0, w.seed, "dZ", w.dtype).to(dev)
    a0 = torch.zeros(f, dtype=torch.float32, device=dev)
    _, Y, Yp = tts.tp_mlp_shard_train_fwd(x, A0, B0, a0)
    outs = dict(dX_out=torch.empty(M, h, dtype=torch.float32, device=dev),
                dA_out=torch.empty(h, f, dtype=torch.float32, device=dev),
                dB_out=torch.empty(f, h, dtype=torch.float32, device=dev),
                da_out=torch.empty(f, dtype=torch.float32, device=dev),
                ws=torch.empty(tts.tp_mlp_shard_backward_workspace(M, f), dtype=torch.uint8,
                               device=dev))
    fn = lambda: tts.tp_mlp_shard_backward(x, A0, B0, Y, Yp, dZ, **outs)
    fn()
    t, _ = component_time(fn, stream)
    fl = 8 * M * h * f
    res = {"mlp_shard_backward_rank0": {
        "ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 1),
        "pct_peak": round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
        "flops": fl,
        "what": "tp_mlp_shard_backward: dY = dZ·B_0^T ⊙ GeLU'(Y), dB_0, dA_0, da_0, dX_0 "
                "partial, for %d tokens, h=%d, f=%d" % (M, h, f)}}
    log(f"training: {res}")
    del dZ, Y, Yp, outs
    return res


def attn_backward_rank0(w, wl, tts, torch, x, Wqkv0, Wo0, dev, stream):
    """Rank 0's attention-share backward at the block's shape: its training
    forward once, then the backward timed with HIP events."""
    M, h, HD = w.M, w.h, w.Hl * w.d
    dZ = wl.normal((M, h), 1.0, w.seed, "dZ", w.dtype).to(dev)
    _, qkv, O, lse = tts.tp_attn_shard_train_fwd(x, Wqkv0, Wo0, w.b, w.s, w.Hl, w.d)
    outs = dict(dX_out=torch.empty(M, h, dtype=torch.float32, device=dev),
                dWqkv_out=torch.empty(h, 3 * HD, dtype=torch.float32, device=dev),
                dWo_out=torch.empty(HD, h, dtype=torch.float32, device=dev),
                ws=torch.empty(tts.tp_attn_shard_backward_workspace(w.b, w.s, w.Hl, w.d),
                               dtype=torch.uint8, device=dev))
    fn = lambda: tts.tp_attn_shard_backward(x, Wqkv0, Wo0, qkv, O, lse, dZ, w.b, w.s, w.Hl,
                                            w.d, **outs)
    fn()
    t, _ = component_time(fn, stream)
    fl = w.attn_bwd_flops_rank()["total"]
    res = {"attn_shard_backward_rank0": {
        "ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 1),
        "pct_peak": round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
        "flops": fl,
        "what": "tp_attn_shard_backward: dO, dW_o,0, attention-core backward (dQ, dK, dV), "
                "dW_qkv,0, dX_0 partial, for %d sequences of %d, %d local heads" % (
                    w.b, w.s, w.Hl)}}
    log(f"training: {res}")
    del dZ, qkv, O, lse, outs
    return res


# Default CPU-baseline samples (tokens), sized from the oracle's rates on 16
# host threads for 10-30 s each, or the whole workload where that is less:
# block, all of sequence 0 (~15 s); the MLP and attention shards, every token
# (3 s or less); the backward of the attention share, all 8 sequences
# (~18 s); the MLP backward, 12288 tokens (~11 s); the vocabulary ends, 8192
# tokens (~10 s); the K/V split takes all its (sequence, head) pairs (~9 s).
CPU_SAMPLE_TOKENS = {"block": 2048, "attn_bwd": 8 * 2048, "mlp_bwd": 12288, "vocab": 8192}


def cpu_baseline(w, rows_req, env):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    the first tokens (sequence-major) of its batch."""
    import numpy as np
    import oracle
    from synth import workloads as wl

    if rows_req is None:
        rows_req = CPU_SAMPLE_TOKENS.get(w.kind, 1 << 62)
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
    elif w.kind == "vocab":
        R = min(rows_req, w.M)
        tokens_cpu, targets_cpu, H_cpu, E_cpu = (env[k] for k in ("tokens_cpu", "targets_cpu",
                                                                  "H_cpu", "E_cpu"))
        Vr = w.V // w.P
        log(f"oracle: vocab ends over tokens 0..{R - 1}, all {w.P} ranks")
        t0 = time.time()
        for r in range(w.P):
            oracle.vocab_embedding_shard(tokens_cpu[:R].numpy(), E_cpu[r * Vr:(r + 1) * Vr], r * Vr)
        oracle.vocab_ce_combine([oracle.vocab_ce_shard_stats(H_cpu[:R], E_cpu[r * Vr:(r + 1) * Vr],
                                                             targets_cpu[:R].numpy(), r * Vr)
                                 for r in range(w.P)])
        dt = time.time() - t0
        fl = 2 * R * w.h * w.V
        sample = (f"tokens 0..{R - 1}: the embedding lookup and the cross-entropy of all {w.P} "
                  f"ranks; {fl / 1e12:.3f} TFLOP")
    elif w.kind == "kvsplit":
        n = w.b * w.H                               # every (sequence, head) pair
        qkv_cpu = env["qkv_cpu"]
        HD = w.H * w.d
        log(f"oracle: K/V-split attention of {n} (sequence, head) pairs")
        t0 = time.time()
        for pair in range(n):
            rows = slice((pair // w.H) * w.s, (pair // w.H + 1) * w.s)
            hd = pair % w.H
            oracle.attention_kv_split(qkv_cpu[rows, hd * w.d:(hd + 1) * w.d],
                                      qkv_cpu[rows, HD + hd * w.d:HD + (hd + 1) * w.d],
                                      qkv_cpu[rows, 2 * HD + hd * w.d:2 * HD + (hd + 1) * w.d],
                                      w.P, True)
        dt = time.time() - t0
        fl = n * 4 * w.d * w.s * (w.s + 1) // 2
        sample = (f"{n} (sequence, head) pairs, all {w.P} ranks' partial scores, the softmax and "
                  f"the output slices; {fl / 1e12:.4f} TFLOP counted as on the GPU")
    elif w.kind == "attn_bwd":
        # whole sequences (the backward of a causal sequence involves all of
        # it), or sequence 0 cut to fewer tokens
        nseq = max(1, min(w.b, rows_req // w.s))
        R = w.s if rows_req >= w.s else rows_req
        X_cpu, Wqkv_cpu, Wo_cpu, dZ_cpu = (env[k] for k in ("X_cpu", "Wqkv_cpu", "Wo_cpu",
                                                             "dZ_cpu"))
        log(f"oracle: attention backward over {nseq} sequence(s) of {R} tokens")
        t0 = time.time()
        oracle.attn_shard_backward(X_cpu[:nseq * R], nseq, R, Wqkv_cpu, Wo_cpu, dZ_cpu[:nseq * R],
                                   w.Hl, w.d, True)
        dt = time.time() - t0
        HD = w.Hl * w.d
        fl = nseq * (2 * (2 * R * w.h * 3 * HD) + 2 * (2 * R * HD * w.h)
                     + 10 * w.Hl * w.d * R * (R + 1) // 2)
        sample = (f"the attention-share backward of {nseq} sequence(s) of {R} tokens (the causal "
                  f"prefix of each); {fl / 1e12:.3f} TFLOP counted, the oracle's "
                  f"recomputation of the forward not counted")
    elif w.kind == "mlp_bwd":
        R = min(rows_req, w.M)
        X_cpu, A_cpu, B_cpu, a_cpu, dZ_cpu = (env[k] for k in ("X_cpu", "A_cpu", "B_cpu",
                                                               "a_cpu", "dZ_cpu"))
        log(f"oracle: MLP backward over tokens 0..{R - 1}")
        t0 = time.time()
        oracle.mlp_shard_backward(X_cpu[:R], A_cpu, B_cpu, dZ_cpu[:R], a_cpu)
        dt = time.time() - t0
        fl = 8 * R * w.h * w.f
        sample = (f"the MLP-share backward over tokens 0..{R - 1} (dA, dB, da and dX of that "
                  f"batch); {fl / 1e12:.3f} TFLOP counted, the oracle's recomputation of Y "
                  f"(a further {2 * R * w.h * w.f / 1e12:.3f} TFLOP) not counted")
    else:
        R = min(rows_req, w.b * w.s)                # tokens, sequence-major
        X_cpu, Wqkv_cpu, Wo_cpu = env["X_cpu"], env["Wqkv_cpu"], env["Wo_cpu"]
        log(f"oracle: attention shard rows 0..{R - 1}")
        t0 = time.time()
        oracle.attn_shard_rows(X_cpu, w.b, w.s, Wqkv_cpu, Wo_cpu, w.Hl, w.d, True,
                               np.arange(R))
        dt = time.time() - t0
        HD = w.Hl * w.d
        full, part = divmod(R, w.s)                 # whole sequences, then a prefix
        pairs = full * w.s * (w.s + 1) // 2 + part * (part + 1) // 2
        fl = 2 * R * w.h * 3 * HD + 4 * HD * pairs + 2 * R * HD * w.h
        sample = (f"tokens 0..{R - 1} of the attention shard ({full} whole sequence(s)"
                  f"{f' and {part} tokens of the next' if part else ''}); {fl / 1e12:.3f} TFLOP")
    log(f"oracle: {dt:.1f} s")
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s",
            "cores": max(oracle.num_threads(), blas_threads()), "kind": "oracle",
            "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count(),
            "sample": sample, "seconds": round(dt, 2),
            "note": "fp64; matmuls via the host BLAS, other steps plain C loops"}


def host_cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
