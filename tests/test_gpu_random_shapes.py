"""Seeded random sweeps of shapes through the GEMM and the attention core
(GPU, through the C ABI, against the fp64 oracle).

The fixed-shape parity tests pin the tile boundaries one by one; these draw
shapes, layouts, epilogues and output types from a seeded generator, so that
combinations nobody wrote down -- a ragged M with a short K and 192-column
tiles, a transposed operand with a one-row output -- also meet the bars.  The
cases are listed by index, so a failure names its draw.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_tensor_shard_amd as tts
from _tiles import split_ways
from _tol import assert_bf16, assert_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 20261203


def banner(msg):
    print(f"[case] {msg}", flush=True)


def gen(shape, sigma, seed, sub, dtype=torch.bfloat16):
    return synth.normal(shape, sigma, seed, sub, dtype)


def _gemm_cases(n=28):
    rng = np.random.default_rng(SEED)
    cases = []
    epilogues = {"nn": ["none", "gelu", "gelu_save"], "nt": ["none", "gelu_bwd"], "tn": ["none"]}
    for i in range(n):
        layout = ["nn", "nt", "tn"][i % 3]
        epi = epilogues[layout][int(rng.integers(0, len(epilogues[layout])))]
        # the training forward's dual store is bf16 only; the others take either
        out = "bf16" if epi == "gelu_save" or rng.random() < 0.5 else "f32"
        if i % 7 == 0:     # large enough for 192-column tiles to be chosen
            M = int(rng.integers(1800, 2600))
            N = 8 * int(rng.integers(700, 1000))
        else:
            M = int(rng.integers(1, 1300))
            N = 8 * int(rng.integers(1, 160))
        K = 8 * int(rng.integers(1, 41))
        if layout == "tn":
            M = 8 * max(1, M // 8)                   # A stored [K, M]: M contiguous
        cases.append((i, layout, epi, out, M, N, K))
    return cases


@pytest.mark.parametrize("i,layout,epi,out,M,N,K", _gemm_cases())
def test_gemm_random(i, layout, epi, out, M, N, K):
    banner(f"random GEMM #{i}: {layout} epi={epi} out={out} M={M} N={N} K={K}")
    s = SEED + i
    A = gen((K, M) if layout == "tn" else (M, K), 1.0, s, "x")
    B = gen((N, K) if layout == "nt" else (K, N), 1 / math.sqrt(K), s, "A")
    bias = gen((N,), 0.5, s, "bias", torch.float32) if epi in ("gelu", "gelu_save") else None
    aux = gen((M, N), 1.0, s, "preact") if epi == "gelu_bwd" else None
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    res = tts.tp_matmul(A.to(DEV), B.to(DEV), bias.to(DEV) if bias is not None else None,
                        trans_a=layout == "tn", trans_b=layout == "nt", epilogue=epi,
                        aux=aux.to(DEV) if aux is not None else None, out_dtype=odt)
    torch.cuda.synchronize()
    a = A.t().contiguous() if layout == "tn" else A
    b = B.t().contiguous() if layout == "nt" else B
    v = oracle.matmul(a, b, bias)
    if epi == "gelu_save":
        C, saved = res
        assert_bf16(saved, v)
        assert_bf16(C, oracle.gelu(v))
        return
    ref = {"none": v, "gelu": oracle.gelu(v) if epi == "gelu" else None,
           "gelu_bwd": v * oracle.gelu_grad(aux) if epi == "gelu_bwd" else None}[epi]
    if out == "bf16":
        assert_bf16(res, ref)
    else:
        assert_f32(res, ref, bar=1e-4)


def _split_cases(n=6):
    rng = np.random.default_rng(SEED + 2)
    cases = []
    for i in range(n):
        layout = ["nn", "nt", "tn"][i % 3]
        count = int(rng.integers(1, 4))
        shapes = [(8 * int(rng.integers(1, 80)), 8 * int(rng.integers(1, 80))) for _ in range(count)]
        K = 256 * int(rng.integers(16, 48))          # 4096 .. 12032: two or four K ranges
        cases.append((i, layout, shapes, K))
    return cases


@pytest.mark.parametrize("i,layout,shapes,K", _split_cases())
def test_matmul_grouped_split_random(i, layout, shapes, K):
    """Grouped f32 products given spare memory, on random shapes small enough
    that their one wave of workgroups takes at most half the compute units:
    the split over K must equal, bit for bit, the ordered sum of the K
    ranges' own launches, and the oracle within the f32 bar."""
    spare = 3 * 256 * 256 * 256 * 4                 # room for any tail of this size
    ways = split_ways(shapes, K, spare)
    assert ways in (2, 4)
    banner(f"random split #{i}: {layout} shapes={shapes} K={K} ways={ways}")
    ta, tb = layout == "tn", layout == "nt"
    seeds = [SEED + 100 + 10 * i + g for g in range(len(shapes))]
    As = [gen((K, m) if ta else (m, K), 1.0, sd, "x") for sd, (m, n) in zip(seeds, shapes)]
    Bs = [gen((n, K) if tb else (K, n), 1 / math.sqrt(K), sd, "A") for sd, (m, n) in zip(seeds, shapes)]
    Ad, Bd = [A.to(DEV) for A in As], [B.to(DEV) for B in Bs]
    ws = torch.full((spare,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN bits: written first
    outs = tts.tp_matmul_grouped(Ad, Bd, trans_a=ta, trans_b=tb, ws=ws)
    kr = K // ways
    ref = None
    for p in range(ways):
        k0, k1 = p * kr, (p + 1) * kr
        part = tts.tp_matmul_grouped(
            [(A[k0:k1] if ta else A[:, k0:k1]).contiguous() for A in Ad],
            [(B[:, k0:k1] if tb else B[k0:k1]).contiguous() for B in Bd], trans_a=ta, trans_b=tb)
        ref = part if ref is None else [r + q for r, q in zip(ref, part)]
    torch.cuda.synchronize()
    for g in range(len(shapes)):
        assert torch.equal(outs[g], ref[g]), g
        a = As[g].t().contiguous() if ta else As[g]
        b = Bs[g].t().contiguous() if tb else Bs[g]
        assert_f32(outs[g], oracle.matmul(a, b), bar=1e-4)


def _attn_cases(n=10):
    rng = np.random.default_rng(SEED + 1)
    cases = []
    for i in range(n):
        b = int(rng.integers(1, 4))
        s = int(rng.integers(1, 700))
        Hl = int(rng.integers(1, 4))
        causal = bool(rng.random() < 0.7)
        cases.append((i, b, s, Hl, causal))
    return cases


@pytest.mark.parametrize("i,b,s,Hl,causal", _attn_cases())
def test_attention_core_random(i, b, s, Hl, causal):
    banner(f"random attention #{i}: b={b} s={s} Hl={Hl} causal={causal}")
    d = 128
    HD = Hl * d
    qkv = gen((b * s, 3 * HD), 1.0, SEED + 100 + i, "x")
    O = tts.tp_attention_core(qkv.to(DEV), b, s, Hl, d, causal)
    torch.cuda.synchronize()
    ref = np.empty((b * s, HD))
    for beta in range(b):
        seq = qkv[beta * s:(beta + 1) * s]
        ref[beta * s:(beta + 1) * s] = oracle.attention_rows(
            seq[:, :HD], seq[:, HD:2 * HD], seq[:, 2 * HD:], np.arange(s), Hl, d, causal)
    assert_bf16(O, ref, per_row=True)
