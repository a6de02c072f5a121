"""GPU parity: every step of the path through the C ABI against the fp64
oracle, on seeded inputs that span several tiles and ragged tails.

Sizes here finish in seconds on the oracle; the full workload shapes are in
test_gpu_fullsize.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_tensor_shard_amd as tts
from _tol import assert_bf16, assert_f32, errors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def banner(msg):
    print(f"[case] {msg}", flush=True)


def gen(shape, sigma, seed, sub, dtype=torch.bfloat16):
    return synth.normal(shape, sigma, seed, sub, dtype)


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (512, 768, 320), (600, 520, 328),
                                   (1, 8, 8), (37, 264, 1032), (1300, 40, 96)])
def test_linear_bf16_f32out(M, N, K):
    banner(f"linear bf16 M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 11, "x")
    W = gen((K, N), 1 / math.sqrt(K), 11, "A")
    C = tts.tp_linear(X.to(DEV), W.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matmul(X, W)
    # identical bf16 inputs on both sides: only f32 accumulation differs
    e = assert_f32(C, ref, bar=1e-4)
    assert e["fro"] < 1e-5, e


@pytest.mark.parametrize("M,N,K", [(512, 512, 256), (333, 264, 200)])
def test_linear_bf16_bias_gelu_bf16out(M, N, K):
    banner(f"linear bf16+bias+gelu M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 12, "x")
    W = gen((K, N), 1 / math.sqrt(K), 12, "A")
    bias = gen((N,), 0.5, 12, "bias", torch.float32)
    C = tts.tp_linear(X.to(DEV), W.to(DEV), bias.to(DEV), gelu=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.gelu(oracle.matmul(X, W, bias))
    e = assert_bf16(C, ref)
    assert e["fro"] < 5e-3, e   # one bf16 rounding of the output


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (100, 36, 52)])
def test_linear_f32(M, N, K):
    banner(f"linear f32 M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 13, "x", torch.float32)
    W = gen((K, N), 1 / math.sqrt(K), 13, "A", torch.float32)
    bias = gen((N,), 0.5, 13, "bias", torch.float32)
    C = tts.tp_linear(X.to(DEV), W.to(DEV), bias.to(DEV), gelu=True)
    torch.cuda.synchronize()
    assert_f32(C, oracle.gelu(oracle.matmul(X, W, bias)))


@pytest.mark.parametrize("count,M,N,K,gelu", [(3, 300, 264, 200, True), (8, 256, 256, 64, False),
                                              (2, 1, 8, 8, False), (33, 40, 520, 96, True)])
def test_linear_batched(count, M, N, K, gelu):
    """Grouped launches: every group g against the oracle's X[g]·W[g] (+bias),
    including a repeated X, a single-tile shape (fewer tiles than XCDs) and
    more groups than one launch takes."""
    banner(f"linear batched count={count} M={M} N={N} K={K} gelu={gelu}")
    Xs = [gen((M, K), 1.0, 70 + g, "x") for g in range(count)]
    Xs[-1] = Xs[0]                                  # a shared activation
    Ws = [gen((K, N), 1 / math.sqrt(K), 70 + g, "A") for g in range(count)]
    bs = [gen((N,), 0.3, 70 + g, "bias", torch.float32) if g % 2 else None for g in range(count)]
    outs = tts.tp_linear_batched([X.to(DEV) for X in Xs], [W.to(DEV) for W in Ws],
                                 [b.to(DEV) if b is not None else None for b in bs], gelu=gelu,
                                 out_dtype=torch.bfloat16 if gelu else torch.float32)
    torch.cuda.synchronize()
    for g in range(count):
        ref = oracle.matmul(Xs[g], Ws[g], bs[g])
        if gelu:
            assert_bf16(outs[g], oracle.gelu(ref))
        else:
            assert_f32(outs[g], ref, bar=1e-4)


@pytest.mark.parametrize("count,M,N,K,gelu", [(3, 2048, 264, 200, True), (5, 4096, 520, 328, False),
                                              (34, 2048, 256, 64, True)])
def test_linear_batched_shared_x(count, M, N, K, gelu):
    """Every group shares X (the column-parallel products of all ranks), with
    whole tile-row bands per XCD: the band tile order, including ragged N and
    K and more groups than one launch takes."""
    banner(f"linear batched shared X count={count} M={M} N={N} K={K} gelu={gelu}")
    X = gen((M, K), 1.0, 80, "x")
    Ws = [gen((K, N), 1 / math.sqrt(K), 80 + g, "A") for g in range(count)]
    Xd = X.to(DEV)
    outs = tts.tp_linear_batched([Xd] * count, [W.to(DEV) for W in Ws], gelu=gelu,
                                 out_dtype=torch.bfloat16 if gelu else torch.float32)
    torch.cuda.synchronize()
    for g in range(count):
        ref = oracle.matmul(X, Ws[g])
        if gelu:
            assert_bf16(outs[g], oracle.gelu(ref))
        else:
            assert_f32(outs[g], ref, bar=1e-4)


def test_linear_deterministic():
    X = gen((700, 512), 1.0, 14, "x").to(DEV)
    W = gen((512, 640), 1 / math.sqrt(512), 14, "A").to(DEV)
    a = tts.tp_linear(X, W)
    b = tts.tp_linear(X, W)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_linear_nan_propagates():
    X = gen((300, 128), 1.0, 15, "x")
    X[7, 3] = float("nan")
    W = gen((128, 256), 1 / math.sqrt(128), 15, "A")
    C = tts.tp_linear(X.to(DEV), W.to(DEV)).cpu()
    assert torch.isnan(C[7]).all()
    C[7] = 0
    assert torch.isfinite(C).all()


# ------------------------------------------------------------------ MLP
def test_mlp_f32_tp2_sums_to_unsharded():
    """fp32 MLP TP shard, tp=2 emulated sequentially: X [2,16,64], A [64,256],
    B [256,64], zero bias; Z = Z_0 + Z_1 against the unsharded MLP."""
    banner("mlp f32 tp=2")
    seed, P, h, F = 1000, 2, 64, 256
    X = gen((32, h), 1.0, seed, "x", torch.float32)
    A = gen((h, F), 1 / math.sqrt(h), seed, "A", torch.float32)
    B = gen((F, h), 1 / math.sqrt(F), seed, "B", torch.float32)
    f = F // P
    Xd = X.to(DEV)
    parts = torch.empty(P, 32, h, dtype=torch.float32, device=DEV)
    for r in range(P):
        tts.tp_mlp_shard(Xd, A[:, r * f:(r + 1) * f].contiguous().to(DEV),
                         B[r * f:(r + 1) * f].contiguous().to(DEV), out=parts[r])
    Z = tts.tp_partial_sum(parts)
    torch.cuda.synchronize()
    assert_f32(Z, oracle.mlp_shard(X, A, B))
    for r in range(P):
        assert_f32(parts[r], oracle.mlp_shard(X, A[:, r * f:(r + 1) * f], B[r * f:(r + 1) * f]))


@pytest.mark.parametrize("M,h,f,bias", [(512, 256, 512, False), (300, 264, 136, True),
                                        (17, 512, 256, False)])
def test_mlp_bf16_small(M, h, f, bias):
    banner(f"mlp bf16 M={M} h={h} f={f} bias={bias}")
    X = gen((M, h), 1.0, 21, "x")
    A = gen((h, f), 1 / math.sqrt(h), 21, "A")
    B = gen((f, h), 1 / math.sqrt(4 * h), 21, "B")
    a = gen((f,), 0.1, 21, "bias", torch.float32) if bias else None
    Z = tts.tp_mlp_shard(X.to(DEV), A.to(DEV), B.to(DEV), a.to(DEV) if bias else None)
    Zb = tts.tp_mlp_shard(X.to(DEV), A.to(DEV), B.to(DEV), a.to(DEV) if bias else None,
                          out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.mlp_shard(X, A, B, a)
    assert_bf16(Z, ref)
    assert_bf16(Zb, ref)


# ------------------------------------------------------------------ partial sum
@pytest.mark.parametrize("P,M,h", [(8, 33, 520), (1, 5, 4), (3, 1000, 64), (2, 3, 16392),
                                   (8, 7, 16384)])     # the row kernel at its widest row
def test_partial_sum_f32(P, M, h):
    banner(f"partial sum f32 P={P} M={M} h={h}")
    parts = gen((P, M, h), 1.0, 31, "partials", torch.float32)
    bias = gen((h,), 1.0, 31, "bias", torch.float32)
    res = gen((M, h), 1.0, 31, "residual", torch.float32)
    Z = tts.tp_partial_sum(parts.to(DEV), bias.to(DEV), res.to(DEV))
    Z0 = tts.tp_partial_sum(parts.to(DEV))
    torch.cuda.synchronize()
    assert_f32(Z, oracle.partial_sum(parts, bias, res), bar=1e-5)
    assert_f32(Z0, oracle.partial_sum(parts), bar=1e-5)
    # ascending-rank f32 order: bit-identical to the same-order host sum
    host = parts[0].clone()
    for r in range(1, P):
        host += parts[r]
    assert torch.equal(Z0.cpu(), host)


def test_partial_sum_mixed_dtypes_and_alias():
    banner("partial sum bf16 parts / bf16 residual / aliasing")
    P, M, h = 4, 64, 256
    parts = gen((P, M, h), 1.0, 32, "partials")
    res = gen((M, h), 1.0, 32, "residual")
    Z = tts.tp_partial_sum(parts.to(DEV), None, res.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16(Z, oracle.partial_sum(parts, None, res), fro=4e-3)
    r32 = gen((M, h), 1.0, 32, "residual", torch.float32).to(DEV)
    p32 = gen((P, M, h), 1.0, 33, "partials", torch.float32)
    ref = oracle.partial_sum(p32, None, r32.cpu())
    tts.tp_partial_sum(p32.to(DEV), None, r32, out=r32)   # Z aliases the residual
    torch.cuda.synchronize()
    assert_f32(r32, ref, bar=1e-5)


# ------------------------------------------------------------------ LayerNorm
@pytest.mark.parametrize("M,h,dtype,affine", [(64, 4096, torch.bfloat16, False),
                                              (37, 520, torch.float32, True),
                                              (3, 12288, torch.float32, False),
                                              (5, 20000, torch.bfloat16, True),
                                              (2, 32768, torch.bfloat16, True)])   # widest row
def test_layernorm(M, h, dtype, affine):
    banner(f"layernorm M={M} h={h} {dtype} affine={affine}")
    x = gen((M, h), 2.0, 41, "x", dtype) + 0.5
    g = gen((h,), 1.0, 41, "gamma", torch.float32) if affine else None
    b = gen((h,), 1.0, 41, "beta", torch.float32) if affine else None
    y = tts.tp_layernorm(x.to(DEV), g.to(DEV) if affine else None, b.to(DEV) if affine else None)
    torch.cuda.synchronize()
    e = assert_bf16(y, oracle.layernorm(x, g, b, 1e-5))
    assert e["fro"] < 4e-3, e   # one bf16 rounding of the output


# ------------------------------------------------------------------ attention
def _qkv_weights(h, Hl, d, seed):
    Wqkv = gen((h, 3 * Hl * d), 1 / math.sqrt(h), seed, "Wqkv")
    Wo = gen((Hl * d, h), 1 / math.sqrt(h), seed, "Wo")
    return Wqkv, Wo


@pytest.mark.parametrize("b,s,Hl,causal", [(2, 256, 2, True), (1, 200, 3, True),
                                           (2, 130, 1, False), (3, 1, 2, True),
                                           (1, 64, 1, True)])
def test_attention_core(b, s, Hl, causal):
    """The attention step alone: with W_qkv = I and W_o = [I | 0] the oracle's
    shard returns O itself."""
    banner(f"attention core b={b} s={s} Hl={Hl} causal={causal}")
    d = 128
    n3 = 3 * Hl * d
    qkv = gen((b * s, n3), 1.0, 51, "x")
    O = tts.tp_attention_core(qkv.to(DEV), b, s, Hl, d, causal)
    torch.cuda.synchronize()
    eye = np.eye(n3)
    ref = oracle.attn_shard_rows(qkv, b, s, eye, np.ascontiguousarray(eye[:Hl * d]), Hl, d,
                                 causal)[:, :Hl * d]
    assert_bf16(O, ref, per_row=True)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_core_moving_max(causal):
    """Keys whose scale grows along the sequence (x1 at the first key, x17 at
    the last): each query's maximum score rises by many log2 units from tile
    to tile, so the kernel's running maximum moves past its slack and the
    accumulator is rescaled on many tiles, not just the first."""
    banner(f"attention core, growing key scale, causal={causal}")
    b, s, Hl, d = 2, 512, 2, 128
    n3 = 3 * Hl * d
    qkv = gen((b * s, n3), 1.0, 53, "x").float()
    scale = 1.0 + torch.arange(s, dtype=torch.float32).repeat(b) / 32.0
    qkv[:, Hl * d:2 * Hl * d] *= scale[:, None]
    qkv = qkv.to(torch.bfloat16)
    O = tts.tp_attention_core(qkv.to(DEV), b, s, Hl, d, causal)
    torch.cuda.synchronize()
    eye = np.eye(n3)
    ref = oracle.attn_shard_rows(qkv, b, s, eye, np.ascontiguousarray(eye[:Hl * d]), Hl, d,
                                 causal)[:, :Hl * d]
    assert_bf16(O, ref, per_row=True)


def test_attention_single_token_is_value():
    banner("attention s=1")
    b, s, Hl, d = 5, 1, 2, 128
    qkv = gen((b * s, 3 * Hl * d), 1.0, 52, "x")
    O = tts.tp_attention_core(qkv.to(DEV), b, s, Hl, d, True).cpu()
    assert torch.equal(O, qkv[:, 2 * Hl * d:])


@pytest.mark.parametrize("b,s,h,Hl", [(2, 192, 512, 2), (1, 300, 264, 1)])
def test_attn_shard_small(b, s, h, Hl):
    banner(f"attn shard b={b} s={s} h={h} Hl={Hl}")
    d = 128
    X = gen((b * s, h), 1.0, 53, "x")
    Wqkv, Wo = _qkv_weights(h, Hl, d, 53)
    Z = tts.tp_attn_shard(X.to(DEV), Wqkv.to(DEV), Wo.to(DEV), b, s, Hl, d, True)
    torch.cuda.synchronize()
    assert_bf16(Z, oracle.attn_shard_rows(X, b, s, Wqkv, Wo, Hl, d, True), per_row=True)


def test_attn_heads_sum_to_full_mha():
    """§3.2: rank partials of head-sharded attention, summed on the GPU, match
    the oracle's unsharded multi-head attention."""
    banner("attn tp=2 sum vs full MHA")
    b, s, H, d, P = 2, 160, 4, 128, 2
    h = H * d
    Hl = H // P
    X = gen((b * s, h), 1.0, 54, "x")
    Wq = gen((h, H * d), 1 / math.sqrt(h), 54, "Wqkv")
    Wk = gen((h, H * d), 1 / math.sqrt(h), 55, "Wqkv")
    Wv = gen((h, H * d), 1 / math.sqrt(h), 56, "Wqkv")
    Wo = gen((H * d, h), 1 / math.sqrt(h), 54, "Wo")
    parts = torch.empty(P, b * s, h, device=DEV)
    for r in range(P):
        sl = slice(r * Hl * d, (r + 1) * Hl * d)
        Wqkv_r = torch.cat([Wq[:, sl], Wk[:, sl], Wv[:, sl]], dim=1).contiguous()
        tts.tp_attn_shard(X.to(DEV), Wqkv_r.to(DEV), Wo[sl].contiguous().to(DEV), b, s, Hl, d,
                          True, out=parts[r])
    Z = tts.tp_partial_sum(parts)
    torch.cuda.synchronize()
    full = oracle.attn_shard_rows(X, b, s, torch.cat([Wq, Wk, Wv], 1), Wo, H, d, True)
    assert_bf16(Z, full, per_row=True)


def _core_ref(qkv, b, s, Hl, d, causal):
    """The oracle's attention over qkv = [Q | K | V] of each sequence."""
    HD = Hl * d
    out = np.empty((b * s, HD))
    for beta in range(b):
        seq = qkv[beta * s:(beta + 1) * s]
        out[beta * s:(beta + 1) * s] = oracle.attention_rows(
            seq[:, :HD], seq[:, HD:2 * HD], seq[:, 2 * HD:], np.arange(s), Hl, d, causal)
    return out


def _one_workgroup_per_block(n_bh, s, causal, cus=256):
    """The launcher's rule: query blocks of 128 take one 4-wave workgroup each
    unless the key tiles of all blocks, spread over two such workgroups per
    CU, come to less than 0.7 of the longest block's; then every block's
    keys are split over an 8-wave workgroup."""
    n_max = -(-s // 64)
    nqb = -(-s // 128)
    per_head = sum(-(-min(s, 128 * (q + 1)) // 64) if causal else n_max for q in range(nqb))
    return 10 * n_bh * per_head >= 7 * n_max * 2 * cus


@pytest.mark.parametrize("b,s,Hl,causal", [(8, 320, 30, True), (4, 200, 64, False)])
def test_attention_core_many_heads(b, s, Hl, causal):
    """Enough query blocks that each runs as one 4-wave workgroup (the
    block-shape path); the small cases above split every block's keys over
    an 8-wave workgroup."""
    banner(f"attention core many heads b={b} s={s} Hl={Hl} causal={causal}")
    assert _one_workgroup_per_block(b * Hl, s, causal)
    assert not _one_workgroup_per_block(2 * 2, 256, True)
    d = 128
    qkv = gen((b * s, 3 * Hl * d), 1.0, 58, "x")
    O = tts.tp_attention_core(qkv.to(DEV), b, s, Hl, d, causal)
    torch.cuda.synchronize()
    assert_bf16(O, _core_ref(qkv, b, s, Hl, d, causal), per_row=True)


def test_attention_core_long_sequence():
    """s = 4100: 33 query blocks and 65 key tiles, a ragged end; sampled rows
    on both sides of tile boundaries far into the sequence."""
    b, s, Hl, d = 1, 4100, 1, 128
    banner(f"attention core long b={b} s={s} Hl={Hl}")
    n3 = 3 * Hl * d
    qkv = gen((b * s, n3), 1.0, 57, "x")
    O = tts.tp_attention_core(qkv.to(DEV), b, s, Hl, d, True).cpu()
    rows = np.array([0, 1, 63, 64, 127, 128, 2047, 2048, 4095, 4096, 4099] +
                    list(np.random.default_rng(57).integers(0, s, 9)), dtype=np.int64)
    eye = np.eye(n3)
    ref = oracle.attn_shard_rows(qkv, b, s, eye, np.ascontiguousarray(eye[:Hl * d]), Hl, d, True,
                                 rows)[:, :Hl * d]
    assert_bf16(O[torch.from_numpy(rows)], ref, per_row=True)


# ------------------------------------------------------------------ block
@pytest.mark.parametrize("P,H", [(1, 2), (3, 3)])
def test_block_one_and_three_ranks(P, H):
    """Degenerate and odd rank counts: P = 1 is the unsharded block; P = 3
    splits F and H three ways."""
    b, s, d, F = 2, 96, 128, 768
    h, seed = H * d, 62 + P
    banner(f"block P={P} H={H} h={h} F={F}")
    x = gen((b * s, h), 1.0, seed, "x")
    rs = lambda r: synth.rank_seed(seed, r)
    Wqkv = [gen((h, 3 * (H // P) * d), 1 / math.sqrt(h), rs(r), "Wqkv") for r in range(P)]
    Wo = [gen(((H // P) * d, h), 1 / math.sqrt(h), rs(r), "Wo") for r in range(P)]
    A = [gen((h, F // P), 1 / math.sqrt(h), rs(r), "A") for r in range(P)]
    B = [gen((F // P, h), 1 / math.sqrt(F), rs(r), "B") for r in range(P)]
    x1 = torch.empty(b * s, h, device=DEV)
    dev = lambda ts: [t.to(DEV) for t in ts]
    out = tts.tp_block_shard(x.to(DEV), dev(Wqkv), dev(Wo), dev(A), dev(B), b, s, H, d, x1=x1)
    torch.cuda.synchronize()
    x1_ref, out_ref = oracle.block_rows(x, b, s, Wqkv, Wo, A, B, H, d)
    assert_bf16(x1, x1_ref, per_row=True)
    assert_bf16(out, out_ref, per_row=True)
    assert_bf16(out.cpu().double() - x1.cpu().double(), out_ref - x1_ref)


def test_block_small_all_ranks():
    banner("block P=2 small")
    P, b, s, H, d, F = 2, 2, 160, 4, 128, 1024
    h = H * d
    seed = 61
    x = gen((b * s, h), 1.0, seed, "x")
    Wqkv = [gen((h, 3 * (H // P) * d), 1 / math.sqrt(h), synth.rank_seed(seed, r), "Wqkv")
            for r in range(P)]
    Wo = [gen(((H // P) * d, h), 1 / math.sqrt(h), synth.rank_seed(seed, r), "Wo") for r in range(P)]
    A = [gen((h, F // P), 1 / math.sqrt(h), synth.rank_seed(seed, r), "A") for r in range(P)]
    B = [gen((F // P, h), 1 / math.sqrt(F), synth.rank_seed(seed, r), "B") for r in range(P)]
    g1 = gen((h,), 1.0, seed, "gamma", torch.float32)
    b1 = gen((h,), 1.0, seed, "beta", torch.float32)
    x1 = torch.empty(b * s, h, device=DEV)
    dev = lambda ts: [t.to(DEV) for t in ts]
    out = tts.tp_block_shard(x.to(DEV), dev(Wqkv), dev(Wo), dev(A), dev(B), b, s, H, d,
                             ln1=(g1.to(DEV), b1.to(DEV)), x1=x1)
    torch.cuda.synchronize()
    x1_ref, out_ref = oracle.block_rows(x, b, s, Wqkv, Wo, A, B, H, d, ln1=(g1, b1))
    assert_bf16(x1, x1_ref, per_row=True)
    assert_bf16(out, out_ref, per_row=True)
    # the residual dominates out: check the block's own contributions too
    assert_bf16(x1.cpu().double().numpy() - oracle.f64(x), x1_ref - oracle.f64(x), per_row=True)
    assert_bf16(out.cpu().double() - x1.cpu().double(), out_ref - x1_ref)


def test_block_timed_matches_block_and_times_the_gelu_gemm():
    """Measurement support: tp_block_shard_timed gives tp_block_shard's bits and
    its events bracket the grouped GeLU GEMM, a part of the whole call."""
    banner("block timed entry point")
    P, b, s, H, d, F = 2, 2, 160, 4, 128, 1024
    h, seed = H * d, 71
    x = gen((b * s, h), 1.0, seed, "x").to(DEV)
    rs = lambda r: synth.rank_seed(seed, r)
    Wqkv = [gen((h, 3 * (H // P) * d), 1 / math.sqrt(h), rs(r), "Wqkv").to(DEV) for r in range(P)]
    Wo = [gen(((H // P) * d, h), 1 / math.sqrt(h), rs(r), "Wo").to(DEV) for r in range(P)]
    A = [gen((h, F // P), 1 / math.sqrt(h), rs(r), "A").to(DEV) for r in range(P)]
    B = [gen((F // P, h), 1 / math.sqrt(F), rs(r), "B").to(DEV) for r in range(P)]
    ref = tts.tp_block_shard(x, Wqkv, Wo, A, B, b, s, H, d)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    whole = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    whole[0].record()
    got = tts.tp_block_shard(x, Wqkv, Wo, A, B, b, s, H, d, gelu_gemm_events=ev)
    whole[1].record()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    t = ev[0].elapsed_time(ev[1])
    assert 0.0 < t < whole[0].elapsed_time(whole[1])


def test_probe_mfma_runs():
    """Measurement support: the register-only MFMA loop launches and returns
    finite sums (its values carry no meaning)."""
    out = torch.empty(4 * 512, device=DEV)
    flops = tts.tp_probe_mfma(4, 3, out=out)
    torch.cuda.synchronize()
    assert flops == 4 * 8 * 32 * 3 * 16384
    assert torch.isfinite(out).all()
