"""GPU parity of the training path: the transposed GEMM layouts and their
epilogues (tp_matmul), the MLP share's training forward and its backward,
each through the C ABI against the fp64 oracle on seeded inputs spanning
several tiles and ragged tails."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_tensor_shard_amd as tts
from _tiles import split_ways, tile_cols
from _tol import assert_bf16, assert_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def banner(msg):
    print(f"[case] {msg}", flush=True)


def gen(shape, sigma, seed, sub, dtype=torch.bfloat16):
    return synth.normal(shape, sigma, seed, sub, dtype)


# ------------------------------------------------------------------ layouts
# (M, N, K): full tiles, ragged M/N/K tails, one row, a K shorter than a tile
SHAPES = [(256, 256, 64), (600, 520, 328), (40, 264, 1032), (1304, 48, 96), (8, 8, 8),
          (520, 264, 2056)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_matmul_nt(M, N, K):
    """C = A·B^T with B stored [N,K] (the input gradient dY·W^T)."""
    banner(f"matmul NT M={M} N={N} K={K}")
    A = gen((M, K), 1.0, 201, "x")
    Bt = gen((N, K), 1 / math.sqrt(K), 201, "A")
    bias = gen((N,), 0.5, 201, "bias", torch.float32)
    C = tts.tp_matmul(A.to(DEV), Bt.to(DEV), bias.to(DEV), trans_b=True)
    torch.cuda.synchronize()
    assert_f32(C, oracle.matmul(A, oracle.f64(Bt).T, bias), bar=1e-4)


@pytest.mark.parametrize("M,N,K", SHAPES + [(264, 256, 333), (256, 520, 1), (8, 16, 7)])
def test_matmul_tn(M, N, K):
    """C = A^T·B with A stored [K,M] (the weight gradient X^T·dY); K needs no
    alignment here, so odd K exercises the row-range tail of both operands."""
    banner(f"matmul TN M={M} N={N} K={K}")
    At = gen((K, M), 1.0, 202, "x")
    B = gen((K, N), 1 / math.sqrt(K), 202, "A")
    C = tts.tp_matmul(At.to(DEV), B.to(DEV), trans_a=True)
    torch.cuda.synchronize()
    assert_f32(C, oracle.matmul(oracle.f64(At).T, B), bar=1e-4)


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0)])
def test_matmul_bf16_out(ta, tb):
    M, N, K = 392, 776, 200 if ta else 192
    banner(f"matmul bf16 out ta={ta} tb={tb} M={M} N={N} K={K}")
    A = gen((K, M) if ta else (M, K), 1.0, 203, "x")
    B = gen((N, K) if tb else (K, N), 1 / math.sqrt(K), 203, "A")
    C = tts.tp_matmul(A.to(DEV), B.to(DEV), trans_a=bool(ta), trans_b=bool(tb),
                      out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = oracle.f64(A).T if ta else A
    b = oracle.f64(B).T if tb else B
    e = assert_bf16(C, oracle.matmul(a, b))
    assert e["fro"] < 5e-3, e      # one bf16 rounding of the output


def test_matmul_strided_leading_dims():
    """Leading dimensions wider than the logical shapes (column slices)."""
    banner("matmul strided")
    M, N, K = 304, 136, 264
    Abig = gen((K, M + 40), 1.0, 204, "x")
    Bbig = gen((N, K + 24), 1 / math.sqrt(K), 204, "A")
    L = tts.lib()
    Ad, Bd = Abig.to(DEV), Bbig.to(DEV)
    for ta, tb in [(1, 0), (0, 1)]:
        if ta:
            Bk = gen((K, N + 8), 1 / math.sqrt(K), 205, "A").to(DEV)
            Cd = torch.full((M, N + 16), 7.0, device=DEV)
            st = L.tp_matmul(tts._dev(Ad, "A"), M + 40, 1, tts._dev(Bk, "B"), N + 8, 0, None,
                             tts._dev(Cd, "C"), N + 16, None, 0, M, N, K, 0, 0, None)
            ref = oracle.matmul(oracle.f64(Abig)[:, :M].T, oracle.f64(Bk.cpu())[:, :N])
        else:
            Xk = gen((M, K + 8), 1.0, 206, "x").to(DEV)
            Cd = torch.full((M, N + 16), 7.0, device=DEV)
            st = L.tp_matmul(tts._dev(Xk, "A"), K + 8, 0, tts._dev(Bd, "B"), K + 24, 1, None,
                             tts._dev(Cd, "C"), N + 16, None, 0, M, N, K, 0, 0, None)
            ref = oracle.matmul(oracle.f64(Xk.cpu())[:, :K], oracle.f64(Bbig)[:, :K].T)
        torch.cuda.synchronize()
        assert st == 0
        assert_f32(Cd[:, :N], ref, bar=1e-4)
        assert torch.all(Cd[:, N:] == 7.0), "wrote past N"


# ------------------------------------------------------------------ epilogues
@pytest.mark.parametrize("M,N,K,out", [(600, 520, 328, torch.float32),
                                       (256, 264, 64, torch.bfloat16)])
def test_matmul_gelu_bwd(M, N, K, out):
    """C = (A·B^T) ⊙ GeLU'(aux): the chain rule through the column-parallel
    layer's GeLU, with aux the saved pre-activation."""
    banner(f"matmul NT gelu_bwd M={M} N={N} K={K} out={out}")
    A = gen((M, K), 1.0, 207, "x")
    Bt = gen((N, K), 1 / math.sqrt(K), 207, "A")
    aux = gen((M, N), 1.5, 207, "preact")
    C = tts.tp_matmul(A.to(DEV), Bt.to(DEV), trans_b=True, epilogue="gelu_bwd",
                      aux=aux.to(DEV), out_dtype=out)
    torch.cuda.synchronize()
    ref = oracle.matmul(A, oracle.f64(Bt).T) * oracle.gelu_grad(aux)
    if out == torch.float32:
        # the GeLU' evaluation in f32 (erfc to 1.5e-7) adds ~1e-6 relative
        assert_f32(C, ref, bar=1e-4)
    else:
        assert_bf16(C, ref)


@pytest.mark.parametrize("M,N,K", [(600, 520, 328), (256, 256, 64)])
def test_matmul_gelu_save(M, N, K):
    """C = GeLU(A·B + bias) and aux = A·B + bias in one epilogue."""
    banner(f"matmul NN gelu_save M={M} N={N} K={K}")
    A = gen((M, K), 1.0, 208, "x")
    B = gen((K, N), 1 / math.sqrt(K), 208, "A")
    bias = gen((N,), 0.5, 208, "bias", torch.float32)
    C, aux = tts.tp_matmul(A.to(DEV), B.to(DEV), bias.to(DEV), epilogue="gelu_save",
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Y = oracle.matmul(A, B, bias)
    assert_bf16(aux, Y)
    assert_bf16(C, oracle.gelu(Y))
    # the saved pre-activation is the exact bf16 rounding of the f32 value
    # whose GeLU was stored: GeLU(aux) and C differ by one rounding at most
    g = oracle.gelu(aux)
    assert_bf16(C, g)


# ------------------------------------------------------------------ MLP training
def mlp_inputs(M, h, f, seed):
    X = gen((M, h), 1.0, seed, "x")
    A = gen((h, f), 1 / math.sqrt(h), seed, "A")
    B = gen((f, h), 1 / math.sqrt(f), seed, "B")
    a = gen((f,), 0.5, seed, "bias", torch.float32)
    dZ = gen((M, h), 1.0, seed, "dZ")
    return X, A, B, a, dZ


@pytest.mark.parametrize("M,h,f", [(520, 264, 136), (256, 512, 256)])
def test_mlp_train_fwd(M, h, f):
    banner(f"mlp train fwd M={M} h={h} f={f}")
    X, A, B, a, _ = mlp_inputs(M, h, f, 210)
    Z, Y, Yp = tts.tp_mlp_shard_train_fwd(X.to(DEV), A.to(DEV), B.to(DEV), a.to(DEV))
    torch.cuda.synchronize()
    Yr = oracle.matmul(X, A, a)
    assert_bf16(Y, Yr)
    assert_bf16(Yp, oracle.gelu(Yr))
    assert_bf16(Z, oracle.mlp_shard(X, A, B, a))


@pytest.mark.parametrize("M,h,f,dx", [(520, 264, 136, torch.float32),
                                      (1000, 512, 264, torch.bfloat16),
                                      (8, 64, 32, torch.float32),
                                      (2048, 256, 512, torch.float32)])
def test_mlp_backward(M, h, f, dx):
    """Every gradient of one rank's MLP share against the oracle's chain rule
    (pinned by float64 autograd and finite differences on the CPU)."""
    banner(f"mlp backward M={M} h={h} f={f} dx={dx}")
    X, A, B, a, dZ = mlp_inputs(M, h, f, 211)
    Xd, Ad, Bd, ad, dZd = (t.to(DEV) for t in (X, A, B, a, dZ))
    _, Y, Yp = tts.tp_mlp_shard_train_fwd(Xd, Ad, Bd, ad)
    dX, dA, dB, da = tts.tp_mlp_shard_backward(Xd, Ad, Bd, Y, Yp, dZd, dx_dtype=dx)
    torch.cuda.synchronize()
    rX, rA, rB, ra = oracle.mlp_shard_backward(X, A, B, dZ, a)
    # bf16 bars: Y, Y' and dY are held in bf16 between the products
    assert_bf16(dX, rX)
    assert_bf16(dA, rA)
    assert_bf16(dB, rB)
    assert_bf16(da.reshape(1, -1), ra.reshape(1, -1))


def test_mlp_backward_no_bias_grad_and_deterministic():
    banner("mlp backward repeat")
    M, h, f = 700, 256, 136
    X, A, B, a, dZ = mlp_inputs(M, h, f, 212)
    Xd, Ad, Bd, ad, dZd = (t.to(DEV) for t in (X, A, B, a, dZ))
    _, Y, Yp = tts.tp_mlp_shard_train_fwd(Xd, Ad, Bd, ad)
    r1 = tts.tp_mlp_shard_backward(Xd, Ad, Bd, Y, Yp, dZd)
    r2 = tts.tp_mlp_shard_backward(Xd, Ad, Bd, Y, Yp, dZd)
    r3 = tts.tp_mlp_shard_backward(Xd, Ad, Bd, Y, Yp, dZd, bias_grad=False)
    torch.cuda.synchronize()
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)
    assert r3[3] is None
    for u, v in zip(r1[:3], r3[:3]):
        assert torch.equal(u, v)


def test_mlp_backward_ranks_sum_to_unsharded():
    """Two emulated ranks' dX_i summed with tp_partial_sum (the backward
    all-reduce's arithmetic) against the unsharded MLP's dX."""
    banner("mlp backward 2 ranks")
    M, h, f, P = 512, 256, 512, 2
    X, A, B, a, dZ = mlp_inputs(M, h, f, 213)
    fl = f // P
    Xd, dZd = X.to(DEV), dZ.to(DEV)
    parts = []
    for r in range(P):
        Ar = A[:, r * fl:(r + 1) * fl].contiguous().to(DEV)
        Br = B[r * fl:(r + 1) * fl].contiguous().to(DEV)
        ar = a[r * fl:(r + 1) * fl].contiguous().to(DEV)
        _, Y, Yp = tts.tp_mlp_shard_train_fwd(Xd, Ar, Br, ar)
        parts.append(tts.tp_mlp_shard_backward(Xd, Ar, Br, Y, Yp, dZd)[0])
    dX = tts.tp_partial_sum(torch.stack(parts))
    torch.cuda.synchronize()
    rX = oracle.mlp_shard_backward(X, A, B, dZ, a)[0]
    assert_bf16(dX, rX)


# ------------------------------------------------------------------ attention training
def _heads(t, beta, s, k, HD):
    """sequence beta's block k (0 = Q, 1 = K, 2 = V) of a [b·s, 3·HD] tensor."""
    return oracle.f64(t)[beta * s:(beta + 1) * s, k * HD:(k + 1) * HD]


@pytest.mark.parametrize("b,s,Hl,causal", [(2, 128, 2, True), (1, 200, 3, True),
                                           (2, 384, 1, True), (1, 200, 2, False),
                                           (3, 64, 2, False), (2, 1, 2, True),
                                           (1, 520, 1, True)])
def test_attention_core_backward(b, s, Hl, causal):
    """dQ, dK, dV of the attention core against the oracle's softmax chain
    rule, per sequence, with ragged sequence ends and both masks."""
    banner(f"attention core backward b={b} s={s} Hl={Hl} causal={causal}")
    d, HD = 128, Hl * 128
    qkv = gen((b * s, 3 * HD), 1.0, 220, "x")
    dO = gen((b * s, HD), 1.0, 220, "dZ")
    qd = qkv.to(DEV)
    O, lse = tts.tp_attention_core_train(qd, b, s, Hl, d, causal)
    dqkv = tts.tp_attention_core_backward(qd, O, dO.to(DEV), lse, b, s, Hl, d, causal)
    torch.cuda.synchronize()
    for beta in range(b):
        ref = oracle.attention_backward(_heads(qkv, beta, s, 0, HD), _heads(qkv, beta, s, 1, HD),
                                        _heads(qkv, beta, s, 2, HD),
                                        oracle.f64(dO)[beta * s:(beta + 1) * s], Hl, d, causal)
        got = dqkv[beta * s:(beta + 1) * s]
        for k in range(3):
            g = got[:, k * HD:(k + 1) * HD]
            if s == 1 and k < 2:
                # one key: the softmax is constant and Q, K get zero gradient;
                # the kernel's dS = P·(dP - D) keeps only the rounding residue
                # of two dot products of the same vectors taken in different
                # orders, far below the scale of dV = dO
                scale = float(np.sqrt(np.mean(oracle.f64(dO) ** 2)))
                assert float(g.abs().max()) <= 1e-4 * scale
            else:
                assert_bf16(g, ref[k], per_row=True)


def test_attention_train_forward_unchanged():
    """The training forward's O equals the inference forward's bit for bit."""
    banner("attention train forward == forward")
    b, s, Hl = 2, 300, 2
    qkv = gen((b * s, 3 * Hl * 128), 1.0, 221, "x").to(DEV)
    O1 = tts.tp_attention_core(qkv, b, s, Hl)
    O2, lse = tts.tp_attention_core_train(qkv, b, s, Hl)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    assert torch.isfinite(lse).all()


@pytest.mark.parametrize("b,s,h,Hl,causal,dx", [(2, 256, 256, 2, True, torch.float32),
                                                (1, 200, 264, 1, True, torch.bfloat16),
                                                (2, 136, 128, 2, False, torch.float32)])
def test_attn_shard_backward(b, s, h, Hl, causal, dx):
    """Every gradient of one rank's attention share (dX_i partial, dW_qkv,i,
    dW_o,i) against the oracle, through the training forward's activations."""
    banner(f"attn shard backward b={b} s={s} h={h} Hl={Hl} causal={causal} dx={dx}")
    HD = Hl * 128
    X = gen((b * s, h), 1.0, 222, "x")
    Wqkv = gen((h, 3 * HD), 1 / math.sqrt(h), 222, "Wqkv")
    Wo = gen((HD, h), 1 / math.sqrt(h), 222, "Wo")
    dZ = gen((b * s, h), 1.0, 222, "dZ")
    Xd, Wqd, Wod = X.to(DEV), Wqkv.to(DEV), Wo.to(DEV)
    Z, qkv, O, lse = tts.tp_attn_shard_train_fwd(Xd, Wqd, Wod, b, s, Hl, causal=causal)
    dX, dWqkv, dWo = tts.tp_attn_shard_backward(Xd, Wqd, Wod, qkv, O, lse, dZ.to(DEV), b, s, Hl,
                                                causal=causal, dx_dtype=dx)
    torch.cuda.synchronize()
    assert_bf16(Z, oracle.attn_shard_rows(X, b, s, Wqkv, Wo, Hl, 128, causal), per_row=True)
    rX, rWqkv, rWo = oracle.attn_shard_backward(X, b, s, Wqkv, Wo, dZ, Hl, 128, causal)
    assert_bf16(dX, rX, per_row=True)
    assert_bf16(dWqkv, rWqkv, per_row=True)
    assert_bf16(dWo, rWo, per_row=True)


@pytest.mark.parametrize("ta,tb,shapes,K,ways", [
    (1, 0, [(512, 768), (256, 520)], 4096, 2),     # weight-gradient layout, N ragged
    (0, 0, [(300, 264), (512, 256)], 8192, 4),     # forward layout, M ragged
    (0, 1, [(256, 512), (40, 264)], 4096, 2)])     # input-gradient layout
def test_matmul_grouped_split_last_wave(ta, tb, shapes, K, ways):
    """Given spare memory, a launch whose one wave fills few compute units runs
    every tile as `ways` workgroups over equal K ranges and adds the ranges'
    f32 blocks to C in range order: each element equals, bit for bit, that
    ordered sum of `ways` launches over the K ranges alone (without spare
    memory); and the whole against the oracle."""
    spare = (ways - 1) * 16 * 256 * 256 * 4
    assert split_ways(shapes, K, spare) == ways
    banner(f"matmul grouped split ta={ta} tb={tb} shapes={shapes} K={K} ways={ways}")
    As = [gen((K, m) if ta else (m, K), 1.0, 240 + g, "x") for g, (m, n) in enumerate(shapes)]
    Bs = [gen((n, K) if tb else (K, n), 1 / math.sqrt(K), 240 + g, "A")
          for g, (m, n) in enumerate(shapes)]
    Ad, Bd = [A.to(DEV) for A in As], [B.to(DEV) for B in Bs]
    ws = torch.full((spare,), 0x7F, dtype=torch.uint8, device=DEV)   # garbage: written first
    outs = tts.tp_matmul_grouped(Ad, Bd, trans_a=bool(ta), trans_b=bool(tb), ws=ws)

    def k_range(t, k0, k1, k_rows):
        return (t[k0:k1] if k_rows else t[:, k0:k1]).contiguous()
    kr = K // ways
    ref = None
    for p in range(ways):
        k0, k1 = p * kr, (p + 1) * kr
        part = tts.tp_matmul_grouped([k_range(A, k0, k1, ta) for A in Ad],
                                     [k_range(B, k0, k1, not tb) for B in Bd],
                                     trans_a=bool(ta), trans_b=bool(tb))
        ref = part if ref is None else [r + q for r, q in zip(ref, part)]
    torch.cuda.synchronize()
    for g in range(len(shapes)):
        assert torch.equal(outs[g], ref[g]), g
        a = oracle.f64(As[g]).T if ta else As[g]
        b = oracle.f64(Bs[g]).T if tb else Bs[g]
        assert_f32(outs[g], oracle.matmul(a, b), bar=1e-4)


def test_matmul_grouped_spare_too_small_means_no_split():
    """Spare memory smaller than the split's blocks (here 1 MiB against the
    4 MiB two K ranges of 16 tail tiles need) leaves the launch unsplit: its
    result equals, bit for bit, the launch given no spare memory."""
    shapes, K = [(512, 768), (256, 520)], 4096
    assert split_ways(shapes, K, 4 << 20) == 2 and split_ways(shapes, K, 1 << 20) == 0
    banner(f"matmul grouped, spare too small: shapes={shapes} K={K}")
    As = [gen((K, m), 1.0, 245 + g, "x").to(DEV) for g, (m, n) in enumerate(shapes)]
    Bs = [gen((K, n), 1 / math.sqrt(K), 245 + g, "A").to(DEV) for g, (m, n) in enumerate(shapes)]
    ws = torch.full((1 << 20,), 0x7F, dtype=torch.uint8, device=DEV)
    small = tts.tp_matmul_grouped(As, Bs, trans_a=True, ws=ws)
    plain = tts.tp_matmul_grouped(As, Bs, trans_a=True)
    torch.cuda.synchronize()
    for u, v in zip(small, plain):
        assert torch.equal(u, v)
    assert torch.equal(ws, torch.full_like(ws, 0x7F))      # never touched


def test_attn_shard_backward_split_last_wave():
    """16 sequences of 256 tokens, 8 local heads, h = 512: the weight-gradient
    launch (dW_qkv 24 tiles, dW_o 8: 32 workgroups, under half the CUs, K =
    4096 tokens) runs each tile as two workgroups over the halves of K and
    adds the second half into C afterwards, in the dO buffer's memory.  Every
    gradient against the oracle, and a repeat bit for bit."""
    b, s, h, Hl = 16, 256, 512, 8
    HD = Hl * 128
    assert tile_cols([(h, 3 * HD), (HD, h)], b * s, trans_a=True) == 256
    assert split_ways([(h, 3 * HD), (HD, h)], b * s, b * s * HD * 2) == 2
    banner(f"attn shard backward, split last wave: b={b} s={s} h={h} Hl={Hl}")
    X = gen((b * s, h), 1.0, 226, "x")
    Wqkv = gen((h, 3 * HD), 1 / math.sqrt(h), 226, "Wqkv")
    Wo = gen((HD, h), 1 / math.sqrt(h), 226, "Wo")
    dZ = gen((b * s, h), 1.0, 226, "dZ")
    Xd, Wqd, Wod, dZd = X.to(DEV), Wqkv.to(DEV), Wo.to(DEV), dZ.to(DEV)
    _, qkv, O, lse = tts.tp_attn_shard_train_fwd(Xd, Wqd, Wod, b, s, Hl)
    g1 = tts.tp_attn_shard_backward(Xd, Wqd, Wod, qkv, O, lse, dZd, b, s, Hl)
    g2 = tts.tp_attn_shard_backward(Xd, Wqd, Wod, qkv, O, lse, dZd, b, s, Hl)
    torch.cuda.synchronize()
    for u, v in zip(g1, g2):
        assert torch.equal(u, v)
    rX, rWqkv, rWo = oracle.attn_shard_backward(X, b, s, Wqkv, Wo, dZ, Hl, 128, True)
    assert_bf16(g1[0], rX, per_row=True)
    assert_bf16(g1[1], rWqkv, per_row=True)
    assert_bf16(g1[2], rWo, per_row=True)


def test_attn_backward_deterministic_and_ranks_sum():
    """Two emulated ranks (heads split) summed with tp_partial_sum against the
    unsharded share's dX; and a repeated call gives identical bits."""
    banner("attn backward 2 ranks + repeat")
    b, s, h, H, P = 1, 256, 256, 2, 2
    HD = H * 128
    X = gen((b * s, h), 1.0, 223, "x")
    Wq, Wk, Wv = (gen((h, HD), 1 / math.sqrt(h), 223 + k, "Wqkv") for k in range(3))
    Wo = gen((HD, h), 1 / math.sqrt(h), 223, "Wo")
    dZ = gen((b * s, h), 1.0, 223, "dZ")
    Xd, dZd = X.to(DEV), dZ.to(DEV)
    parts = []
    for r in range(P):
        c = slice(r * 128, (r + 1) * 128)
        Wqkv_r = torch.cat([Wq[:, c], Wk[:, c], Wv[:, c]], dim=1).contiguous().to(DEV)
        Wo_r = Wo[c].contiguous().to(DEV)
        _, qkv, O, lse = tts.tp_attn_shard_train_fwd(Xd, Wqkv_r, Wo_r, b, s, 1)
        g1 = tts.tp_attn_shard_backward(Xd, Wqkv_r, Wo_r, qkv, O, lse, dZd, b, s, 1)
        g2 = tts.tp_attn_shard_backward(Xd, Wqkv_r, Wo_r, qkv, O, lse, dZd, b, s, 1)
        torch.cuda.synchronize()
        for u, v in zip(g1, g2):
            assert torch.equal(u, v)
        parts.append(g1[0])
    dX = tts.tp_partial_sum(torch.stack(parts))
    torch.cuda.synchronize()
    Wqkv_full = torch.cat([Wq, Wk, Wv], dim=1)
    rX = oracle.attn_shard_backward(X, b, s, Wqkv_full, Wo, dZ, H, 128, True)[0]
    assert_bf16(dX, rX, per_row=True)


@pytest.mark.parametrize("ta,tb,shapes,K", [
    (1, 0, [(264, 520), (520, 264), (8, 16)], 333),     # weight gradients: A stored [K, M]
    (1, 0, [(512, 256), (256, 768)], 1024),
    (0, 1, [(600, 520), (40, 264)], 328),
    (0, 0, [(300, 264), (16, 8), (256, 512)], 200)])
def test_matmul_grouped(ta, tb, shapes, K):
    """One launch of products with different M and N (and leading
    dimensions): every group against the oracle."""
    banner(f"matmul grouped ta={ta} tb={tb} shapes={shapes} K={K}")
    As = [gen((K, m) if ta else (m, K), 1.0, 230 + g, "x") for g, (m, n) in enumerate(shapes)]
    Bs = [gen((n, K) if tb else (K, n), 1 / math.sqrt(K), 230 + g, "A")
          for g, (m, n) in enumerate(shapes)]
    outs = tts.tp_matmul_grouped([A.to(DEV) for A in As], [B.to(DEV) for B in Bs],
                                 trans_a=bool(ta), trans_b=bool(tb))
    torch.cuda.synchronize()
    for g in range(len(shapes)):
        a = oracle.f64(As[g]).T if ta else As[g]
        b = oracle.f64(Bs[g]).T if tb else Bs[g]
        assert_f32(outs[g], oracle.matmul(a, b), bar=1e-4)


# ------------------------------------------------------------------ vocabulary ends
@pytest.mark.parametrize("M,h,V_r,P,out", [(300, 64, 520, 2, torch.float32),
                                           (1024, 256, 64, 4, torch.bfloat16)])
def test_vocab_embedding(M, h, V_r, P, out):
    """Each rank's lookup is exact (a copy), and the ranks' partial sum is the
    full table's rows, bit for bit."""
    banner(f"vocab embedding M={M} h={h} V_r={V_r} P={P} out={out}")
    V = V_r * P
    E = gen((V, h), 0.02, 240, "E")
    tokens = synth.token_ids(M, V, 240, "tokens")
    tokens[:4] = torch.tensor([0, V - 1, V_r - 1, V_r], dtype=torch.int32)
    td = tokens.to(DEV)
    parts = torch.stack([tts.tp_vocab_embedding_shard(td, E[r * V_r:(r + 1) * V_r].contiguous().to(DEV),
                                                      r * V_r, out_dtype=torch.float32)
                         for r in range(P)])
    Z = tts.tp_partial_sum(parts)
    one = tts.tp_vocab_embedding_shard(td, E[:V_r].contiguous().to(DEV), 0, out_dtype=out)
    torch.cuda.synchronize()
    for r in range(P):
        ref = oracle.vocab_embedding_shard(tokens.numpy(), E[r * V_r:(r + 1) * V_r], r * V_r)
        assert np.array_equal(parts[r].cpu().double().numpy(), ref)
    assert np.array_equal(Z.cpu().double().numpy(), oracle.f64(E)[tokens.long().numpy()])
    assert np.array_equal(one.cpu().double().numpy(),
                          oracle.vocab_embedding_shard(tokens.numpy(), E[:V_r], 0))


@pytest.mark.parametrize("M,h,V_r,P", [(300, 264, 520, 3), (512, 512, 6400 // 8, 8),
                                       (1, 64, 8, 2), (700, 128, 1032, 1), (2304, 128, 3840, 2),
                                       (2304, 128, 3848, 2)])
def test_vocab_cross_entropy(M, h, V_r, P):
    """Per-rank statistics and the combined loss against the oracle; the
    all-ranks entry point equals the per-rank path bit for bit.  In the last
    two cases the per-rank launches take 256-column output tiles and the
    all-ranks launch 384-column ones: the statistics, kept per 128-column
    piece, do not depend on the width (V_r = 3848: each rank's last
    384-column tile holds 8 columns, one partial piece)."""
    banner(f"vocab cross-entropy M={M} h={h} V_r={V_r} P={P}")
    if (M, P) == (2304, 2):
        assert tile_cols([(M, V_r)], h, trans_b=True, epilogue="ce_stats") == 256
        assert tile_cols([(M, V_r)] * P, h, trans_b=True, epilogue="ce_stats") == 384
    V = V_r * P
    H = gen((M, h), 1.0, 241, "x")
    E = gen((V, h), 0.02 * math.sqrt(4096 / h), 241, "E")
    targets = synth.token_ids(M, V, 241, "targets")
    Hd, td = H.to(DEV), targets.to(DEV)
    Es = [E[r * V_r:(r + 1) * V_r].contiguous().to(DEV) for r in range(P)]
    stats = torch.stack([tts.tp_vocab_ce_shard(Hd, Es[r], td, r * V_r) for r in range(P)])
    loss, mean = tts.tp_vocab_ce_combine(stats)
    loss2, mean2 = tts.tp_vocab_parallel_ce(Hd, Es, td)
    torch.cuda.synchronize()
    ref_stats = [oracle.vocab_ce_shard_stats(H, E[r * V_r:(r + 1) * V_r], targets.numpy(), r * V_r)
                 for r in range(P)]
    for r in range(P):
        m, s, t = ref_stats[r]
        assert_f32(stats[r, 0].reshape(1, -1), m.reshape(1, -1), bar=1e-4)
        assert_f32(stats[r, 1].reshape(1, -1), s.reshape(1, -1), bar=1e-4)
        # the target logit is 0 exactly off the rank, the f32 logit on it
        assert_f32(stats[r, 2].reshape(1, -1), t.reshape(1, -1), bar=1e-4)
    ref = oracle.vocab_ce_combine(ref_stats)
    assert_f32(loss.reshape(1, -1), ref.reshape(1, -1), bar=1e-4)
    assert abs(float(mean) - ref.mean()) <= 1e-4 * abs(ref.mean())
    assert torch.equal(loss, loss2) and torch.equal(mean, mean2)
