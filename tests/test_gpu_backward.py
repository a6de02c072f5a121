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
    Bt = gen((N, K), 1 / math.sqrt(K), 201, "w")
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
    B = gen((K, N), 1 / math.sqrt(K), 202, "w")
    C = tts.tp_matmul(At.to(DEV), B.to(DEV), trans_a=True)
    torch.cuda.synchronize()
    assert_f32(C, oracle.matmul(oracle.f64(At).T, B), bar=1e-4)


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0)])
def test_matmul_bf16_out(ta, tb):
    M, N, K = 392, 776, 200 if ta else 192
    banner(f"matmul bf16 out ta={ta} tb={tb} M={M} N={N} K={K}")
    A = gen((K, M) if ta else (M, K), 1.0, 203, "x")
    B = gen((N, K) if tb else (K, N), 1 / math.sqrt(K), 203, "w")
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
    Bbig = gen((N, K + 24), 1 / math.sqrt(K), 204, "w")
    L = tts.lib()
    Ad, Bd = Abig.to(DEV), Bbig.to(DEV)
    for ta, tb in [(1, 0), (0, 1)]:
        if ta:
            Bk = gen((K, N + 8), 1 / math.sqrt(K), 205, "w").to(DEV)
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
    Bt = gen((N, K), 1 / math.sqrt(K), 207, "w")
    aux = gen((M, N), 1.5, 207, "y")
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
    B = gen((K, N), 1 / math.sqrt(K), 208, "w")
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
    a = gen((f,), 0.5, seed, "a", torch.float32)
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
