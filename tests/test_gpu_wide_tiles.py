"""GPU parity of the GEMM with 256x384 output tiles.

Products in the forward layout (plain, GeLU and dual-store epilogues) and
the input-gradient layout (B stored [N,K]: plain and GeLU-backward
epilogues), K a multiple of 64, whose waves of workgroups the wider tile
fills better run on the 384-column kernel (the launcher's choice; each shape
below is checked to take it).  Per
output element the K loop is the same MFMA sequence as in the 256-column
kernel, so each case meets the same bars: f32 output within 1e-4 of the
oracle, bf16 output within the bf16 bar; and a sub-block computed by the
256-column kernel agrees with the wide launch bit for bit.  The shapes
cover ragged M and N (a last tile 1/3 or 2/3 full), even and odd counts of
64-wide K tiles, bias and GeLU, both output types, the shared-X band order,
a grouped launch whose products differ in M and N, several tiles per
compute unit, and NaN propagation.
"""
import math

import pytest
import torch

import oracle
import synth
import transformer_tensor_shard_amd as tts
from _tiles import tile_cols
from _tol import assert_bf16, assert_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def banner(msg):
    print(f"[case] {msg}", flush=True)


def gen(shape, sigma, seed, sub, dtype=torch.bfloat16):
    return synth.normal(shape, sigma, seed, sub, dtype)


def wide(prods, K, **kw):
    assert tile_cols(prods, K, **kw) == 384, prods
    assert tts.tp_gemm_tile_cols(prods, K, **kw) == 384, prods


def test_wide_bias_gelu_bf16_matches_narrow_kernel_bitwise():
    M, N, K = 2304, 7680, 128
    wide([(M, N)], K, epilogue="gelu")
    banner(f"wide tiles linear bias+gelu bf16 M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 601, "x")
    W = gen((K, N), 1 / math.sqrt(K), 601, "A")
    bias = gen((N,), 0.5, 601, "bias", torch.float32)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), bias.to(DEV)
    C = tts.tp_linear(Xd, Wd, bd, gelu=True, out_dtype=torch.bfloat16)
    # the first 256 rows alone are 30 tiles of 256 columns (one wave)
    assert tts.tp_gemm_tile_cols([(256, N)], K, epilogue="gelu") == 256
    C0 = tts.tp_linear(Xd[:256].contiguous(), Wd, bd, gelu=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(C[:256].view(torch.int16), C0.view(torch.int16))
    assert_bf16(C, oracle.gelu(oracle.matmul(X, W, bias)))


def test_wide_f32_ragged_matches_narrow_kernel_bitwise():
    M, N, K = 2250, 7560, 192                 # ragged M and N, 3 K tiles
    wide([(M, N)], K)
    banner(f"wide tiles linear f32 M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 602, "x")
    W = gen((K, N), 1 / math.sqrt(K), 602, "A")
    Xd, Wd = X.to(DEV), W.to(DEV)
    C = tts.tp_linear(Xd, Wd, out_dtype=torch.float32)
    C0 = tts.tp_linear(Xd[2048:].contiguous(), Wd, out_dtype=torch.float32)   # last tile row
    torch.cuda.synchronize()
    assert torch.equal(C[2048:], C0)
    e = assert_f32(C, oracle.matmul(X, W), bar=1e-4)
    assert e["fro"] < 1e-5, e


def test_wide_bf16_plain_ragged_m_long_k():
    M, N, K = 4000, 4608, 1088                # 17 K tiles (odd), M ragged
    wide([(M, N)], K)
    banner(f"wide tiles linear bf16 M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 603, "x")
    W = gen((K, N), 1 / math.sqrt(K), 603, "A")
    C = tts.tp_linear(X.to(DEV), W.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16(C, oracle.matmul(X, W))


def test_wide_shared_x_band_order():
    count, M, N, K = 3, 2048, 3072, 64
    wide([(M, N)] * count, K, epilogue="gelu")
    banner(f"wide tiles shared X count={count} M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 604, "x")
    Ws = [gen((K, N), 1 / math.sqrt(K), 604 + g, "A") for g in range(count)]
    Xd = X.to(DEV)
    outs = tts.tp_linear_batched([Xd] * count, [W.to(DEV) for W in Ws], gelu=True,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for g in range(count):
        assert_bf16(outs[g], oracle.gelu(oracle.matmul(X, Ws[g])))


def test_wide_grouped_different_shapes():
    K = 128
    shapes = [(2304, 3840), (2100, 3904)]     # 3904 = 10 tiles of 384 + 64 columns
    wide(shapes, K)
    banner(f"wide tiles grouped shapes={shapes} K={K}")
    As = [gen((m, K), 1.0, 605 + g, "x") for g, (m, _) in enumerate(shapes)]
    Bs = [gen((K, n), 1 / math.sqrt(K), 605 + g, "A") for g, (_, n) in enumerate(shapes)]
    outs = tts.tp_matmul_grouped([A.to(DEV) for A in As], [B.to(DEV) for B in Bs],
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    for A, B, C in zip(As, Bs, outs):
        assert_f32(C, oracle.matmul(A, B), bar=1e-4)


def test_wide_several_tiles_per_cu():
    M, N, K = 12288, 6144, 64                 # 768 tiles: 3 per compute unit
    wide([(M, N)], K, epilogue="gelu")
    banner(f"wide tiles several waves M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 606, "x")
    W = gen((K, N), 1 / math.sqrt(K), 606, "A")
    bias = gen((N,), 0.5, 606, "bias", torch.float32)
    C = tts.tp_linear(X.to(DEV), W.to(DEV), bias.to(DEV), gelu=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16(C, oracle.gelu(oracle.matmul(X, W, bias)))


def test_wide_nan_row_stays_in_its_row():
    """A NaN in one row of X makes exactly that output row NaN (through the
    GeLU epilogue); an Inf in one weight column makes that column non-finite
    and leaves the rest exact."""
    M, N, K = 2304, 7680, 128
    wide([(M, N)], K, epilogue="gelu")
    banner(f"wide tiles NaN/Inf M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 607, "x")
    W = gen((K, N), 1 / math.sqrt(K), 607, "A")
    X[1000, 5] = float("nan")
    W[7, 5000] = float("inf")
    C = tts.tp_linear(X.to(DEV), W.to(DEV), gelu=True, out_dtype=torch.float32).cpu()
    bad_r = torch.isnan(C).all(dim=1)
    assert bad_r[1000] and bad_r.sum() == 1
    fin = torch.isfinite(C)
    fin[1000] = True
    assert not fin[:, 5000].all()
    fin[:, 5000] = True
    assert fin.all()
    keep = torch.ones(M, dtype=torch.bool)
    keep[1000] = False
    cols = torch.ones(N, dtype=torch.bool)
    cols[5000] = False
    ref = oracle.gelu(oracle.matmul(X[keep].contiguous(), W[:, cols].contiguous()))
    assert_f32(C[keep][:, cols], ref, bar=1e-4)


def test_wide_gelu_save_matches_narrow_kernel_bitwise():
    """The training forward's dual store: C = GeLU(v) and aux = v, both bf16."""
    M, N, K = 2304, 7680, 128
    wide([(M, N)], K, epilogue="gelu_save")
    banner(f"wide tiles gelu_save M={M} N={N} K={K}")
    X = gen((M, K), 1.0, 608, "x")
    W = gen((K, N), 1 / math.sqrt(K), 608, "A")
    bias = gen((N,), 0.5, 608, "bias", torch.float32)
    Xd, Wd, bd = X.to(DEV), W.to(DEV), bias.to(DEV)
    C, aux = tts.tp_matmul(Xd, Wd, bd, epilogue="gelu_save", out_dtype=torch.bfloat16)
    assert tts.tp_gemm_tile_cols([(256, N)], K, epilogue="gelu_save") == 256
    C0, aux0 = tts.tp_matmul(Xd[:256].contiguous(), Wd, bd, epilogue="gelu_save",
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(C[:256].view(torch.int16), C0.view(torch.int16))
    assert torch.equal(aux[:256].view(torch.int16), aux0.view(torch.int16))
    v = oracle.matmul(X, W, bias)
    assert_bf16(aux, v)
    assert_bf16(C, oracle.gelu(v))


def test_wide_nt_f32_ragged_matches_narrow_kernel_bitwise():
    """B stored [N,K] (the input-gradient layout dY·W^T), ragged M and N."""
    M, N, K = 2250, 7560, 192
    wide([(M, N)], K, trans_b=True)
    banner(f"wide tiles NT f32 M={M} N={N} K={K}")
    A = gen((M, K), 1.0, 609, "x")
    B = gen((N, K), 1 / math.sqrt(K), 609, "A")
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = tts.tp_matmul(Ad, Bd, trans_b=True, out_dtype=torch.float32)
    C0 = tts.tp_matmul(Ad[2048:].contiguous(), Bd, trans_b=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(C[2048:], C0)
    e = assert_f32(C, oracle.matmul(A, B.t().contiguous()), bar=1e-4)
    assert e["fro"] < 1e-5, e


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_wide_nt_gelu_bwd(out):
    """C = (A·B^T) ⊙ GeLU'(aux), the GeLU's backward with the saved
    pre-activation; N ragged against 384 and K over 17 K tiles."""
    M, N, K = 2304, 7560, 1088
    wide([(M, N)], K, trans_b=True, epilogue="gelu_bwd")
    banner(f"wide tiles NT gelu_bwd {out} M={M} N={N} K={K}")
    A = gen((M, K), 1.0, 610, "x")
    B = gen((N, K), 1 / math.sqrt(K), 610, "A")
    aux = gen((M, N), 1.0, 610, "preact")
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    Ad, Bd, auxd = A.to(DEV), B.to(DEV), aux.to(DEV)
    G = tts.tp_matmul(Ad, Bd, trans_b=True, epilogue="gelu_bwd", aux=auxd, out_dtype=odt)
    G0 = tts.tp_matmul(Ad[:256].contiguous(), Bd, trans_b=True, epilogue="gelu_bwd",
                       aux=auxd[:256].contiguous(), out_dtype=odt)
    torch.cuda.synchronize()
    assert torch.equal(G[:256], G0)
    ref = oracle.matmul(A, B.t().contiguous()) * oracle.gelu_grad(aux)
    if out == "bf16":
        assert_bf16(G, ref)
    else:
        assert_f32(G, ref, bar=1e-4)
