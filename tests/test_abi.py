"""The C ABI of libtp.so on the CPU: it loads, exports every symbol that
include/tp.h declares, binds to torch's HIP runtime, and rejects bad
arguments with the documented status before launching anything (no compute
call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

import transformer_tensor_shard_amd as tts
from transformer_tensor_shard_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp.h")

FAKE = ctypes.c_void_p(0x100000)        # aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x100004)    # 4-byte aligned only
BIG = 1 << 40


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (tp_\w+)", out))
    assert set(names) == exported, (set(names) ^ exported)
    assert set(names) == set(_lib.SIGNATURES)


def test_loads_and_reports_version():
    L = tts.lib()
    assert L.tp_abi_version() == 2
    assert L.tp_status_string(0) == b"ok"
    assert L.tp_status_string(99) == b"unknown status"


def test_single_hip_runtime_mapped():
    tts.lib()
    maps = open("/proc/self/maps").read()
    libs = {m for m in re.findall(r"(\S*libamdhip64[^\s]*)", maps)}
    assert len({os.path.realpath(p) for p in libs}) == 1, libs


def mlp(**kw):
    a = dict(X=FAKE, A=FAKE, a=None, B=FAKE, Z=FAKE, ws=FAKE, wsb=BIG, M=64, h=64, f=32,
             i=_lib.TP_BF16, o=_lib.TP_F32)
    a.update(kw)
    return tts.lib().tp_mlp_shard(a["X"], a["A"], a["a"], a["B"], a["Z"], a["ws"], a["wsb"],
                                  a["M"], a["h"], a["f"], a["i"], a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _lib.TP_ERR_NULL),
    (dict(B=None), _lib.TP_ERR_NULL),
    (dict(M=0), _lib.TP_ERR_SHAPE),            # empty input is rejected, not launched
    (dict(f=-8), _lib.TP_ERR_SHAPE),
    (dict(h=12), _lib.TP_ERR_SHAPE),           # bf16 rows must be 16-byte multiples
    (dict(i=7), _lib.TP_ERR_DTYPE),
    (dict(o=2), _lib.TP_ERR_DTYPE),
    (dict(A=FAKE_ODD), _lib.TP_ERR_ALIGN),
    (dict(ws=None), _lib.TP_ERR_WORKSPACE),
    (dict(wsb=16), _lib.TP_ERR_WORKSPACE),
])
def test_mlp_shard_rejects(kw, status):
    assert mlp(**kw) == status


def mlp_noalloc(**kw):
    a = dict(X=FAKE, A=FAKE, a=None, B=FAKE, Z=FAKE, M=64, h=64, f=32, i=_lib.TP_BF16,
             o=_lib.TP_F32)
    a.update(kw)
    return tts.lib().tp_mlp_shard_noalloc(a["X"], a["A"], a["a"], a["B"], a["Z"], a["M"], a["h"],
                                          a["f"], a["i"], a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _lib.TP_ERR_NULL),
    (dict(M=0), _lib.TP_ERR_SHAPE),
    (dict(h=12), _lib.TP_ERR_SHAPE),
    (dict(o=2), _lib.TP_ERR_DTYPE),
    (dict(Z=FAKE_ODD), _lib.TP_ERR_ALIGN),
    # Y'_i of one 256-row tile must fit the fixed 64 MiB scratch
    (dict(f=131080), _lib.TP_ERR_SCRATCH),
    (dict(f=65544, i=_lib.TP_F32), _lib.TP_ERR_SCRATCH),
])
def test_mlp_shard_noalloc_rejects(kw, status):
    assert mlp_noalloc(**kw) == status
    assert b"scratch" in tts.lib().tp_status_string(_lib.TP_ERR_SCRATCH)


def test_mlp_workspace_size():
    L = tts.lib()
    assert L.tp_mlp_shard_workspace(100, 64, _lib.TP_BF16) == 12800
    assert L.tp_mlp_shard_workspace(100, 64, _lib.TP_F32) == 25600
    assert L.tp_mlp_shard_workspace(0, 64, _lib.TP_F32) == 0


def attn(**kw):
    a = dict(X=FAKE, Wqkv=FAKE, Wo=FAKE, Z=FAKE, ws=FAKE, wsb=BIG, b=2, s=64, h=512, Hl=4, d=128,
             causal=1, o=_lib.TP_F32)
    a.update(kw)
    return tts.lib().tp_attn_shard(a["X"], a["Wqkv"], a["Wo"], a["Z"], a["ws"], a["wsb"], a["b"],
                                   a["s"], a["h"], a["Hl"], a["d"], a["causal"], a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Wo=None), _lib.TP_ERR_NULL),
    (dict(d=64), _lib.TP_ERR_SHAPE),            # the kernel's head tile is 128
    (dict(s=0), _lib.TP_ERR_SHAPE),
    (dict(h=500), _lib.TP_ERR_SHAPE),
    (dict(o=3), _lib.TP_ERR_DTYPE),
    (dict(Z=FAKE_ODD), _lib.TP_ERR_ALIGN),
    (dict(wsb=1024), _lib.TP_ERR_WORKSPACE),
])
def test_attn_shard_rejects(kw, status):
    assert attn(**kw) == status


def test_partial_sum_rejects():
    L = tts.lib()
    assert L.tp_partial_sum(None, 0, FAKE, 0, 2, 4, 8, None, None, 0, None) == _lib.TP_ERR_NULL
    assert L.tp_partial_sum(FAKE, 0, FAKE, 0, 0, 4, 8, None, None, 0, None) == _lib.TP_ERR_SHAPE
    assert L.tp_partial_sum(FAKE, 0, FAKE, 0, 2, 4, 6, None, None, 0, None) == _lib.TP_ERR_SHAPE
    assert L.tp_partial_sum(FAKE, 0, FAKE, 9, 2, 4, 8, None, None, 0, None) == _lib.TP_ERR_DTYPE
    assert L.tp_partial_sum(FAKE, 0, FAKE, 0, 2, 4, 8, FAKE_ODD, None, 0, None) == _lib.TP_ERR_ALIGN


def block(**kw):
    P = kw.pop("P", 2)
    arr = (ctypes.c_void_p * P)(*([FAKE.value] * P))
    a = dict(x=FAKE, out=FAKE, x1=None, eps=1e-5, W=arr, ws=FAKE, wsb=BIG, b=1, s=64, h=512,
             H=4, d=128, F=1024)
    a.update(kw)
    return tts.lib().tp_block_shard(a["x"], a["out"], _lib.TP_F32, a["x1"], None, None, None,
                                    None, a["eps"], a["W"], a["W"], a["W"], a["W"], P, a["ws"],
                                    a["wsb"], a["b"], a["s"], a["h"], a["H"], a["d"], a["F"], None)


def test_block_shard_rejects():
    assert block(h=640) == _lib.TP_ERR_SHAPE          # h != H*d
    assert block(P=3) == _lib.TP_ERR_SHAPE             # H=4 does not divide by 3
    assert block(F=1000) == _lib.TP_ERR_SHAPE
    assert block(eps=0.0) == _lib.TP_ERR_SHAPE
    arr = (ctypes.c_void_p * 2)(FAKE.value, None)
    assert block(W=arr) == _lib.TP_ERR_NULL
    assert block(wsb=100) == _lib.TP_ERR_WORKSPACE


def test_block_workspace_grows_with_ranks():
    L = tts.lib()
    w2 = L.tp_block_shard_workspace(1, 64, 512, 4, 128, 1024, 2)
    w4 = L.tp_block_shard_workspace(1, 64, 512, 4, 128, 1024, 4)
    assert w4 > w2 > 0
    assert L.tp_block_shard_workspace(1, 64, 512, 4, 128, 1024, 3) == 0


def test_linear_and_layernorm_reject():
    L = tts.lib()
    assert L.tp_linear(FAKE, 8, FAKE, 8, None, FAKE, 8, 4, 8, 16, 1, 0, 0, None) == _lib.TP_ERR_SHAPE
    assert L.tp_linear(FAKE, 16, FAKE, 8, None, FAKE, 8, 4, 8, 16, 1, 0, 5, None) == _lib.TP_ERR_DTYPE
    assert L.tp_layernorm(FAKE, 1, FAKE, None, None, 1e-5, 4, 20, None) == _lib.TP_ERR_SHAPE
    assert L.tp_layernorm(FAKE, 1, FAKE, None, None, 1e-5, 4, 1 << 20, None) == _lib.TP_ERR_SHAPE
    assert L.tp_attention_core(FAKE, 100, FAKE, 1, 8, 1, 128, 1, None) == _lib.TP_ERR_SHAPE


def test_python_binding_raises_valueerror_on_shape():
    import torch
    with pytest.raises(ValueError):
        tts._check(_lib.TP_ERR_SHAPE, "x")
    with pytest.raises(tts.TpError):
        tts._check(_lib.TP_ERR_LAUNCH, "x")
    with pytest.raises(ValueError):
        tts._dev(torch.zeros(2), "cpu tensor")


def test_linear_batched_rejects():
    L = tts.lib()
    two = (ctypes.c_void_p * 2)(FAKE.value, FAKE.value)
    hole = (ctypes.c_void_p * 2)(FAKE.value, None)
    odd = (ctypes.c_void_p * 2)(FAKE.value, FAKE_ODD.value)
    call = lambda X=two, W=two, C=two, count=2, K=16, epi=0: L.tp_linear_batched(
        X, K, W, 8, None, C, 8, count, 4, 8, K, _lib.TP_BF16, _lib.TP_F32, epi, None)
    assert call(count=0) == _lib.TP_ERR_SHAPE
    assert call(W=hole) == _lib.TP_ERR_NULL
    assert call(C=hole) == _lib.TP_ERR_NULL
    assert call(K=12) == _lib.TP_ERR_SHAPE          # bf16 needs K % 8 == 0
    assert call(epi=5) == _lib.TP_ERR_DTYPE
    assert call(X=odd) == _lib.TP_ERR_ALIGN
    assert L.tp_linear_batched(None, 16, two, 8, None, two, 8, 2, 4, 8, 16, 1, 0, 0, None) \
        == _lib.TP_ERR_NULL


def matmul(**kw):
    a = dict(A=FAKE, lda=64, ta=0, B=FAKE, ldb=64, tb=0, bias=None, C=FAKE, ldc=64, aux=None,
             ldaux=0, M=32, N=64, K=64, o=_lib.TP_F32, epi=_lib.TP_EPI_NONE)
    a.update(kw)
    return tts.lib().tp_matmul(a["A"], a["lda"], a["ta"], a["B"], a["ldb"], a["tb"], a["bias"],
                               a["C"], a["ldc"], a["aux"], a["ldaux"], a["M"], a["N"], a["K"],
                               a["o"], a["epi"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), _lib.TP_ERR_NULL),
    (dict(C=None), _lib.TP_ERR_NULL),
    (dict(ta=1, tb=1), _lib.TP_ERR_DTYPE),                 # A^T·B^T has no kernel
    (dict(ta=2), _lib.TP_ERR_DTYPE),
    (dict(ta=1, epi=_lib.TP_EPI_GELU), _lib.TP_ERR_DTYPE),  # TN takes no epilogue
    (dict(epi=_lib.TP_EPI_GELU_BWD), _lib.TP_ERR_DTYPE),    # GeLU backward is NT only
    (dict(epi=_lib.TP_EPI_GELU_SAVE, aux=FAKE, ldaux=64), _lib.TP_ERR_DTYPE),  # needs bf16 out
    (dict(tb=1, epi=_lib.TP_EPI_GELU_BWD), _lib.TP_ERR_NULL),  # aux missing
    (dict(o=5), _lib.TP_ERR_DTYPE),
    (dict(M=0), _lib.TP_ERR_SHAPE),
    (dict(K=60, lda=64), _lib.TP_ERR_SHAPE),               # NN: K is A's contiguous dim
    (dict(ta=1, lda=32, M=28, K=60), _lib.TP_ERR_SHAPE),   # TN: M is A's contiguous dim
    (dict(tb=1, ldb=64, N=60), _lib.TP_ERR_SHAPE),         # C's rows must be 16-byte multiples
    (dict(ldc=60), _lib.TP_ERR_SHAPE),
    (dict(lda=32), _lib.TP_ERR_SHAPE),                     # lda < K
    (dict(tb=1, ldb=32), _lib.TP_ERR_SHAPE),               # B^T stored [N,K]: ldb < K
    (dict(ta=1, lda=16), _lib.TP_ERR_SHAPE),               # A^T stored [K,M]: lda < M
    (dict(lda=1 << 23), _lib.TP_ERR_SHAPE),                # 256 rows past 32-bit offsets
    (dict(tb=1, epi=_lib.TP_EPI_GELU_BWD, aux=FAKE, ldaux=1 << 23), _lib.TP_ERR_SHAPE),  # aux rows too
    (dict(B=FAKE_ODD), _lib.TP_ERR_ALIGN),
    (dict(tb=1, epi=_lib.TP_EPI_GELU_BWD, aux=FAKE_ODD, ldaux=64), _lib.TP_ERR_ALIGN),
])
def test_matmul_rejects(kw, status):
    assert matmul(**kw) == status


def test_matmul_accepts_the_documented_forms_on_cpu_arguments():
    """Every supported (trans_a, trans_b, epilogue) passes validation: with a
    NULL A it must fail on the pointer, not on the form."""
    for ta, tb, epi, o in [(0, 0, 0, 0), (0, 0, 1, 1), (0, 0, 3, 1), (0, 1, 0, 0), (0, 1, 2, 1),
                           (1, 0, 0, 0), (1, 0, 0, 1)]:
        assert matmul(A=None, ta=ta, tb=tb, epi=epi, o=o, aux=FAKE, ldaux=64) == _lib.TP_ERR_NULL


def mlp_bwd(**kw):
    a = dict(X=FAKE, A=FAKE, B=FAKE, Y=FAKE, Yp=FAKE, dZ=FAKE, dX=FAKE, dA=FAKE, dB=FAKE,
             da=FAKE, ws=FAKE, wsb=BIG, M=300, h=64, f=32, o=_lib.TP_F32)
    a.update(kw)
    return tts.lib().tp_mlp_shard_backward(a["X"], a["A"], a["B"], a["Y"], a["Yp"], a["dZ"],
                                           a["dX"], a["dA"], a["dB"], a["da"], a["ws"], a["wsb"],
                                           a["M"], a["h"], a["f"], a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Y=None), _lib.TP_ERR_NULL),
    (dict(dB=None), _lib.TP_ERR_NULL),
    (dict(o=4), _lib.TP_ERR_DTYPE),
    (dict(M=0), _lib.TP_ERR_SHAPE),
    (dict(h=60), _lib.TP_ERR_SHAPE),
    (dict(f=12), _lib.TP_ERR_SHAPE),
    (dict(M=65536 * 256 + 1), _lib.TP_ERR_SHAPE),   # more bias-sum chunks than a grid column
    (dict(ws=None), _lib.TP_ERR_WORKSPACE),
    (dict(wsb=300 * 32 * 2), _lib.TP_ERR_WORKSPACE),  # dY fits, the bias partials do not
    (dict(dA=FAKE_ODD), _lib.TP_ERR_ALIGN),
    (dict(da=FAKE_ODD), _lib.TP_ERR_ALIGN),
])
def test_mlp_backward_rejects(kw, status):
    assert mlp_bwd(**kw) == status


def test_mlp_backward_workspace_size():
    L = tts.lib()
    # dY: 300*32*2 = 19200 bytes (a multiple of 256); partials: 2 chunks * 32 * 4 -> 256
    assert L.tp_mlp_shard_backward_workspace(300, 32) == 19200 + 256
    assert L.tp_mlp_shard_backward_workspace(0, 32) == 0


def test_mlp_train_fwd_rejects():
    L = tts.lib()
    call = lambda Y=FAKE, Yp=FAKE, h=64, o=_lib.TP_F32: L.tp_mlp_shard_train_fwd(
        FAKE, FAKE, None, FAKE, FAKE, Y, Yp, 100, h, 32, o, None)
    assert call(Y=None) == _lib.TP_ERR_NULL
    assert call(Yp=None) == _lib.TP_ERR_NULL
    assert call(h=20) == _lib.TP_ERR_SHAPE
    assert call(o=9) == _lib.TP_ERR_DTYPE
    assert call(Yp=FAKE_ODD) == _lib.TP_ERR_ALIGN


def test_matmul_grouped_rejects():
    L = tts.lib()
    P2 = ctypes.c_void_p * 2
    I2 = ctypes.c_int64 * 2
    ok, hole = P2(FAKE.value, FAKE.value), P2(FAKE.value, None)
    odd = P2(FAKE.value, FAKE_ODD.value)
    call = lambda A=ok, lda=I2(64, 128), ta=1, C=ok, M=I2(64, 128), N=I2(32, 64), count=2, K=100, \
        ws=None: \
        L.tp_matmul_grouped(A, lda, ta, ok, I2(64, 64), 0, C, I2(64, 64), M, N, count, K,
                            _lib.TP_F32, ws, 1 << 20, None)
    assert call(A=hole) == _lib.TP_ERR_NULL
    assert call(count=0) == _lib.TP_ERR_SHAPE
    assert call(count=17) == _lib.TP_ERR_SHAPE
    assert call(M=I2(64, 60)) == _lib.TP_ERR_SHAPE      # TN: M is A's contiguous dimension
    assert call(lda=I2(64, 32)) == _lib.TP_ERR_SHAPE    # group 1's lda < M
    assert call(ta=2) == _lib.TP_ERR_DTYPE
    assert call(C=odd) == _lib.TP_ERR_ALIGN
    assert call(ws=FAKE_ODD) == _lib.TP_ERR_ALIGN        # the optional workspace, misaligned
    assert L.tp_matmul_grouped(None, I2(64, 64), 1, ok, I2(64, 64), 0, ok, I2(64, 64), I2(64, 64),
                               I2(64, 64), 2, 64, 0, None, 0, None) == _lib.TP_ERR_NULL


def test_vocab_rejects():
    L = tts.lib()
    T4 = ctypes.c_void_p(0x100000)          # 4-byte aligned token ids
    T_odd = ctypes.c_void_p(0x100002)
    emb = lambda tok=T4, M=10, V=64, h=32, o=_lib.TP_F32, out=FAKE: L.tp_vocab_embedding_shard(
        tok, M, FAKE, V, h, 0, out, o, None)
    assert emb(tok=None) == _lib.TP_ERR_NULL
    assert emb(M=0) == _lib.TP_ERR_SHAPE
    assert emb(h=20) == _lib.TP_ERR_SHAPE
    assert emb(V=60) == _lib.TP_ERR_SHAPE
    assert emb(o=3) == _lib.TP_ERR_DTYPE
    assert emb(tok=T_odd) == _lib.TP_ERR_ALIGN
    assert emb(out=FAKE_ODD) == _lib.TP_ERR_ALIGN
    ce = lambda H=FAKE, V=64, stats=FAKE, ws=FAKE, wsb=BIG: L.tp_vocab_ce_shard(
        H, FAKE, T4, 10, 32, V, 0, stats, ws, wsb, None)
    assert ce(H=None) == _lib.TP_ERR_NULL
    assert ce(V=12) == _lib.TP_ERR_SHAPE
    assert ce(ws=None) == _lib.TP_ERR_WORKSPACE
    assert ce(wsb=8) == _lib.TP_ERR_WORKSPACE
    assert ce(stats=FAKE_ODD) == _lib.TP_ERR_ALIGN
    assert L.tp_vocab_ce_shard_workspace(300, 520) == 12032  # 300 rows x 5 pieces of 128 columns x 8 B, to 256 B
    assert L.tp_vocab_ce_combine(None, 2, 10, FAKE, None, None) == _lib.TP_ERR_NULL
    assert L.tp_vocab_ce_combine(FAKE, 0, 10, FAKE, None, None) == _lib.TP_ERR_SHAPE
    two = (ctypes.c_void_p * 2)(FAKE.value, FAKE.value)
    hole = (ctypes.c_void_p * 2)(FAKE.value, None)
    par = lambda E=two, P=2, wsb=BIG: L.tp_vocab_parallel_ce(FAKE, E, P, T4, 10, 32, 64, FAKE,
                                                             None, FAKE, wsb, None)
    assert par(E=hole) == _lib.TP_ERR_NULL
    assert par(P=0) == _lib.TP_ERR_SHAPE
    assert par(wsb=100) == _lib.TP_ERR_WORKSPACE
    assert L.tp_vocab_parallel_ce_workspace(10, 64, 2) > 0


def test_kv_split_rejects():
    L = tts.lib()
    kv = lambda qkv=FAKE, ld=3 * 4 * 128, O=FAKE, ldo=4 * 128, b=2, s=64, H=4, d=128, P=4, \
        ws=FAKE, wsb=BIG: L.tp_attention_kv_split(qkv, ld, O, ldo, b, s, H, d, P, 1, ws, wsb, None)
    assert kv(qkv=None) == _lib.TP_ERR_NULL
    assert kv(O=None) == _lib.TP_ERR_NULL
    assert kv(P=3) == _lib.TP_ERR_SHAPE          # d not divisible by P
    assert kv(P=32) == _lib.TP_ERR_SHAPE         # d/P = 4 features: not a 16-byte slice
    assert kv(s=60) == _lib.TP_ERR_SHAPE         # s % 8
    assert kv(s=8200) == _lib.TP_ERR_SHAPE       # rows longer than 8192
    assert kv(ld=3 * 4 * 128 - 8) == _lib.TP_ERR_SHAPE
    assert kv(ldo=4 * 128 - 8) == _lib.TP_ERR_SHAPE
    assert kv(b=0) == _lib.TP_ERR_SHAPE
    assert kv(ws=None) == _lib.TP_ERR_WORKSPACE
    assert kv(wsb=1024) == _lib.TP_ERR_WORKSPACE
    assert kv(O=FAKE_ODD) == _lib.TP_ERR_ALIGN
    assert kv(ws=FAKE_ODD) == _lib.TP_ERR_ALIGN


def test_kv_split_workspace_size():
    L = tts.lib()
    # 32 pairs at most in flight
    # per pair: P f32 partial-score matrices stored as 128 x 128 tiles (s
    # rounded up to a multiple of 128), a bf16 weight matrix of s x s, the f32
    # product with V [s, d] and the row sums [s]
    assert L.tp_attention_kv_split_workspace(2, 64, 4, 128, 4) == \
        8 * (4 * 4 * 128 * 128 + 2 * 64 * 64 + 64 * 516)
    assert L.tp_attention_kv_split_workspace(1, 136, 1, 64, 2) == \
        1 * (4 * 2 * 256 * 256 + 2 * 136 * 136 + 136 * 260)
    assert L.tp_attention_kv_split_workspace(4, 2048, 32, 128, 4) == \
        32 * (2048 * 2048 * 18 + 2048 * 516)
    assert L.tp_attention_kv_split_workspace(0, 64, 4, 128, 4) == 0
