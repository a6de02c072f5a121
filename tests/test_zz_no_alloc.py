"""The allocation-free MLP share (tp_mlp_shard_noalloc) through the C ABI.

It must give tp_mlp_shard's result bit for bit -- the same kernels on blocks
of token rows that fit the library's fixed scratch -- on consecutive calls
that share that scratch, the second one smaller, and meet the oracle's bars
("图解Transformer并行计算" §2.1: Z_i = GeLU(X·A_i + a_i)·B_i).
"""
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


def _inputs(M, h, f, seed, dtype, bias):
    X = synth.normal((M, h), 1.0, seed, "x", dtype)
    A = synth.normal((h, f), 1 / math.sqrt(h), seed, "A", dtype)
    B = synth.normal((f, h), 1 / math.sqrt(f), seed, "B", dtype)
    a = synth.normal((f,), 0.5, seed, "bias", torch.float32) if bias else None
    return X, A, B, a


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    cases = [
        # Y'_i is 2600 x 32768 bf16 = 170 MB: three row blocks of the 64 MiB
        # scratch (1024, 1024 and 552 rows)
        (2600, 256, 32768, torch.bfloat16, torch.float32, False),
        # then a smaller call into the same scratch, with a bias and bf16 output
        (300, 128, 1024, torch.bfloat16, torch.bfloat16, True),
        # and the f32 path (a rank of the tp=2 f32 MLP workload's shape)
        (32, 64, 128, torch.float32, torch.float32, False),
    ]
    for i, (M, h, f, dt, out_dt, bias) in enumerate(cases):
        banner(f"noalloc call {i}: M={M} h={h} f={f} in={dt} out={out_dt} bias={bias}")
        X, A, B, a = _inputs(M, h, f, 400 + i, dt, bias)
        Xd, Ad, Bd = X.to(DEV), A.to(DEV), B.to(DEV)
        ad = a.to(DEV) if a is not None else None
        Z_na = tts.tp_mlp_shard_noalloc(Xd, Ad, Bd, ad, out_dtype=out_dt)
        Z_ws = tts.tp_mlp_shard(Xd, Ad, Bd, ad, out_dtype=out_dt)
        torch.cuda.synchronize()
        assert torch.equal(Z_na, Z_ws), f"call {i} differs from tp_mlp_shard"
        rows = np.unique(np.r_[0, 1, 1023, 1024, 2047, 2048, M - 1,
                               np.random.default_rng(i).integers(0, M, 9)])
        rows = rows[rows < M]
        ref = oracle.mlp_shard(X[torch.from_numpy(rows)], A, B, a)
        got = Z_na.cpu()[torch.from_numpy(rows)]
        if dt == torch.float32:
            assert_f32(got, ref)
        else:
            assert_bf16(got, ref)


def test_noalloc_rejects_a_width_beyond_its_scratch():
    banner("noalloc f beyond the scratch")
    X = torch.zeros(8, 8, dtype=torch.bfloat16, device=DEV)
    A = torch.zeros(8, 131080, dtype=torch.bfloat16, device=DEV)
    B = torch.zeros(131080, 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tts.TpError) as e:
        tts.tp_mlp_shard_noalloc(X, A, B)
    assert e.value.status == 7
