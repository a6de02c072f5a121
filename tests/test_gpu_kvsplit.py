"""GPU parity of the K/V-split attention (Q, K, V split along the feature
dimension over P ranks, partial scores summed before the softmax, each rank
its output slice) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_tensor_shard_amd as tts
from _tol import assert_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def banner(msg):
    print(f"\n[kv-split] {msg}", flush=True)


@pytest.mark.parametrize("b,s,H,d,P,causal", [
    (1, 256, 2, 128, 4, True),     # the d/P = 32 split, several 128x128 score tiles
    (2, 136, 1, 64, 2, False),     # ragged s (not a multiple of 64)
    (1, 64, 3, 128, 1, True),      # P = 1: plain attention
    (1, 128, 2, 128, 8, True),     # d/P = 16
    (3, 8, 2, 64, 8, False),       # tiny s, d/P = 8
    (1, 520, 20, 128, 4, True),    # 20 pairs: one partial chunk of pairs, ragged s
    (3, 136, 12, 128, 4, False),   # 36 pairs: a second chunk of pairs, ragged s
    (1, 2056, 2, 128, 4, True),    # s > 2048: the softmax's second row unit, wide score grids
])
def test_kv_split(b, s, H, d, P, causal):
    banner(f"b={b} s={s} H={H} d={d} P={P} causal={causal}")
    qkv = synth.normal((b * s, 3 * H * d), 1.0, 61, "x", torch.bfloat16)
    O = tts.tp_attention_kv_split(qkv.to(DEV), b, s, H, P, d, causal)
    torch.cuda.synchronize()
    assert_bf16(O, oracle.attention_kv_split_rows(qkv, b, s, H, d, P, causal), per_row=True)


def test_kv_split_strided_operands():
    """qkv with a row pitch wider than 3·H·d and O written into a wider buffer:
    the columns outside the head outputs stay untouched."""
    banner("strided operands")
    b, s, H, d, P = 2, 96, 2, 128, 4
    HD = H * d
    qkv_w = synth.normal((b * s, 3 * HD + 64), 1.0, 62, "x", torch.bfloat16)
    out = torch.full((b * s, HD + 128), 7.0, dtype=torch.bfloat16, device=DEV)
    tts.tp_attention_kv_split(qkv_w.to(DEV)[:, :3 * HD], b, s, H, P, d, True,
                              out=out[:, :HD])
    torch.cuda.synchronize()
    ref = oracle.attention_kv_split_rows(qkv_w[:, :3 * HD].contiguous(), b, s, H, d, P, True)
    assert_bf16(out[:, :HD], ref, per_row=True)
    assert torch.all(out[:, HD:] == 7.0)


def test_kv_split_agrees_with_head_sharded_core():
    """The feature-split and the head-sharded computations of one attention
    agree (both against the oracle, and with each other within bf16)."""
    banner("against the head-sharded core")
    b, s, H, d = 1, 192, 2, 128
    qkv = synth.normal((b * s, 3 * H * d), 1.0, 63, "x", torch.bfloat16).to(DEV)
    O_b = tts.tp_attention_kv_split(qkv, b, s, H, 4, d, True).float().cpu().numpy()
    O_a = tts.tp_attention_core(qkv, b, s, H, d, True).float().cpu().numpy()
    assert np.linalg.norm(O_a - O_b) <= 1e-2 * np.linalg.norm(O_a)


def test_kv_split_fullsize_sampled():
    """The benchmark's workload (4 sequences of 2048, 32 heads of 128, P = 4),
    launched as the benchmark launches it; every row of eight (sequence, head)
    pairs -- both sides of the 32-pair chunk boundary among them -- against
    the oracle, which computes each pair on its own."""
    from synth import workloads as wl
    w = wl.WORKLOADS["kvsplit_bf16_h4096_tp4"]
    b, s, H, d, P = w.b, w.s, w.H, w.d, w.P
    banner(f"{w.name}: b={b} s={s} H={H} d={d} P={P}")
    qkv = wl.kvsplit_inputs(w)
    O = tts.tp_attention_kv_split(qkv.to(DEV), b, s, H, P, d, True).cpu()
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    pairs = {(0, 0), (0, 31), (1, 0), (b - 1, H - 1)}
    while len(pairs) < 8:
        pairs.add((int(rng.integers(0, b)), int(rng.integers(0, H))))
    HD = H * d
    for beta, hd in sorted(pairs):
        rows = slice(beta * s, (beta + 1) * s)
        Q = qkv[rows, hd * d:(hd + 1) * d]
        K = qkv[rows, HD + hd * d:HD + (hd + 1) * d]
        V = qkv[rows, 2 * HD + hd * d:2 * HD + (hd + 1) * d]
        ref = oracle.attention_kv_split(Q, K, V, P, True)[1]
        assert_bf16(O[rows, hd * d:(hd + 1) * d], ref, per_row=True)
    assert torch.isfinite(O).all()


def test_kv_split_longest_sequence():
    """s = 8192, the longest sequence the K/V split accepts: one (sequence,
    head) pair, all rows against the oracle."""
    b, s, H, d, P = 1, 8192, 1, 128, 4
    banner(f"longest sequence: b={b} s={s} H={H} d={d} P={P}")
    qkv = synth.normal((b * s, 3 * H * d), 1.0, 64, "x", torch.bfloat16)
    O = tts.tp_attention_kv_split(qkv.to(DEV), b, s, H, P, d, True).cpu()
    torch.cuda.synchronize()
    ref = oracle.attention_kv_split(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], P, True)[1]
    assert_bf16(O, ref, per_row=True)
