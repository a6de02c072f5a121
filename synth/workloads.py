"""The synthetic workloads: shapes, value distributions and seeds.

Every input is N(0, sigma^2), drawn by ``synth.normal``; weights use
sigma = 1/sqrt(fan_in) with fan_in the UNSHARDED input width (h for A, W_qkv
and W_o; F for B).  Single-rank workloads draw rank 0's slice directly at the
slice shape.  Nothing here computes any part of the method; the FLOP counts
are the matrix-product counts used to report throughput (2 per multiply-add;
causal attention counts only the visible (query, key) pairs).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import normal, fan_in_sigma, rank_seed


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "mlp" | "attn" | "block" | "mlp_bwd" | "attn_bwd" | "vocab" | "kvsplit"
    seed: int
    P: int               # tensor-parallel degree
    b: int
    s: int
    h: int
    F: int = 0           # full FFN width
    H: int = 0           # total heads
    d: int = 128         # head dimension
    V: int = 0           # vocabulary size (vocab-parallel ends)
    dtype: torch.dtype = torch.bfloat16
    all_ranks: bool = False
    description: str = ""

    @property
    def M(self) -> int:
        return self.b * self.s

    @property
    def f(self) -> int:
        return self.F // self.P

    @property
    def Hl(self) -> int:
        return self.H // self.P

    # ---- matrix FLOPs ----------------------------------------------------
    def mlp_flops_rank(self) -> int:
        return 4 * self.M * self.h * self.f

    def attn_flops_rank(self) -> dict:
        qkv = 2 * self.M * self.h * 3 * self.Hl * self.d
        pairs = self.b * self.s * (self.s + 1) // 2
        core = 4 * self.Hl * self.d * pairs
        wo = 2 * self.M * self.Hl * self.d * self.h
        return {"qkv": qkv, "core": core, "wo": wo, "total": qkv + core + wo}

    def attn_bwd_flops_rank(self) -> dict:
        """Backward of one rank's attention share: the projections' input and
        weight gradients (two products each, of the forward's size) and the
        core's five products per visible (query, key) pair (S and dP
        recomputed, dV, dQ, dK: 10·d FLOPs per pair and head)."""
        f = self.attn_flops_rank()
        core = 10 * self.Hl * self.d * (self.b * self.s * (self.s + 1) // 2)
        return {"qkv": 2 * f["qkv"], "core": core, "wo": 2 * f["wo"],
                "total": 2 * f["qkv"] + core + 2 * f["wo"]}

    def kvsplit_bytes(self) -> int:
        """Minimum HBM bytes of the K/V-split attention under the causal mask:
        every rank's f32 partial scores of the visible (query, key) pairs
        written once (the exchange's message) and read once, the bf16 softmax
        weights of those pairs written and read, Q, K, V read and O written
        (the kernels move more: whole 256x256 score tiles on the diagonal and
        whole weight rows)."""
        s, pairs, vis = self.s, self.b * self.H, self.s * (self.s + 1) // 2
        per = 2 * 4 * self.P * vis + 2 * 2 * vis + 2 * 4 * s * self.d
        return pairs * per

    def flops(self) -> int:
        """Matrix FLOPs of one call of the workload's entry point."""
        if self.kind == "mlp":
            return self.mlp_flops_rank() * (self.P if self.all_ranks else 1)
        if self.kind == "mlp_bwd":
            # dY' = dZ·B^T, dB = Y'^T·dZ, dA = X^T·dY, dX = dY·A^T: 4 products
            return 2 * self.mlp_flops_rank()
        if self.kind == "attn":
            return self.attn_flops_rank()["total"]
        if self.kind == "attn_bwd":
            return self.attn_bwd_flops_rank()["total"]
        if self.kind == "vocab":
            return 2 * self.M * self.h * self.V       # the logits H·E^T of all ranks
        if self.kind == "kvsplit":
            # the attention's matrix FLOPs, as for the head-sharded core: 4·d
            # per visible (query, key) pair and head (the ranks' partial
            # scores together make up Q·K^T)
            return 4 * self.H * self.d * self.b * self.s * (self.s + 1) // 2
        return self.P * (self.mlp_flops_rank() + self.attn_flops_rank()["total"])


WORKLOADS = {w.name: w for w in [
    Workload("mlp_f32_h64_tp2", "mlp", 1000, P=2, b=2, s=16, h=64, F=256, dtype=torch.float32,
             all_ranks=True,
             description="fp32 MLP TP shard, tp=2 emulated sequentially, X [2,16,64]"),
    Workload("mlp_bf16_h4096_tp8", "mlp", 1001, P=8, b=8, s=1024, h=4096, F=16384,
             description="bf16 MLP, one rank of tp=8: A_i [4096,2048], B_i [2048,4096], 8192 tokens"),
    Workload("mlp_bf16_h12288_tp8", "mlp", 1002, P=8, b=8, s=2048, h=12288, F=49152,
             description="bf16 MLP, one rank of tp=8 at the 175B layer shape, 16384 tokens"),
    Workload("attn_bf16_h4096_tp4", "attn", 1003, P=4, b=4, s=2048, h=4096, H=32,
             description="bf16 causal self-attention, one rank of tp=4: 8 local heads of 128"),
    Workload("mlp_bwd_bf16_h12288_tp8", "mlp_bwd", 1005, P=8, b=8, s=2048, h=12288, F=49152,
             description="bf16 backward of one rank's MLP share of tp=8 at the 175B layer "
                         "shape, 16384 tokens: dA_i, dB_i, da_i and the dX_i partial"),
    Workload("attn_bwd_bf16_h12288_tp8", "attn_bwd", 1006, P=8, b=8, s=2048, h=12288, H=96,
             description="bf16 backward of one rank's causal attention share of tp=8 at the "
                         "175B layer shape (12 local heads of 128, 8 sequences of 2048): "
                         "dW_qkv,i, dW_o,i and the dX_i partial"),
    Workload("vocab_bf16_h12288_tp8", "vocab", 1007, P=8, b=8, s=2048, h=12288, V=51200,
             all_ranks=True,
             description="bf16 vocab-parallel ends at the 175B layer shape, all 8 ranks of tp=8: "
                         "embedding lookup of 16384 tokens and the stable cross-entropy over "
                         "V = 51200 (GPT-3's 50257 padded to a multiple of 128·8), table tied"),
    Workload("kvsplit_bf16_h4096_tp4", "kvsplit", 1008, P=4, b=4, s=2048, h=4096, H=32,
             all_ranks=True,
             description="bf16 causal self-attention with Q, K, V split along the feature "
                         "dimension over tp=4 (32 of each head's 128 features per rank, the "
                         "ranks' partial scores summed before the softmax), all 4 ranks: 4 "
                         "sequences of 2048, 32 heads, the head-sharded tp=4 attention shape"),
    Workload("block_bf16_h12288_tp8", "block", 1004, P=8, b=8, s=2048, h=12288, H=96, F=49152,
             all_ranks=True,
             description="bf16 pre-LN block at the 175B layer shape, all 8 ranks of tp=8 in turn"),
]}


def mlp_inputs(w: Workload):
    """X and the full (all-rank) or rank-0 A/B of an MLP workload, on the CPU."""
    X = normal((w.M, w.h), 1.0, w.seed, "x", w.dtype)
    width = w.F if w.all_ranks else w.f
    A = normal((w.h, width), fan_in_sigma(w.h), w.seed, "A", w.dtype)
    B = normal((width, w.h), fan_in_sigma(w.F), w.seed, "B", w.dtype)
    return X, A, B


def attn_inputs(w: Workload):
    """X, W_qkv_0 [h, 3·H_l·d] and W_o_0 [H_l·d, h] of an attention workload."""
    X = normal((w.M, w.h), 1.0, w.seed, "x", w.dtype)
    Wqkv = normal((w.h, 3 * w.Hl * w.d), fan_in_sigma(w.h), w.seed, "Wqkv", w.dtype)
    Wo = normal((w.Hl * w.d, w.h), fan_in_sigma(w.h), w.seed, "Wo", w.dtype)
    return X, Wqkv, Wo


def block_input(w: Workload):
    return normal((w.M, w.h), 1.0, w.seed, "x", w.dtype)


def block_rank_weights(w: Workload, r: int):
    """Rank r's W_qkv_r, W_o_r, A_r, B_r of a block workload, on the CPU."""
    sd = rank_seed(w.seed, r)
    Wqkv = normal((w.h, 3 * w.Hl * w.d), fan_in_sigma(w.h), sd, "Wqkv", w.dtype)
    Wo = normal((w.Hl * w.d, w.h), fan_in_sigma(w.h), sd, "Wo", w.dtype)
    A = normal((w.h, w.f), fan_in_sigma(w.h), sd, "A", w.dtype)
    B = normal((w.f, w.h), fan_in_sigma(w.F), sd, "B", w.dtype)
    return Wqkv, Wo, A, B


def mlp_bwd_inputs(w: Workload):
    """X, rank 0's A_i, B_i, a zero bias a_i and the upstream gradient dZ of
    an MLP backward workload, on the CPU.  dZ ~ N(0, 1): the gradient of a
    loss that weighs every output element alike."""
    X = normal((w.M, w.h), 1.0, w.seed, "x", w.dtype)
    A = normal((w.h, w.f), fan_in_sigma(w.h), w.seed, "A", w.dtype)
    B = normal((w.f, w.h), fan_in_sigma(w.F), w.seed, "B", w.dtype)
    a = torch.zeros(w.f, dtype=torch.float32)
    dZ = normal((w.M, w.h), 1.0, w.seed, "dZ", w.dtype)
    return X, A, B, a, dZ


def attn_bwd_inputs(w: Workload):
    """X, rank 0's W_qkv_0, W_o_0 and the upstream gradient dZ ~ N(0, 1) of an
    attention backward workload, on the CPU."""
    X, Wqkv, Wo = attn_inputs(w)
    dZ = normal((w.M, w.h), 1.0, w.seed, "dZ", w.dtype)
    return X, Wqkv, Wo, dZ


def kvsplit_inputs(w: Workload):
    """The fused projection qkv [M, 3·H·d] ~ N(0, 1) (the entries of X·W_qkv
    for X ~ N(0, 1) and W ~ N(0, 1/h)), on the CPU."""
    return normal((w.M, 3 * w.H * w.d), 1.0, w.seed, "x", w.dtype)


def vocab_inputs(w: Workload):
    """Token ids and targets (uniform on [0, V), int32), the final hidden
    states H ~ N(0, 1) [M, h] and the tied table E ~ N(0, 0.02^2) [V, h] (the
    usual embedding initialisation; logits then have std 0.02·sqrt(h)), on the
    CPU."""
    from . import token_ids
    tokens = token_ids(w.M, w.V, w.seed, "tokens")
    targets = token_ids(w.M, w.V, w.seed, "targets")
    H = normal((w.M, w.h), 1.0, w.seed, "x", w.dtype)
    E = normal((w.V, w.h), 0.02, w.seed, "E", w.dtype)
    return tokens, targets, H, E
