"""fp64 CPU oracle for one tensor-parallel rank's share of a Transformer block.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It never imports the HIP library
and the HIP library never imports it.

The matrix products X·W are float64 library matmuls (numpy / OpenBLAS); the
other steps -- exact-erf GeLU, LayerNorm, the per-head softmax attention and
the partial sum -- are plain float64 loops in ``tp_oracle.c``.  This module
converts the shared seeded inputs to float64 exactly and composes those steps
in the order the pages give:

* ``mlp_shard``   -- Y_i = X·A_i (+a_i), GeLU locally, Z_i = GeLU(Y_i)·B_i
  ("图解Transformer并行计算" (un.csdn.net/7y5fj9k05scw) §2.1, §2.2);
* ``attn_shard_rows`` -- local heads' softmax(QK^T/sqrt d)·V, then the row
  slice of W_o (same page §3.1, §3.2);
* ``partial_sum`` -- Z = sum_r Z_r (+ bias) (+ residual): the all-reduce's
  arithmetic (same page §1.1, §2.1);
* ``mlp_shard_backward``, ``attention_backward``, ``attn_shard_backward`` --
  the gradients of the MLP and attention shares by the chain rule (same page
  §2.2 and §3.2, backward: same upstream gradient on every rank, local
  parameter gradients, a partial input gradient summed over ranks);
* ``attention_kv_split`` -- attention with Q, K, V split along the feature
  dimension: partial scores summed over ranks before the softmax, each rank
  the feature slice of the output (ops-transformer article
  (intelliparadigm.com/article/weixin_42537919/2252113) §3.1, strategy B);
* ``vocab_embedding_shard``, ``vocab_ce_shard_stats``, ``vocab_ce_combine`` --
  the vocab-parallel input embedding and the stable parallel cross-entropy
  (same page §4.1, §4.2);
* ``block_rows``  -- the pre-LN block x + attn(LN1(x)), then + mlp(LN2(.)), as
  assembled in section 3.3 of the PyTorch tensor-parallel tutorial
  (hotelren.com/news/6074135), with every rank's share summed.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_gelu.argtypes = [ctypes.c_double]
    lib.orc_gelu.restype = ctypes.c_double
    lib.orc_gelu_inplace.argtypes = [_dp, _i64]
    lib.orc_gelu_grad.argtypes = [ctypes.c_double]
    lib.orc_gelu_grad.restype = ctypes.c_double
    lib.orc_gelu_grad_inplace.argtypes = [_dp, _i64]
    lib.orc_layernorm.argtypes = [_dp, _dp, _dp, ctypes.c_double, _dp, _i64, _i64]
    lib.orc_attention_rows.argtypes = [_dp, _dp, _dp, ctypes.POINTER(_i64), _i64, _i64, _i64,
                                       _i64, ctypes.c_int, _dp]
    lib.orc_partial_sum.argtypes = [_dp, _i64, _i64, _i64, _dp, _dp, _dp]
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """Host threads the oracle's loops use (OpenMP's count)."""
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------- conversion
def f64(t) -> np.ndarray:
    """Exact float64 copy of a CPU tensor/array stored as bf16, fp32 or fp64.

    bf16 is widened by placing its 16 bits in the top half of an IEEE binary32
    word, which is exact; binary32 and binary64 widen exactly as well.
    """
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                bits = t.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32)
                with np.errstate(invalid="ignore"):     # NaN payloads widen quietly
                    return np.ascontiguousarray((bits << 16).view(np.float32).astype(np.float64))
            return np.ascontiguousarray(t.numpy().astype(np.float64))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_dp)


# ---------------------------------------------------------------- primitives
def matmul(X, W, bias=None) -> np.ndarray:
    """Y = X·W (+bias) in float64; X [M,K], W [K,N].

    "图解Transformer并行计算" §1: Y = X @ W with W of shape [h, h'].  The
    product is a library float64 matmul (numpy); the bias is added after it.
    """
    X, W, bias = f64(X), f64(W), f64(bias)
    assert X.ndim == 2 and W.ndim == 2 and X.shape[1] == W.shape[0]
    Y = np.matmul(X, W)
    if bias is not None:
        Y += bias
    return np.ascontiguousarray(Y)


def gelu(x) -> np.ndarray:
    """Exact-erf GeLU applied elementwise."""
    y = np.array(f64(x), dtype=np.float64, copy=True, order="C")
    _load().orc_gelu_inplace(_p(y), y.size)
    return y


def gelu_scalar(x: float) -> float:
    return float(_load().orc_gelu(float(x)))


def layernorm(x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm of each row of x [M,h] (population variance)."""
    x, gamma, beta = f64(x), f64(gamma), f64(beta)
    M, h = x.shape
    y = np.empty_like(x)
    _load().orc_layernorm(_p(x), _p(gamma), _p(beta), float(eps), _p(y), M, h)
    return y


def mlp_shard(X, A_i, B_i, a_i=None) -> np.ndarray:
    """One rank's MLP share, "图解Transformer并行计算" §2.1 / §2.2:
    Y_i = X·A_i (+a_i), Y'_i = GeLU(Y_i) locally, Z_i = Y'_i·B_i (a partial
    sum).  X [M,h], A_i [h,f], B_i [f,h]."""
    X, A_i, B_i = f64(X), f64(A_i), f64(B_i)
    M, h = X.shape
    f = A_i.shape[1]
    assert A_i.shape == (h, f) and B_i.shape == (f, h)
    return matmul(gelu(matmul(X, A_i, a_i)), B_i)


def gelu_grad(x) -> np.ndarray:
    """Derivative of the exact-erf GeLU, elementwise: Phi(x) + x·phi(x)."""
    y = np.array(f64(x), dtype=np.float64, copy=True, order="C")
    _load().orc_gelu_grad_inplace(_p(y), y.size)
    return y


def mlp_shard_backward(X, A_i, B_i, dZ, a_i=None):
    """Gradients of one rank's MLP share Z_i = GeLU(X·A_i + a_i)·B_i.

    "图解Transformer并行计算" §2.2: the backward mirrors the forward.  Every
    rank receives the same upstream gradient dZ of the summed output, computes
    the gradients of its own A_i and B_i, and forms a local input gradient
    dX_i; one all-reduce sums them, dX = sum_r dX_r.  By the chain rule, with
    Y = X·A_i + a_i, Y' = GeLU(Y):
        dB_i = Y'^T·dZ                     [f, h]
        dY'  = dZ·B_i^T                    [M, f]
        dY   = dY' ⊙ GeLU'(Y)             (local, like the forward GeLU)
        dA_i = X^T·dY,   da_i = sum over rows of dY
        dX_i = dY·A_i^T                    [M, h], a partial of dX.
    Returns (dX_i, dA_i, dB_i, da_i); da_i is None without a bias."""
    X, A_i, B_i, dZ = f64(X), f64(A_i), f64(B_i), f64(dZ)
    Y = matmul(X, A_i, a_i)
    Yp = gelu(Y)
    dB = matmul(Yp.T.copy(), dZ)
    dY = matmul(dZ, B_i.T.copy()) * gelu_grad(Y)
    dA = matmul(X.T.copy(), dY)
    da = dY.sum(axis=0) if a_i is not None else None
    dX = matmul(dY, A_i.T.copy())
    return dX, dA, dB, da


def attention_rows(Q, K, V, tpos, Hl: int, d: int, causal: bool) -> np.ndarray:
    """softmax(q·K^T/sqrt d)·V per local head for query rows of one sequence
    (the C loop); Q [nq, Hl·d], K/V [L, Hl·d], tpos [nq] positions."""
    Q, K, V = f64(Q), f64(K), f64(V)
    tpos = np.ascontiguousarray(np.asarray(tpos, dtype=np.int64))
    nq, L = Q.shape[0], K.shape[0]
    assert Q.shape[1] == K.shape[1] == V.shape[1] == Hl * d and V.shape[0] == L
    assert nq == 0 or (tpos.min() >= 0 and tpos.max() < L)
    O = np.empty((nq, Hl * d), dtype=np.float64)
    _load().orc_attention_rows(_p(Q), _p(K), _p(V), tpos.ctypes.data_as(ctypes.POINTER(_i64)),
                               nq, L, Hl, d, int(bool(causal)), _p(O))
    return O


def attn_shard_rows(X, b: int, s: int, Wqkv, Wo, Hl: int, d: int, causal: bool,
                    rows=None) -> np.ndarray:
    """One rank's attention partial Z_i = O_i·W_o,i for the token rows ``rows``
    ("图解Transformer并行计算" §3.1 / §3.2).

    X [b·s, h] (token m = sequence m // s, position m % s); Wqkv [h, 3·Hl·d]
    laid out [W_q | W_k | W_v] for the local heads, head-major within each
    block; Wo [Hl·d, h].  The keys and values of each sequence are projected
    over exactly the prefix the requested rows attend to (all s tokens when
    not causal).  Returns [len(rows), h].
    """
    X, Wqkv, Wo = f64(X), f64(Wqkv), f64(Wo)
    h = X.shape[1]
    HD = Hl * d
    assert X.shape[0] == b * s and Wqkv.shape == (h, 3 * HD) and Wo.shape == (HD, h)
    if rows is None:
        rows = np.arange(b * s, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((rows.size, HD), dtype=np.float64)
    for beta in np.unique(rows // s):
        sel = np.nonzero(rows // s == beta)[0]
        t = rows[sel] % s
        L = int(t.max()) + 1 if causal else s
        xs = X[beta * s: beta * s + L]
        KV = matmul(xs, np.ascontiguousarray(Wqkv[:, HD:]))
        Q = matmul(np.ascontiguousarray(X[rows[sel]]), np.ascontiguousarray(Wqkv[:, :HD]))
        O[sel] = attention_rows(Q, np.ascontiguousarray(KV[:, :HD]),
                                np.ascontiguousarray(KV[:, HD:]), t, Hl, d, causal)
    return matmul(O, Wo)


def attention_kv_split(Q, K, V, P: int, causal: bool):
    """One head's attention with Q, K and V split along the feature dimension
    over P ranks (strategy B, "K/V splitting", of the ops-transformer article
    (intelliparadigm.com/article/weixin_42537919/2252113) §3.1).

    Rank r holds the features F_r = [r·d/P, (r+1)·d/P) of Q, K, V [s, d] and
    computes the partial scores S_r = Q[:, F_r]·K[:, F_r]^T.  The softmax is
    not linear, so the partial scores are summed over the ranks first (in
    rank order); then P = softmax(S/sqrt(d) + causal mask) row by row (the
    maximum subtracted, two passes), and rank r forms its feature slice of
    the output, O[:, F_r] = P·V[:, F_r].  Returns (S_parts [P, s, s],
    O [s, d]) in float64.
    """
    Q, K, V = f64(Q), f64(K), f64(V)
    s, d = Q.shape
    assert K.shape == (s, d) and V.shape == (s, d) and d % P == 0
    w = d // P
    parts = np.stack([Q[:, r * w:(r + 1) * w] @ K[:, r * w:(r + 1) * w].T for r in range(P)])
    S = parts[0].copy()
    for r in range(1, P):
        S += parts[r]
    S /= math.sqrt(d)
    if causal:
        S[np.triu_indices(s, 1)] = -np.inf
    S -= S.max(axis=1, keepdims=True)
    E = np.exp(S)
    Pm = E / E.sum(axis=1, keepdims=True)
    O = np.concatenate([Pm @ V[:, r * w:(r + 1) * w] for r in range(P)], axis=1)
    return parts, O


def attention_kv_split_rows(qkv, b: int, s: int, H: int, d: int, P: int, causal: bool):
    """attention_kv_split for every (sequence, head) of a fused projection
    qkv [b·s, 3·H·d] laid out [Q | K | V], head-major within each block;
    returns O [b·s, H·d] (head-major columns, each head's features in rank
    order)."""
    qkv = f64(qkv)
    HD = H * d
    assert qkv.shape == (b * s, 3 * HD)
    O = np.empty((b * s, HD), dtype=np.float64)
    for beta in range(b):
        rows = slice(beta * s, (beta + 1) * s)
        for hd in range(H):
            c = slice(hd * d, (hd + 1) * d)
            O[rows, c] = attention_kv_split(qkv[rows, c], qkv[rows, HD + hd * d:HD + (hd + 1) * d],
                                            qkv[rows, 2 * HD + hd * d:2 * HD + (hd + 1) * d],
                                            P, causal)[1]
    return O


def attention_backward(Q, K, V, dO, Hl: int, d: int, causal: bool):
    """Gradients of O = softmax(Q·K^T/sqrt d + mask)·V for one sequence and
    every local head, given the upstream gradient dO.

    "图解Transformer并行计算" §3.2 (backward): each rank computes the
    gradients of its own heads' parameters from the same upstream gradient.
    Per head, with S = Q K^T / sqrt(d) (keys after the query masked out when
    causal) and P the row-wise softmax of S, the chain rule gives
        dV = P^T·dO,   dP = dO·V^T,
        dS_ij = P_ij·(dP_ij - sum_k P_ik·dP_ik)   (the softmax Jacobian, row i)
        dQ = dS·K / sqrt(d),   dK = dS^T·Q / sqrt(d).
    The products are float64 library matmuls; softmax subtracts the row max.
    Q, K, V, dO [s, Hl·d] (head j in columns j·d..j·d+d-1).  Returns
    (dQ, dK, dV), each [s, Hl·d].
    """
    Q, K, V, dO = f64(Q), f64(K), f64(V), f64(dO)
    s = Q.shape[0]
    assert K.shape == V.shape == dO.shape == Q.shape == (s, Hl * d)
    dQ, dK, dV = (np.zeros_like(Q) for _ in range(3))
    visible = np.tril(np.ones((s, s), dtype=bool)) if causal else np.ones((s, s), dtype=bool)
    for j in range(Hl):
        c = slice(j * d, (j + 1) * d)
        S = np.matmul(Q[:, c], K[:, c].T) / math.sqrt(d)
        S = np.where(visible, S, -np.inf)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)
        dV[:, c] = np.matmul(P.T, dO[:, c])
        dP = np.matmul(dO[:, c], V[:, c].T)
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dQ[:, c] = np.matmul(dS, K[:, c]) / math.sqrt(d)
        dK[:, c] = np.matmul(dS.T, Q[:, c]) / math.sqrt(d)
    return dQ, dK, dV


def attn_shard_backward(X, b: int, s: int, Wqkv, Wo, dZ, Hl: int, d: int, causal: bool):
    """Gradients of one rank's attention share Z_i = O_i·W_o,i, where O_i is
    its local heads' attention over qkv = X·W_qkv,i ("图解Transformer并行计算"
    §3.2, backward: the same dZ reaches every rank; each computes the
    gradients of its own W_o,i and W_qkv,i and a local input gradient, which
    one all-reduce sums over ranks into dX).  By the chain rule:
        dW_o,i = O_i^T·dZ,        dO_i = dZ·W_o,i^T,
        (dQ, dK, dV) = attention_backward per sequence -> dqkv [b·s, 3·Hl·d],
        dW_qkv,i = X^T·dqkv,      dX_i = dqkv·W_qkv,i^T.
    X [b·s, h] (token m = sequence m // s, position m % s); Wqkv [h, 3·Hl·d]
    laid out [W_q | W_k | W_v]; Wo [Hl·d, h]; dZ [b·s, h].
    Returns (dX_i, dW_qkv,i, dW_o,i)."""
    X, Wqkv, Wo, dZ = f64(X), f64(Wqkv), f64(Wo), f64(dZ)
    HD = Hl * d
    M = b * s
    assert X.shape[0] == M and Wqkv.shape[1] == 3 * HD and Wo.shape == (HD, X.shape[1])
    qkv = matmul(X, Wqkv)
    O = np.empty((M, HD), dtype=np.float64)
    dqkv = np.empty((M, 3 * HD), dtype=np.float64)
    dO = matmul(dZ, Wo.T.copy())
    for beta in range(b):
        r = slice(beta * s, (beta + 1) * s)
        Qs, Ks, Vs = (np.ascontiguousarray(qkv[r, k * HD:(k + 1) * HD]) for k in range(3))
        O[r] = attention_rows(Qs, Ks, Vs, np.arange(s), Hl, d, causal)
        g = attention_backward(Qs, Ks, Vs, dO[r], Hl, d, causal)
        for k in range(3):
            dqkv[r, k * HD:(k + 1) * HD] = g[k]
    dWo = matmul(O.T.copy(), dZ)
    dWqkv = matmul(X.T.copy(), dqkv)
    dX = matmul(dqkv, Wqkv.T.copy())
    return dX, dWqkv, dWo


def partial_sum(parts, bias=None, residual=None) -> np.ndarray:
    """Z = sum_r parts[r] (+bias per column) (+residual); parts [P, M, h]."""
    parts = f64(parts)
    P = parts.shape[0]
    M, h = parts.shape[1], parts.shape[2]
    bias, residual = f64(bias), f64(residual)
    if residual is not None:
        residual = np.ascontiguousarray(residual.reshape(M, h))
    Z = np.empty((M, h), dtype=np.float64)
    _load().orc_partial_sum(_p(parts), P, M, h, _p(bias), _p(residual), _p(Z))
    return Z


# ---------------------------------------------------------------- vocabulary ends
def vocab_embedding_shard(tokens, E_r, vocab_start: int) -> np.ndarray:
    """One rank's share of the vocab-parallel input embedding
    ("图解Transformer并行计算" §4.1): the rank holds rows vocab_start ..
    vocab_start + V_r - 1 of the table E [V, h]; a token in that range gets its
    row, any other token a zero vector, so the sum over ranks (the all-reduce)
    is the full lookup.  tokens [M] integers, E_r [V_r, h].  Returns [M, h]."""
    E_r = f64(E_r)
    t = np.asarray(tokens, dtype=np.int64).reshape(-1)
    out = np.zeros((t.size, E_r.shape[1]), dtype=np.float64)
    local = t - int(vocab_start)
    mine = (local >= 0) & (local < E_r.shape[0])
    out[mine] = E_r[local[mine]]
    return out


def vocab_ce_shard_stats(H, E_r, targets, vocab_start: int):
    """One rank's local part of the vocab-parallel cross-entropy
    ("图解Transformer并行计算" §4.2): its logits are H·E_r^T over its vocab
    range (the output layer shares the input embedding's table).  In the stable
    form (reading: the page's exp-sum over raw logits overflows; the row maximum
    is reduced first), the rank reports per token row
        m_r = max_j logit_j,  s_r = sum_j exp(logit_j - m_r),
        t_r = the target's logit if the target is in the rank's range, else 0.
    H [M, h], E_r [V_r, h], targets [M].  Returns (m_r, s_r, t_r), each [M]."""
    H, E_r = f64(H), f64(E_r)
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    logits = np.matmul(H, E_r.T)
    m = logits.max(axis=1)
    s = np.exp(logits - m[:, None]).sum(axis=1)
    local = t - int(vocab_start)
    mine = (local >= 0) & (local < E_r.shape[0])
    tl = np.zeros(t.size, dtype=np.float64)
    tl[mine] = logits[np.nonzero(mine)[0], local[mine]]
    return m, s, tl


def vocab_ce_combine(stats):
    """The all-reduces of the vocab-parallel cross-entropy and the loss
    ("图解Transformer并行计算" §4.2): over the ranks' (m_r, s_r, t_r), the global
    maximum m = max_r m_r, the global exp-sum s = sum_r s_r·exp(m_r - m) and the
    target logit t = sum_r t_r (one rank holds it); the per-token loss is
    -log softmax(target) = log(s) + m - t.  Returns the loss [M]."""
    m = np.max(np.stack([np.asarray(st[0], dtype=np.float64) for st in stats]), axis=0)
    s = sum(np.asarray(st[1], dtype=np.float64) * np.exp(np.asarray(st[0]) - m) for st in stats)
    t = sum(np.asarray(st[2], dtype=np.float64) for st in stats)
    return np.log(s) + m - t


# ---------------------------------------------------------------- composites
def block_rows(x, b: int, s: int, Wqkv_list, Wo_list, A_list, B_list, H: int, d: int,
               rows=None, ln1=(None, None), ln2=(None, None), eps: float = 1e-5,
               causal: bool = True):
    """Pre-LN block with P ranks' shares summed, for the token rows ``rows``.

      x1  = x  + sum_r Attn_r(LN1(x))
      out = x1 + sum_r MLP_r(LN2(x1))

    Returns (x1_rows, out_rows), both [len(rows), h] float64.  LN1 is taken over
    exactly the prefix rows the sampled queries attend to; rows are independent
    everywhere else.  Weights are converted one rank at a time.
    """
    P = len(Wqkv_list)
    xf = f64(x)
    h = xf.shape[1]
    Hl = H // P
    if rows is None:
        rows = np.arange(b * s, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    # LN1 of the prefix rows each sampled query reads (all of its sequence
    # when not causal); other rows are never read.
    need = np.zeros(b * s, dtype=bool)
    for m in rows:
        beta, t = divmod(int(m), s)
        need[beta * s: beta * s + (t + 1 if causal else s)] = True
    idx = np.nonzero(need)[0]
    xn = np.zeros_like(xf)
    xn[idx] = layernorm(xf[idx], ln1[0], ln1[1], eps)
    attn_parts = np.empty((P, rows.size, h), dtype=np.float64)
    for r in range(P):
        attn_parts[r] = attn_shard_rows(xn, b, s, f64(Wqkv_list[r]), f64(Wo_list[r]),
                                        Hl, d, causal, rows)
    x1 = partial_sum(attn_parts, None, xf[rows])
    del attn_parts
    xn2 = layernorm(x1, ln2[0], ln2[1], eps)
    mlp_parts = np.empty((P, rows.size, h), dtype=np.float64)
    for r in range(P):
        mlp_parts[r] = mlp_shard(xn2, f64(A_list[r]), f64(B_list[r]))
    out = partial_sum(mlp_parts, None, x1)
    return x1, out
