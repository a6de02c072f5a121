"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Each test ties the oracle to something it does not compute the same way: the
invariants of the tensor-parallel method ("图解Transformer并行计算"
(un.csdn.net/7y5fj9k05scw) §1.1, §1.2, §2.1, §3.2), closed forms, textbook
values, library routines in float64 and brute-force pure-Python loops over
tiny inputs.  Every shape is non-square so a transposed operand cannot pass.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(12345)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------- input conversion
def _bf16_from_definition(bits: int) -> float:
    """Value of a bfloat16 bit pattern from the format's definition: 1 sign
    bit, 8 exponent bits (bias 127), 7 fraction bits; exponent 0 encodes
    zero and subnormals (fraction * 2^-133), exponent 255 infinities (zero
    fraction) and NaNs."""
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(frac, -133)
    return sign * math.ldexp(128 + frac, e - 134)


def test_f64_widens_every_bf16_pattern_exactly():
    """Every GPU comparison feeds the oracle the shared bf16 inputs through
    oracle.f64; all 65536 bit patterns (both zeros, subnormals, the largest
    finite values, both infinities, NaNs) must widen to exactly the value the
    format defines, and agree bit for bit with torch's own widening."""
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    t = bits.view(torch.bfloat16)
    got = oracle.f64(t)
    assert got.dtype == np.float64 and got.shape == (65536,)
    lib = t.double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), lib[~nan].view(np.uint64))
    for i, b in enumerate(bits.numpy().astype(np.uint16).tolist()):
        want = _bf16_from_definition(b)
        if math.isnan(want):
            assert math.isnan(got[i]), hex(b)
        else:
            assert got[i] == want and math.copysign(1.0, got[i]) == math.copysign(1.0, want), hex(b)
    # landmarks, spelled out
    by_bits = {int(b): float(v) for b, v in zip(bits.numpy().astype(np.uint16), got)}
    assert by_bits[0x3F80] == 1.0 and by_bits[0xC000] == -2.0
    assert by_bits[0x0001] == 2.0 ** -133 and by_bits[0x8001] == -(2.0 ** -133)
    assert by_bits[0x7F7F] == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert by_bits[0x7F80] == math.inf and by_bits[0xFF80] == -math.inf
    assert by_bits[0x0000] == 0.0 and math.copysign(1.0, by_bits[0x8000]) == -1.0


def test_f64_widens_f32_exactly():
    g = torch.Generator().manual_seed(77)
    t = torch.randn(100000, generator=g) * torch.exp2(torch.randint(-140, 120, (100000,),
                                                                    generator=g).float())
    special = torch.tensor([0.0, -0.0, float("inf"), float("-inf"), float("nan"),
                            3.4028234663852886e38, -3.4028234663852886e38, 1.401298464324817e-45,
                            -1.401298464324817e-45, 1.1754943508222875e-38])
    t = torch.cat([t, special])
    got = oracle.f64(t)
    lib = t.double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), lib[~nan].view(np.uint64))
    # a binary32 value is the rational its bits define: compare with the
    # struct module's own decoding of the same bytes
    import struct
    raw = t.numpy().tobytes()
    for i in range(0, 100010, 997):
        (v,) = struct.unpack_from("<f", raw, 4 * i)
        assert (math.isnan(v) and math.isnan(got[i])) or got[i] == v


def test_f64_random_bf16_round_trip():
    """1e5 random bf16 values of every magnitude: widening is exact, so
    rounding back to bf16 returns the same bits."""
    g = torch.Generator().manual_seed(78)
    t = (torch.randn(100000, generator=g) *
         torch.exp2(torch.randint(-130, 127, (100000,), generator=g).float())).to(torch.bfloat16)
    got = oracle.f64(t)
    back = torch.from_numpy(got).to(torch.bfloat16)
    assert torch.equal(back.view(torch.int16), t.view(torch.int16))
    assert np.array_equal(got, t.double().numpy())


# --------------------------------------------------------------- matmul
def test_matmul_matches_library():
    X = RNG.standard_normal((13, 29))
    W = RNG.standard_normal((29, 11))
    bias = RNG.standard_normal(11)
    assert rel(oracle.matmul(X, W), X @ W) < 1e-14
    assert rel(oracle.matmul(X, W, bias), X @ W + bias) < 1e-14


def test_matmul_brute_force_exact_sums():
    X = RNG.standard_normal((3, 5))
    W = RNG.standard_normal((5, 4))
    Y = oracle.matmul(X, W)
    for m in range(3):
        for n in range(4):
            ref = math.fsum(X[m, k] * W[k, n] for k in range(5))
            assert abs(Y[m, n] - ref) <= 1e-14 * (1 + abs(ref))


def test_matmul_identity_gives_input():
    X = RNG.standard_normal((6, 8))
    assert np.array_equal(oracle.matmul(X, np.eye(8)), X)


def test_column_split_concat_is_full_product():
    """§1.2: Y_r = X·W_r on column blocks; concatenation equals X·W (up to the
    library's summation order)."""
    X = RNG.standard_normal((10, 24))
    W = RNG.standard_normal((24, 36))
    full = oracle.matmul(X, W)
    for P in (2, 3, 4):
        c = 36 // P
        parts = [oracle.matmul(X, np.ascontiguousarray(W[:, r * c:(r + 1) * c])) for r in range(P)]
        assert rel(np.concatenate(parts, axis=1), full) < 1e-15


def test_row_split_sum_is_full_product():
    """§1.1: W split on rows, X split on columns; summing the partials gives X·W."""
    X = RNG.standard_normal((9, 32))
    W = RNG.standard_normal((32, 20))
    full = oracle.matmul(X, W)
    for P in (2, 4, 8):
        c = 32 // P
        parts = np.stack([oracle.matmul(np.ascontiguousarray(X[:, r * c:(r + 1) * c]),
                                        np.ascontiguousarray(W[r * c:(r + 1) * c]))
                          for r in range(P)])
        assert rel(oracle.partial_sum(parts), full) < 1e-14


def test_split_gather_reconstruction_is_exact():
    """Splitting a weight into P blocks and concatenating them back is the identity."""
    W = torch.randn(128, 256, dtype=torch.float64)
    for dim in (0, 1):
        parts = torch.split(W, W.shape[dim] // 4, dim=dim)
        assert torch.equal(torch.cat(parts, dim=dim), W)


# --------------------------------------------------------------- GeLU
def _golden_phi():
    rows = []
    with open(os.path.join(HERE, "golden", "normal_cdf.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                x, p = line.split()
                rows.append((float(x), float(p)))
    return rows


def test_gelu_textbook_values():
    for x, phi in _golden_phi():
        assert abs(oracle.gelu_scalar(x) - x * phi) <= 1e-15 * max(1.0, abs(x))


def test_gelu_closed_forms():
    assert oracle.gelu_scalar(0.0) == 0.0
    for x in np.linspace(-6, 6, 97):
        # GeLU(x) - GeLU(-x) = x because erf is odd
        assert abs(oracle.gelu_scalar(x) - oracle.gelu_scalar(-x) - x) <= 4e-16 * max(1, abs(x))
    assert abs(oracle.gelu_scalar(12.0) - 12.0) < 1e-15
    assert abs(oracle.gelu_scalar(-12.0)) < 1e-30


def _erf_series(x):
    # Maclaurin series erf(x) = 2/sqrt(pi) * sum_n (-1)^n x^(2n+1) / (n! (2n+1))
    term, n = x, 0
    terms = []
    while True:
        t = term / (2 * n + 1)
        terms.append(t)
        if abs(t) < 1e-30:
            break
        n += 1
        term *= -x * x / n
    return 2.0 / math.sqrt(math.pi) * math.fsum(terms)


def test_gelu_matches_independent_erf_series():
    for x in np.linspace(-3, 3, 61):
        ref = 0.5 * x * (1.0 + _erf_series(x / math.sqrt(2.0)))
        assert abs(oracle.gelu_scalar(x) - ref) <= 1e-13


def test_gelu_vector_matches_torch_exact_gelu():
    x = RNG.standard_normal(1000) * 3
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.max(np.abs(oracle.gelu(x) - ref)) < 1e-14
    tanh = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu(x) - tanh)) > 1e-5  # not the tanh form


# --------------------------------------------------------------- MLP
def _mlp_weights(M=12, h=16, F=48):
    X = RNG.standard_normal((M, h))
    A = RNG.standard_normal((h, F)) / math.sqrt(h)
    B = RNG.standard_normal((F, h)) / math.sqrt(F)
    a = RNG.standard_normal(F) * 0.1
    return X, A, B, a


def test_mlp_unsharded_matches_library():
    X, A, B, a = _mlp_weights()
    t = lambda v: torch.from_numpy(v)
    ref = (torch.nn.functional.gelu(t(X) @ t(A) + t(a)) @ t(B)).numpy()
    assert rel(oracle.mlp_shard(X, A, B, a), ref) < 1e-13


@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_mlp_shards_sum_to_unsharded(P):
    """§2.1: column-split A, local GeLU, row-split B; Z = sum_i Z_i."""
    X, A, B, a = _mlp_weights(F=48)
    f = 48 // P
    parts = np.stack([oracle.mlp_shard(X, np.ascontiguousarray(A[:, r * f:(r + 1) * f]),
                                       np.ascontiguousarray(B[r * f:(r + 1) * f]),
                                       a[r * f:(r + 1) * f]) for r in range(P)])
    assert rel(oracle.partial_sum(parts), oracle.mlp_shard(X, A, B, a)) < 1e-13


def test_mlp_row_split_first_layer_is_wrong():
    """§2.1 negative control: splitting A by rows puts GeLU before the sum, which
    gives a different answer (GeLU(Y1+Y2) != GeLU(Y1)+GeLU(Y2))."""
    X, A, B, _ = _mlp_weights(F=48)
    h = 16
    wrong = sum(oracle.matmul(oracle.gelu(oracle.matmul(np.ascontiguousarray(X[:, r * 8:(r + 1) * 8]),
                                                        np.ascontiguousarray(A[r * 8:(r + 1) * 8]))), B)
                for r in range(h // 8))
    assert rel(wrong, oracle.mlp_shard(X, A, B)) > 1e-2


def test_mlp_brute_force():
    M, h, f = 3, 4, 6
    X = RNG.standard_normal((M, h))
    A = RNG.standard_normal((h, f))
    B = RNG.standard_normal((f, h))
    a = RNG.standard_normal(f)
    Z = oracle.mlp_shard(X, A, B, a)
    for m in range(M):
        g = []
        for n in range(f):
            y = math.fsum(X[m, k] * A[k, n] for k in range(h)) + a[n]
            g.append(0.5 * y * (1 + math.erf(y / math.sqrt(2))))
        for j in range(h):
            ref = math.fsum(g[n] * B[n, j] for n in range(f))
            assert abs(Z[m, j] - ref) <= 1e-13 * (1 + abs(ref))


# --------------------------------------------------------------- attention
def _attn_setup(b=2, s=7, H=4, d=3):
    h = H * d
    X = RNG.standard_normal((b * s, h))
    Wq = RNG.standard_normal((h, H * d)) / math.sqrt(h)
    Wk = RNG.standard_normal((h, H * d)) / math.sqrt(h)
    Wv = RNG.standard_normal((h, H * d)) / math.sqrt(h)
    Wo = RNG.standard_normal((H * d, h)) / math.sqrt(h)
    return X, Wq, Wk, Wv, Wo


def _rank_qkv(Wq, Wk, Wv, r, Hl, d):
    sl = slice(r * Hl * d, (r + 1) * Hl * d)
    return np.ascontiguousarray(np.concatenate([Wq[:, sl], Wk[:, sl], Wv[:, sl]], axis=1))


def _torch_mha(X, Wq, Wk, Wv, Wo, b, s, H, d, causal):
    t = lambda v: torch.from_numpy(v)
    q = (t(X) @ t(Wq)).view(b, s, H, d).transpose(1, 2)
    k = (t(X) @ t(Wk)).view(b, s, H, d).transpose(1, 2)
    v = (t(X) @ t(Wv)).view(b, s, H, d).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    return (o.transpose(1, 2).reshape(b * s, H * d) @ t(Wo)).numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_attention_full_matches_library(causal):
    b, s, H, d = 2, 7, 4, 3
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    ours = oracle.attn_shard_rows(X, b, s, _rank_qkv(Wq, Wk, Wv, 0, H, d), Wo, H, d, causal)
    assert rel(ours, _torch_mha(X, Wq, Wk, Wv, Wo, b, s, H, d, causal)) < 1e-13


@pytest.mark.parametrize("P", [2, 4])
def test_head_sharded_attention_sums_to_full_mha(P):
    """§3.2: each rank runs its H/P heads and multiplies by its row block of
    W_o; the sum over ranks equals full multi-head attention."""
    b, s, H, d = 2, 6, 4, 5
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    Hl = H // P
    parts = np.stack([oracle.attn_shard_rows(X, b, s, _rank_qkv(Wq, Wk, Wv, r, Hl, d),
                                             np.ascontiguousarray(Wo[r * Hl * d:(r + 1) * Hl * d]),
                                             Hl, d, True) for r in range(P)])
    full = oracle.attn_shard_rows(X, b, s, _rank_qkv(Wq, Wk, Wv, 0, H, d), Wo, H, d, True)
    assert rel(oracle.partial_sum(parts), full) < 1e-13


def test_attention_sampled_rows_equal_full_rows():
    b, s, H, d = 3, 9, 2, 4
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    Wqkv = _rank_qkv(Wq, Wk, Wv, 0, H, d)
    full = oracle.attn_shard_rows(X, b, s, Wqkv, Wo, H, d, True)
    rows = np.array([26, 0, 9, 13, 17, 4])
    assert rel(oracle.attn_shard_rows(X, b, s, Wqkv, Wo, H, d, True, rows), full[rows]) < 1e-14


def test_attention_single_token_returns_value_projection():
    """s = 1: softmax over one key is 1, so O = V and Z = V·W_o."""
    b, s, H, d = 4, 1, 2, 3
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    ours = oracle.attn_shard_rows(X, b, s, _rank_qkv(Wq, Wk, Wv, 0, H, d), Wo, H, d, True)
    assert rel(ours, (X @ Wv) @ Wo) < 1e-14


def test_attention_equal_scores_give_causal_running_mean():
    """W_k = 0 makes every score 0: causal softmax weights are 1/(t+1) over
    u <= t, so O_t is the running mean of v_0..v_t (pins the mask direction)."""
    b, s, H, d = 2, 8, 2, 3
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    Wk = np.zeros_like(Wk)
    O_ref = np.zeros((b * s, H * d))
    V = X @ Wv
    for beta in range(b):
        for t in range(s):
            O_ref[beta * s + t] = V[beta * s: beta * s + t + 1].mean(axis=0)
    ours = oracle.attn_shard_rows(X, b, s, _rank_qkv(Wq, Wk, Wv, 0, H, d), np.eye(H * d), H, d, True)
    assert rel(ours, O_ref) < 1e-14


def test_attention_brute_force():
    b, s, H, d = 1, 3, 2, 2
    h = 4
    X = RNG.standard_normal((s, h))
    Wqkv = RNG.standard_normal((h, 3 * H * d))
    Wo = RNG.standard_normal((H * d, h))
    Z = oracle.attn_shard_rows(X, b, s, Wqkv, Wo, H, d, True)
    proj = [[math.fsum(X[t, k] * Wqkv[k, n] for k in range(h)) for n in range(3 * H * d)] for t in range(s)]
    for t in range(s):
        o = []
        for j in range(H):
            q = proj[t][j * d:(j + 1) * d]
            sc = []
            for u in range(t + 1):
                kv = proj[u][H * d + j * d: H * d + (j + 1) * d]
                sc.append(math.fsum(q[c] * kv[c] for c in range(d)) / math.sqrt(d))
            mx = max(sc)
            w = [math.exp(v - mx) for v in sc]
            den = math.fsum(w)
            for c in range(d):
                o.append(math.fsum(w[u] * proj[u][2 * H * d + j * d + c] for u in range(t + 1)) / den)
        for n in range(h):
            ref = math.fsum(o[k] * Wo[k, n] for k in range(H * d))
            assert abs(Z[t, n] - ref) <= 1e-13 * (1 + abs(ref))


# --------------------------------------------------------------- LayerNorm
def test_layernorm_moments():
    x = RNG.standard_normal((17, 40)) * 3 + 1.5
    eps = 1e-5
    y = oracle.layernorm(x, eps=eps)
    var = x.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-14
    assert np.max(np.abs(y.var(axis=1) - var / (var + eps))) < 1e-13


def test_layernorm_matches_library():
    x = RNG.standard_normal((9, 24))
    g = RNG.standard_normal(24)
    bta = RNG.standard_normal(24)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(g),
                                         torch.from_numpy(bta), eps=1e-5).numpy()
    assert rel(oracle.layernorm(x, g, bta, 1e-5), ref) < 1e-14


# --------------------------------------------------------------- partial sum
def test_partial_sum_exact_against_fsum():
    P, M, h = 8, 5, 7
    parts = RNG.standard_normal((P, M, h)) * 10.0 ** RNG.integers(-3, 4, size=(P, M, h))
    bias = RNG.standard_normal(h)
    res = RNG.standard_normal((M, h))
    Z = oracle.partial_sum(parts, bias, res)
    for m in range(M):
        for c in range(h):
            terms = [*parts[:, m, c], bias[c], res[m, c]]
            ref = math.fsum(terms)
            assert abs(Z[m, c] - ref) <= 1e-15 * 16 * math.fsum(abs(v) for v in terms)
    # the bias is added once per element, not once per rank
    Z0 = oracle.partial_sum(parts)
    assert rel(Z - Z0, np.broadcast_to(bias, (M, h)) + res) < 1e-12


# --------------------------------------------------------------- block
def _block_weights(P, h, H, d, F, seed=7):
    rng = np.random.default_rng(seed)
    Wq = rng.standard_normal((h, H * d)) / math.sqrt(h)
    Wk = rng.standard_normal((h, H * d)) / math.sqrt(h)
    Wv = rng.standard_normal((h, H * d)) / math.sqrt(h)
    Wo = rng.standard_normal((H * d, h)) / math.sqrt(H * d)
    A = rng.standard_normal((h, F)) / math.sqrt(h)
    B = rng.standard_normal((F, h)) / math.sqrt(F)
    Hl, f = H // P, F // P
    qkv = [_rank_qkv(Wq, Wk, Wv, r, Hl, d) for r in range(P)]
    wo = [np.ascontiguousarray(Wo[r * Hl * d:(r + 1) * Hl * d]) for r in range(P)]
    a = [np.ascontiguousarray(A[:, r * f:(r + 1) * f]) for r in range(P)]
    bb = [np.ascontiguousarray(B[r * f:(r + 1) * f]) for r in range(P)]
    return qkv, wo, a, bb


def test_block_brute_force():
    """A pure-Python pre-LN block on a tiny input (P=2, h=8, H=2, d=4, s=3, F=16)."""
    P, b, s, H, d, F = 2, 2, 3, 2, 4, 16
    h = H * d
    x = RNG.standard_normal((b * s, h))
    qkv, wo, A, B = _block_weights(P, h, H, d, F)
    g1, b1 = RNG.standard_normal(h), RNG.standard_normal(h)
    g2, b2 = RNG.standard_normal(h), RNG.standard_normal(h)
    eps = 1e-5
    x1_o, out_o = oracle.block_rows(x, b, s, qkv, wo, A, B, H, d, ln1=(g1, b1), ln2=(g2, b2), eps=eps)

    def ln(row, g, bt):
        mu = math.fsum(row) / len(row)
        var = math.fsum((v - mu) ** 2 for v in row) / len(row)
        return [(v - mu) / math.sqrt(var + eps) * g[i] + bt[i] for i, v in enumerate(row)]

    def mm(vec, W):
        return [math.fsum(vec[k] * W[k][n] for k in range(len(vec))) for n in range(len(W[0]))]

    Hl, f = H // P, F // P
    xn = [ln(list(x[m]), g1, b1) for m in range(b * s)]
    x1 = [list(x[m]) for m in range(b * s)]
    for r in range(P):
        proj = [mm(xn[m], qkv[r].tolist()) for m in range(b * s)]
        for m in range(b * s):
            beta, t = divmod(m, s)
            o = []
            for j in range(Hl):
                q = proj[m][j * d:(j + 1) * d]
                sc = [math.fsum(q[c] * proj[beta * s + u][Hl * d + j * d + c] for c in range(d)) / math.sqrt(d)
                      for u in range(t + 1)]
                mx = max(sc)
                w = [math.exp(v - mx) for v in sc]
                den = math.fsum(w)
                o += [math.fsum(w[u] * proj[beta * s + u][2 * Hl * d + j * d + c] for u in range(t + 1)) / den
                      for c in range(d)]
            z = mm(o, wo[r].tolist())
            x1[m] = [x1[m][c] + z[c] for c in range(h)]
    out = [row[:] for row in x1]
    for m in range(b * s):
        xn2 = ln(x1[m], g2, b2)
        for r in range(P):
            y = mm(xn2, A[r].tolist())
            g = [0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in y]
            z = mm(g, B[r].tolist())
            out[m] = [out[m][c] + z[c] for c in range(h)]
    assert rel(x1_o, np.array(x1)) < 1e-12
    assert rel(out_o, np.array(out)) < 1e-12


def test_block_ranks_sum_to_unsharded_block():
    b, s, H, d, F = 2, 5, 4, 4, 64
    h = H * d
    x = RNG.standard_normal((b * s, h))
    full = _block_weights(1, h, H, d, F, seed=3)
    shard = _block_weights(4, h, H, d, F, seed=3)
    x1a, outa = oracle.block_rows(x, b, s, *full, H, d)
    x1b, outb = oracle.block_rows(x, b, s, *shard, H, d)
    assert rel(x1a, x1b) < 1e-13 and rel(outa, outb) < 1e-13
    rows = [9, 0, 6]
    x1c, outc = oracle.block_rows(x, b, s, *shard, H, d, rows=rows)
    assert rel(outc, outb[rows]) < 1e-14 and rel(x1c, x1b[rows]) < 1e-14


# ------------------------------------------------------------------ backward of the MLP share
def test_gelu_grad_closed_forms():
    """GeLU'(x) = Phi(x) + x·phi(x): GeLU'(0) = 1/2; GeLU(x) - GeLU(-x) = x
    gives GeLU'(x) + GeLU'(-x) = 1; the slope tends to 1 and 0 at the ends;
    and it is the central difference of the oracle's own GeLU."""
    x = np.linspace(-6, 6, 241)
    g = oracle.gelu_grad(x)
    assert abs(oracle.gelu_grad(np.array([0.0]))[0] - 0.5) < 1e-15
    assert np.abs(g + oracle.gelu_grad(-x) - 1.0).max() < 1e-14
    assert abs(oracle.gelu_grad(np.array([12.0]))[0] - 1.0) < 1e-12
    assert abs(oracle.gelu_grad(np.array([-12.0]))[0]) < 1e-12
    eps = 1e-6
    fd = (oracle.gelu(x + eps) - oracle.gelu(x - eps)) / (2 * eps)
    assert np.abs(fd - g).max() < 1e-8


def test_mlp_backward_matches_autograd():
    """Library check: torch autograd in float64 on the unsharded formula."""
    rng = np.random.default_rng(5)
    X, A, B = rng.normal(size=(7, 10)), rng.normal(size=(10, 6)) / 3, rng.normal(size=(6, 10)) / 3
    a, dZ = rng.normal(size=6), rng.normal(size=(7, 10))
    dX, dA, dB, da = oracle.mlp_shard_backward(X, A, B, dZ, a)
    t = [torch.tensor(v, requires_grad=True) for v in (X, A, B, a)]
    Z = torch.nn.functional.gelu(t[0] @ t[1] + t[3]) @ t[2]
    Z.backward(torch.tensor(dZ))
    for mine, ref in zip((dX, dA, dB, da), t):
        assert np.abs(mine - ref.grad.numpy()).max() < 1e-12


def test_mlp_backward_finite_differences():
    """Brute force: <grad, V> equals the central difference of <dZ, Z> along
    V for each input (X, A, B), on a tiny shard."""
    rng = np.random.default_rng(6)
    X, A, B = rng.normal(size=(3, 5)), rng.normal(size=(5, 4)) / 2, rng.normal(size=(4, 5)) / 2
    dZ = rng.normal(size=(3, 5))
    grads = oracle.mlp_shard_backward(X, A, B, dZ)
    loss = lambda X, A, B: float((dZ * oracle.mlp_shard(X, A, B)).sum())
    eps = 1e-6
    for k, g in enumerate(grads[:3]):
        V = rng.normal(size=g.shape)
        args = [X, A, B]
        plus = [v + eps * V if i == k else v for i, v in enumerate(args)]
        minus = [v - eps * V if i == k else v for i, v in enumerate(args)]
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert abs(fd - float((g * V).sum())) < 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("P", [2, 4])
def test_mlp_backward_ranks_sum_to_unsharded(P):
    """§2.2's backward: each rank gets the same dZ; the rank partials dX_r sum
    to the unsharded dX (the backward all-reduce), the dA_r are the column
    blocks of the unsharded dA and the dB_r its row blocks."""
    rng = np.random.default_rng(7 + P)
    M, h, F = 9, 12, 8 * P
    X, A, B = rng.normal(size=(M, h)), rng.normal(size=(h, F)) / 4, rng.normal(size=(F, h)) / 4
    dZ = rng.normal(size=(M, h))
    dX, dA, dB, _ = oracle.mlp_shard_backward(X, A, B, dZ)
    f = F // P
    parts = [oracle.mlp_shard_backward(X, A[:, r * f:(r + 1) * f], B[r * f:(r + 1) * f], dZ)
             for r in range(P)]
    assert np.abs(sum(p[0] for p in parts) - dX).max() < 1e-12
    assert np.abs(np.concatenate([p[1] for p in parts], axis=1) - dA).max() < 1e-12
    assert np.abs(np.concatenate([p[2] for p in parts], axis=0) - dB).max() < 1e-12


def test_mlp_backward_needs_the_gelu_derivative():
    """Negative control: skipping the GeLU derivative (or using GeLU itself)
    in place of GeLU' changes dA, so the chain-rule factor is pinned."""
    rng = np.random.default_rng(9)
    X, A, B, dZ = rng.normal(size=(6, 8)), rng.normal(size=(8, 5)), rng.normal(size=(5, 8)), \
        rng.normal(size=(6, 8))
    _, dA, _, _ = oracle.mlp_shard_backward(X, A, B, dZ)
    dYp = oracle.matmul(dZ, B.T.copy())
    wrong = oracle.matmul(X.T.copy(), dYp)                           # no GeLU' factor
    assert np.abs(wrong - dA).max() > 1e-3


# --------------------------------------------------------------- attention backward
def _sdpa_grads(Q, K, V, dO, Hl, d, causal):
    """float64 autograd through torch's scaled_dot_product_attention, heads
    split out of the [s, Hl·d] layout."""
    s = Q.shape[0]
    t = [torch.tensor(v, requires_grad=True) for v in (Q, K, V)]
    heads = lambda x: x.view(s, Hl, d).transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(heads(t[0]), heads(t[1]), heads(t[2]),
                                                         is_causal=causal)
    o.transpose(0, 1).reshape(s, Hl * d).backward(torch.tensor(dO))
    return [v.grad.numpy() for v in t]


@pytest.mark.parametrize("causal", [True, False])
def test_attention_backward_matches_autograd(causal):
    rng = np.random.default_rng(21)
    s, Hl, d = 11, 3, 5
    Q, K, V, dO = (rng.normal(size=(s, Hl * d)) for _ in range(4))
    ours = oracle.attention_backward(Q, K, V, dO, Hl, d, causal)
    for mine, ref in zip(ours, _sdpa_grads(Q, K, V, dO, Hl, d, causal)):
        assert np.abs(mine - ref).max() < 1e-12


def test_attention_backward_finite_differences():
    """Brute force: <grad, W> is the central difference of <dO, O> along W,
    with O from the oracle's own forward loop (a different code path)."""
    rng = np.random.default_rng(22)
    s, Hl, d = 6, 2, 3
    Q, K, V, dO = (rng.normal(size=(s, Hl * d)) for _ in range(4))
    grads = oracle.attention_backward(Q, K, V, dO, Hl, d, True)
    loss = lambda Q, K, V: float((dO * oracle.attention_rows(Q, K, V, np.arange(s), Hl, d,
                                                              True)).sum())
    eps = 1e-6
    for k, g in enumerate(grads):
        W = rng.normal(size=g.shape)
        args = [Q, K, V]
        plus = [v + eps * W if i == k else v for i, v in enumerate(args)]
        minus = [v - eps * W if i == k else v for i, v in enumerate(args)]
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert abs(fd - float((g * W).sum())) < 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("causal", [True, False])
def test_attention_backward_key_shift_invariance(causal):
    """Adding one vector c to every key adds q·c/sqrt d to a whole score row,
    which softmax ignores: the loss does not depend on c, so the key
    gradients of each head sum to zero (each dS row sums to zero)."""
    rng = np.random.default_rng(23)
    s, Hl, d = 9, 2, 4
    Q, K, V, dO = (rng.normal(size=(s, Hl * d)) for _ in range(4))
    _, dK, _ = oracle.attention_backward(Q, K, V, dO, Hl, d, causal)
    assert np.abs(dK.sum(axis=0)).max() < 1e-12 * np.abs(dK).max() * s


def test_attention_backward_single_key():
    """s = 1: the softmax over one key is the constant 1, so O = V: dV = dO
    and Q, K get no gradient."""
    rng = np.random.default_rng(24)
    Q, K, V, dO = (rng.normal(size=(1, 6)) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(Q, K, V, dO, 2, 3, True)
    assert np.abs(dQ).max() == 0 and np.abs(dK).max() == 0
    assert np.array_equal(dV, dO)


def test_attention_backward_needs_the_softmax_row_term():
    """Negative control: dropping the row term sum_k P_ik dP_ik from dS changes
    dQ, so the softmax Jacobian's second term is pinned."""
    rng = np.random.default_rng(25)
    s, Hl, d = 7, 1, 4
    Q, K, V, dO = (rng.normal(size=(s, Hl * d)) for _ in range(4))
    dQ, _, _ = oracle.attention_backward(Q, K, V, dO, Hl, d, True)
    S = np.where(np.tril(np.ones((s, s), bool)), Q @ K.T / math.sqrt(d), -np.inf)
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    wrong = (P * (dO @ V.T)) @ K / math.sqrt(d)
    assert np.abs(wrong - dQ).max() > 1e-3


@pytest.mark.parametrize("causal", [True, False])
def test_attn_shard_backward_matches_autograd(causal):
    """The whole attention share, X -> qkv -> attention -> W_o, through torch
    autograd in float64."""
    b, s, H, d = 2, 5, 2, 3
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    Wqkv = _rank_qkv(Wq, Wk, Wv, 0, H, d)
    dZ = np.random.default_rng(26).normal(size=(b * s, X.shape[1]))
    dX, dWqkv, dWo = oracle.attn_shard_backward(X, b, s, Wqkv, Wo, dZ, H, d, causal)
    t = [torch.tensor(v, requires_grad=True) for v in (X, Wqkv, Wo)]
    qkv = t[0] @ t[1]
    sp = lambda k: qkv[:, k * H * d:(k + 1) * H * d].reshape(b, s, H, d).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(sp(0), sp(1), sp(2), is_causal=causal)
    (o.transpose(1, 2).reshape(b * s, H * d) @ t[2]).backward(torch.tensor(dZ))
    for mine, ref in zip((dX, dWqkv, dWo), t):
        assert np.abs(mine - ref.grad.numpy()).max() < 1e-11


@pytest.mark.parametrize("P", [2, 4])
def test_attn_shard_backward_ranks_sum_to_unsharded(P):
    """§3.2's backward: the rank partials dX_r sum to the unsharded dX, each
    rank's dW_qkv,r holds its heads' columns of the unsharded [dW_q|dW_k|dW_v]
    and dW_o,r its row block of dW_o."""
    b, s, H, d = 2, 6, 4, 3
    X, Wq, Wk, Wv, Wo = _attn_setup(b, s, H, d)
    dZ = np.random.default_rng(27 + P).normal(size=(b * s, X.shape[1]))
    full = oracle.attn_shard_backward(X, b, s, _rank_qkv(Wq, Wk, Wv, 0, H, d), Wo, dZ, H, d, True)
    Hl, HD = H // P, H * d
    dX = 0
    for r in range(P):
        rows = slice(r * Hl * d, (r + 1) * Hl * d)
        g = oracle.attn_shard_backward(X, b, s, _rank_qkv(Wq, Wk, Wv, r, Hl, d),
                                       np.ascontiguousarray(Wo[rows]), dZ, Hl, d, True)
        dX = dX + g[0]
        want = np.concatenate([full[1][:, k * HD:(k + 1) * HD][:, rows] for k in range(3)], axis=1)
        assert np.abs(g[1] - want).max() < 1e-12
        assert np.abs(g[2] - full[2][rows]).max() < 1e-12
    assert np.abs(dX - full[0]).max() < 1e-12


# --------------------------------------------------------------- vocabulary ends
@pytest.mark.parametrize("P", [2, 4])
def test_vocab_embedding_ranks_sum_to_lookup(P):
    """§4.1: each rank looks up its vocab range and returns zeros elsewhere; the
    sum over ranks is the full table's row, exactly (one non-zero term)."""
    rng = np.random.default_rng(31 + P)
    V, h, M = 8 * P, 5, 23
    E = rng.normal(size=(V, h))
    tokens = np.concatenate([[0, V - 1, V // P - 1, V // P], rng.integers(0, V, M - 4)])
    Vr = V // P
    parts = [oracle.vocab_embedding_shard(tokens, E[r * Vr:(r + 1) * Vr], r * Vr) for r in range(P)]
    assert np.array_equal(sum(parts), E[tokens])
    for r, part in enumerate(parts):
        outside = (tokens < r * Vr) | (tokens >= (r + 1) * Vr)
        assert not part[outside].any()


@pytest.mark.parametrize("P", [1, 2, 4])
def test_vocab_ce_matches_library(P):
    """The sharded, stable cross-entropy equals torch's cross_entropy on the
    full logits H·E^T in float64."""
    rng = np.random.default_rng(41 + P)
    V, h, M = 12 * P, 7, 19
    H, E = rng.normal(size=(M, h)), rng.normal(size=(V, h))
    targets = rng.integers(0, V, M)
    Vr = V // P
    stats = [oracle.vocab_ce_shard_stats(H, E[r * Vr:(r + 1) * Vr], targets, r * Vr)
             for r in range(P)]
    loss = oracle.vocab_ce_combine(stats)
    ref = torch.nn.functional.cross_entropy(torch.tensor(H @ E.T), torch.tensor(targets),
                                            reduction="none").numpy()
    assert np.abs(loss - ref).max() < 1e-12


def test_vocab_ce_brute_force():
    """Pure-Python loops on a tiny case: -log(exp(l_t) / sum_j exp(l_j))."""
    rng = np.random.default_rng(43)
    V, h, M, P = 6, 3, 4, 3
    H, E = rng.normal(size=(M, h)), rng.normal(size=(V, h))
    targets = [0, 5, 2, 3]
    Vr = V // P
    loss = oracle.vocab_ce_combine([oracle.vocab_ce_shard_stats(H, E[r * Vr:(r + 1) * Vr],
                                                                targets, r * Vr) for r in range(P)])
    for i in range(M):
        logit = [math.fsum(H[i, k] * E[j, k] for k in range(h)) for j in range(V)]
        ref = math.log(math.fsum(math.exp(v) for v in logit)) - logit[targets[i]]
        assert abs(loss[i] - ref) < 1e-12


def test_vocab_ce_stable_for_large_logits():
    """Logits of order 1e3 overflow exp in float64; the max-first form stays
    finite and equals the shifted computation (negative control: the page's
    exp-sum over raw logits is inf)."""
    rng = np.random.default_rng(44)
    V, h, M, P = 8, 4, 5, 2
    H, E = 400 * rng.normal(size=(M, h)), rng.normal(size=(V, h))
    targets = rng.integers(0, V, M)
    Vr = V // P
    stats = [oracle.vocab_ce_shard_stats(H, E[r * Vr:(r + 1) * Vr], targets, r * Vr)
             for r in range(P)]
    loss = oracle.vocab_ce_combine(stats)
    assert np.isfinite(loss).all()
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.exp(H @ E.T).sum(axis=1)).all()
    L = H @ E.T
    ref = np.log(np.exp(L - L.max(1, keepdims=True)).sum(1)) + L.max(1) - L[np.arange(M), targets]
    assert np.abs(loss - ref).max() < 1e-9 * np.abs(ref).max()


def test_vocab_ce_target_logit_from_one_rank():
    """Exactly one rank holds each target; the others report 0."""
    rng = np.random.default_rng(45)
    V, h, M, P = 12, 3, 30, 3
    H, E = rng.normal(size=(M, h)), rng.normal(size=(V, h))
    targets = rng.integers(0, V, M)
    Vr = V // P
    for r in range(P):
        _, _, t = oracle.vocab_ce_shard_stats(H, E[r * Vr:(r + 1) * Vr], targets, r * Vr)
        mine = (targets >= r * Vr) & (targets < (r + 1) * Vr)
        assert not t[~mine].any()
        assert np.allclose(t[mine], (H @ E.T)[np.nonzero(mine)[0], targets[mine]], atol=1e-13)


# ---------------------------------------------- K/V-split attention (strategy B)
def _sdpa64(Q, K, V, causal):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(t))[None, None] for t in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)[0, 0].numpy()


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_kv_split_matches_library_attention(P, causal):
    """Summing the feature slices' partial scores before the softmax and
    concatenating the ranks' output slices gives the head's attention: the
    same as float64 scaled_dot_product_attention on the unsplit Q, K, V."""
    rng = np.random.default_rng(100 + P)
    s, d = 37, 32
    Q, K, V = (rng.standard_normal((s, d)) for _ in range(3))
    _, O = oracle.attention_kv_split(Q, K, V, P, causal)
    ref = _sdpa64(Q, K, V, causal)
    assert np.abs(O - ref).max() <= 1e-12 * np.abs(ref).max()


def test_kv_split_partial_scores_sum_to_full_scores():
    rng = np.random.default_rng(7)
    s, d, P = 19, 16, 4
    Q, K, V = (rng.standard_normal((s, d)) for _ in range(3))
    parts, _ = oracle.attention_kv_split(Q, K, V, P, True)
    assert parts.shape == (P, s, s)
    full = Q @ K.T
    assert np.abs(parts.sum(axis=0) - full).max() <= 1e-12 * np.abs(full).max()
    # every partial is a product over its own features only
    w = d // P
    assert np.array_equal(parts[2], Q[:, 2 * w:3 * w] @ K[:, 2 * w:3 * w].T)


def test_kv_split_softmax_of_partials_is_wrong():
    """Negative control: finishing each rank's softmax on its own partial
    scores (and averaging the ranks' outputs) is not the attention; the sum of
    the partial scores must come first."""
    rng = np.random.default_rng(8)
    s, d, P = 24, 16, 2
    Q, K, V = (rng.standard_normal((s, d)) * 2 for _ in range(3))
    parts, O = oracle.attention_kv_split(Q, K, V, P, False)
    w = d // P
    wrong = []
    for r in range(P):
        S = parts[r] / math.sqrt(d)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        wrong.append((E / E.sum(axis=1, keepdims=True)) @ V)
    wrong = sum(wrong) / P
    assert np.abs(wrong - O).max() > 0.1 * np.abs(O).max()


def test_kv_split_brute_force():
    """Tiny case by scalar loops: s = 3, d = 4, P = 2, causal."""
    Q = [[0.5, -1.0, 2.0, 0.25], [1.5, 0.0, -0.5, 1.0], [-2.0, 1.0, 0.5, -0.75]]
    K = [[1.0, 0.5, -0.5, 2.0], [-1.0, 1.5, 0.25, 0.0], [0.5, -2.0, 1.0, 1.0]]
    V = [[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 0.0, 2.0], [0.25, -0.5, 1.5, -1.0]]
    s, d, P = 3, 4, 2
    w = d // P
    ref = [[0.0] * d for _ in range(s)]
    for t in range(s):
        sc = []
        for u in range(t + 1):
            part = [math.fsum(Q[t][c] * K[u][c] for c in range(r * w, (r + 1) * w)) for r in range(P)]
            sc.append(math.fsum(part) / math.sqrt(d))
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        z = math.fsum(e)
        for c in range(d):
            ref[t][c] = math.fsum(e[u] / z * V[u][c] for u in range(t + 1))
    _, O = oracle.attention_kv_split(np.array(Q), np.array(K), np.array(V), P, True)
    assert np.abs(O - np.array(ref)).max() <= 1e-14


def test_kv_split_rows_layout():
    """The fused-projection wrapper splits heads and Q/K/V blocks as the
    attention core's layout does: it equals the per-head attention oracle."""
    rng = np.random.default_rng(9)
    b, s, H, d, P = 2, 11, 3, 16, 4
    qkv = rng.standard_normal((b * s, 3 * H * d))
    O = oracle.attention_kv_split_rows(qkv, b, s, H, d, P, True)
    HD = H * d
    for beta in range(b):
        rows = slice(beta * s, (beta + 1) * s)
        ref = oracle.attention_rows(qkv[rows, :HD], qkv[rows, HD:2 * HD], qkv[rows, 2 * HD:],
                                    np.arange(s), H, d, True)
        assert np.abs(O[rows] - ref).max() <= 1e-12
