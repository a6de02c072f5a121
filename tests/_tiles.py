"""The bf16 GEMM's choice of output-tile width, restated for the tests.

A launch is costed in waves of workgroups (one 256-row tile per workgroup,
one workgroup per compute unit): a wave of 256-column tiles counts 16, of
192-column tiles 14, of 384-column tiles 23.  A width other than 256 is
taken only when it saves more than 2 (1/8 of a 256-column wave), 192 before
384; 384-column tiles exist for the forward layout (plain, GeLU and the
dual-store epilogues) and the input-gradient layout (B transposed: plain and
GeLU backward; also the cross-entropy statistics, which have no 192-column
kernel) with K a multiple of 64, not for the weight-gradient layout (A
transposed).
"""


def tiles(prods, w):
    return sum(-(-m // 256) * -(-n // w) for m, n in prods)


def waves(prods, w, cus=256):
    return -(-tiles(prods, w) // cus)


def tile_cols(prods, K, *, trans_a=False, trans_b=False, epilogue="none", cus=256):
    if tiles(prods, 192) > 0x7FFFFFFF // 16:
        return 256
    best, cost = 256, 16 * waves(prods, 256, cus)
    if epilogue != "ce_stats" and 14 * waves(prods, 192, cus) < cost - 2:
        best, cost = 192, 14 * waves(prods, 192, cus)
    epis = ("none", "gelu_bwd", "ce_stats") if trans_b else ("none", "gelu", "gelu_save")
    wide_ok = not trans_a and epilogue in epis and K % 64 == 0
    if wide_ok and 23 * waves(prods, 384, cus) < cost - 2:
        best = 384
    return best
