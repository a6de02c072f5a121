"""The bf16 GEMM's choice of output-tile width, restated for the tests.

A launch whose products are all at most 128 columns wide takes 128-column
tiles (not the cross-entropy statistics).  Otherwise a launch is costed in waves of workgroups (one 256-row tile per workgroup,
one workgroup per compute unit): a wave of 256-column tiles counts 16, of
192-column tiles 14, of 384-column tiles 23.  A width other than 256 is
taken only when it saves more than 2 (1/8 of a 256-column wave), 192 before
384; 384-column tiles exist for the forward layout (plain, GeLU and the
dual-store epilogues) and the input-gradient layout (B transposed: plain and
GeLU backward; also the cross-entropy statistics, which have no 192-column
kernel) with K a multiple of 64, not for the weight-gradient layout (A
transposed).

A launch with f32 output and no epilogue, on 256- or 192-column tiles, whose
caller offers spare device memory may split its last, partly filled wave:
with W = 8·sum_g ceil(tiles_g / 8) workgroups (each XCD takes its share of
every product's tiles) the last
wave holds t = W mod CUs; 4 ways when 4t <= CUs and K >= 8192, else 2 ways
when 2t <= CUs and K >= 4096, K a multiple of 64·ways, and (ways - 1)·t
blocks of 256 x width f32 fitting the spare memory.
"""


def tiles(prods, w):
    return sum(-(-m // 256) * -(-n // w) for m, n in prods)


def waves(prods, w, cus=256):
    return -(-tiles(prods, w) // cus)


def tile_cols(prods, K, *, trans_a=False, trans_b=False, epilogue="none", cus=256):
    if tiles(prods, 192) > 0x7FFFFFFF // 16:
        return 256
    if epilogue != "ce_stats" and all(n <= 128 for m, n in prods):
        return 128
    best, cost = 256, 16 * waves(prods, 256, cus)
    if epilogue != "ce_stats" and 14 * waves(prods, 192, cus) < cost - 2:
        best, cost = 192, 14 * waves(prods, 192, cus)
    epis = ("none", "gelu_bwd", "ce_stats") if trans_b else ("none", "gelu", "gelu_save")
    wide_ok = not trans_a and epilogue in epis and K % 64 == 0
    if wide_ok and 23 * waves(prods, 384, cus) < cost - 2:
        best = 384
    return best


def workgroups(prods, w):
    def cdiv(a, b):
        return -(-a // b)
    return 8 * sum(cdiv(cdiv(m, 256) * cdiv(n, w), 8) for m, n in prods)


def split_ways(prods, K, spare_bytes, w=256, cus=256):
    tail = workgroups(prods, w) % cus
    if tail == 0:
        return 0
    for ways in (4, 2):
        if ways * tail > cus or K % (64 * ways) or K < 2048 * ways:
            continue
        if (ways - 1) * tail * 256 * w * 4 <= spare_bytes:
            return ways
    return 0
