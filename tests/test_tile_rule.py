"""The GEMM's output-tile width rule as the library applies it (host logic,
CPU: with no GPU present the library answers for 256 compute units) against
its restatement in _tiles.py, over shapes that fall on every side of the
cost model's thresholds.  The width never changes a result; the GPU tests
pin each width's arithmetic against the oracle."""
import itertools

import pytest

import transformer_tensor_shard_amd as tts
from _tiles import tile_cols


@pytest.fixture(scope="module")
def lib():
    try:
        tts.lib()
    except RuntimeError as e:       # not built
        pytest.skip(str(e))


LAYOUTS = [dict(), dict(trans_b=True), dict(trans_a=True)]
EPIS = {(): ["none", "gelu", "gelu_save"], ("trans_b",): ["none", "gelu_bwd"], ("trans_a",): ["none"]}


def test_rule_matches_restatement(lib):
    Ms = [256, 2250, 2304, 4096, 8192, 12288, 16384]
    Ns = [1536, 2048, 3072, 3904, 4608, 6144, 7680, 12288]
    checked = 0
    for lay, M, N, K, count in itertools.product(LAYOUTS, Ms, Ns, [64, 72, 128, 12288], [1, 3, 8]):
        for epi in EPIS[tuple(lay)]:
            prods = [(M, N)] * count
            want = tile_cols(prods, K, epilogue=epi, **lay)
            got = tts.tp_gemm_tile_cols(prods, K, epilogue=epi, **lay)
            assert got == want, (lay, epi, prods, K, got, want)
            checked += 1
    assert checked > 1000


def test_rule_on_the_benchmarked_products(lib):
    """The block's four forward products at the 175B layer shape (8 ranks) and
    one rank's take 384-column tiles; the h = 4096 MLP shard keeps 256; the
    tp = 4 attention share's QKV product takes 384 (256 tiles, one wave,
    against two waves of 192-column tiles), its W_o product keeps 256."""
    big = {((16384, 6144), 12288, "gelu"), ((16384, 4608), 12288, "none"),
           ((16384, 12288), 6144, "none"), ((16384, 12288), 1536, "none")}
    for (shape, K, epi), count in itertools.product(big, [1, 8]):
        assert tts.tp_gemm_tile_cols([shape] * count, K, epilogue=epi) == 384, (shape, count)
    assert tts.tp_gemm_tile_cols([(8192, 2048)], 4096, epilogue="gelu") == 256
    assert tts.tp_gemm_tile_cols([(8192, 4096)], 2048) == 256
    assert tts.tp_gemm_tile_cols([(8192, 3072)], 4096) == 384
    assert tts.tp_gemm_tile_cols([(8192, 4096)], 1024) == 256
    # the training forward's dual store and the backward's input gradients
    # take 384 too; the weight gradients (A transposed) keep 256
    assert tts.tp_gemm_tile_cols([(16384, 6144)], 12288, epilogue="gelu_save") == 384
    assert tts.tp_gemm_tile_cols([(16384, 6144)], 12288, trans_b=True, epilogue="gelu_bwd") == 384
    assert tts.tp_gemm_tile_cols([(16384, 12288)], 6144, trans_b=True) == 384
    assert tts.tp_gemm_tile_cols([(16384, 12288)], 4608, trans_b=True) == 384
    assert tts.tp_gemm_tile_cols([(6144, 12288), (12288, 6144)], 16384, trans_a=True) == 256


def test_rule_rejects_invalid_launches(lib):
    for shapes, K, kw in [([], 64, {}), ([(0, 64)], 64, {}), ([(64, 64)], 0, {}),
                          ([(64, 64)] * 17, 64, {}),
                          ([(64, 64)], 64, dict(trans_a=True, trans_b=True))]:
        with pytest.raises(ValueError):
            tts.tp_gemm_tile_cols(shapes, K, **kw)
