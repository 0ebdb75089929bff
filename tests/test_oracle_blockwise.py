"""Pins of the blockwise oracle (oracle/blockwise.py): special cases that
reduce to the pinned rowwise and tensorwise quantizers and the pinned
rowwise-scaled GEMM, block locality, and a hand-built two-block product."""
import numpy as np
import pytest

import oracle
from oracle import blockwise as bw
from oracle import tensorwise as tw
from oracle.swiglu import round_bf16

CODECS = [oracle.E4M3FN, oracle.E4M3FNUZ]


def bits(rng, shape, scale=1.0):
    return round_bf16(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("codec", CODECS)
def test_row_blocks_of_one_tile_are_rowwise(codec):
    """Columns <= 128 and block_rows = 1: one tile per row, i.e. the rowwise quantizer."""
    x = bits(np.random.default_rng(0), (1, 37, 120), 3.0)
    q, s = bw.quantize_blockwise(x, 1, codec)
    qr, sr = oracle.quantize_rowwise(x[0], codec)
    assert np.array_equal(q[0], qr) and np.array_equal(s[0, :, 0], sr)


@pytest.mark.parametrize("codec", CODECS)
def test_single_square_tile_is_tensorwise(codec):
    x = bits(np.random.default_rng(1), (1, 100, 128), 2.0)
    q, s = bw.quantize_blockwise(x, 128, codec)
    qt, st = tw.quantize_tensorwise(x, codec)
    assert np.array_equal(q, qt) and s.shape == (1, 1, 1) and s[0, 0, 0] == st


def test_tiles_are_independent():
    """An outlier changes only its own tile's scale and codes; tiles cover ragged edges."""
    rng = np.random.default_rng(2)
    x = bits(rng, (2, 200, 300))
    q0, s0 = bw.quantize_blockwise(x, 128, oracle.E4M3FN)
    assert s0.shape == (2, 2, 3)
    y = x.copy()
    y[1, 150, 260] = round_bf16(np.array([1000.0]))[0]
    q1, s1 = bw.quantize_blockwise(y, 128, oracle.E4M3FN)
    changed = s1 != s0
    assert changed.sum() == 1 and changed[1, 1, 2]
    mask = np.ones_like(q0, bool)
    mask[1, 128:, 256:] = False
    assert np.array_equal(q0[mask], q1[mask])


@pytest.mark.parametrize("codec", CODECS)
def test_gemm_one_contraction_block_matches_rowwise_gemm(codec):
    """K <= 128 and N <= 128: one scale per row of A and one per expert of B, i.e. the rowwise GEMM
    with those scales."""
    rng = np.random.default_rng(3)
    M, N, K, E = 90, 100, 112, 3
    offs = np.array([30, 30, 90], np.int32)
    qa, sa = bw.quantize_blockwise(bits(rng, (1, M, K)), 1, codec)
    qb, sb = bw.quantize_blockwise(bits(rng, (E, N, K), 0.02), 128, codec)
    got = bw.mm_grouped_m_blockwise(qa[0], sa[0], qb, sb, offs, codec, codec)
    want = oracle.mm_grouped_m(qa[0], sa[0, :, 0], qb, np.repeat(sb[:, 0, :], N, axis=1), offs, codec, codec)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.allclose(got[fin], want[fin], rtol=1e-14, atol=0)


def test_gemm_two_blocks_by_hand():
    """K = 256 in two blocks with different scales; values chosen so every code is exact."""
    codec = oracle.E4M3FN
    a = np.zeros((1, 1, 256))
    a[0, 0, 0], a[0, 0, 128] = 2.0, 0.5          # block maxima 2 and 0.5
    b = np.zeros((1, 1, 256))
    b[0, 0, 0], b[0, 0, 128] = 4.0, 1.0
    qa, sa = bw.quantize_blockwise(round_bf16(a), 1, codec)
    qb, sb = bw.quantize_blockwise(round_bf16(b), 128, codec)
    out = bw.mm_grouped_m_blockwise(qa[0], sa[0], qb, sb, np.array([1], np.int32), codec, codec)
    assert out[0, 0] == 2.0 * 4.0 + 0.5 * 1.0


def test_gemm_equals_dequantized_product():
    rng = np.random.default_rng(4)
    M, N, K = 64, 300, 400
    qa, sa = bw.quantize_blockwise(bits(rng, (1, M, K)), 1, oracle.E4M3FN)
    qb, sb = bw.quantize_blockwise(bits(rng, (1, N, K), 0.02), 128, oracle.E4M3FN)
    got = bw.mm_grouped_m_blockwise(qa[0], sa[0], qb, sb, np.array([M], np.int32), 0, 0)
    A = bw.dequantize_blockwise(qa, sa, 1, 0)[0]
    B = bw.dequantize_blockwise(qb, sb, 128, 0)[0]
    assert np.allclose(got, A @ B.T, rtol=1e-12, atol=1e-12)


def test_token_blocks_restart_at_groups():
    blocks = bw.token_blocks(np.array([130, 130, 400, 999], np.int32), 500)
    assert blocks == [(0, 0, 128), (0, 128, 130), (2, 130, 258), (2, 258, 386), (2, 386, 400), (3, 400, 500)]


@pytest.mark.parametrize("codec", CODECS)
def test_token_blocks_of_short_groups_are_colwise(codec):
    """Groups of at most 128 tokens: one block per group, i.e. the colwise grouped quantizer."""
    rng = np.random.default_rng(5)
    offs = np.array([50, 50, 170, 290], np.int32)
    x = bits(rng, (300, 64), 2.0)
    init = np.full((64, 304), 0x5A, np.uint8)
    q, s = bw.quantize_blockwise_tokens(x, offs, codec, ld_q=304, q_init=init)
    qc, sc = oracle.quantize_colwise_grouped(x, offs, codec, q_init=init, ld_q=304)
    assert np.array_equal(q, qc)
    assert np.array_equal(s, sc[[0, 2, 3]])              # the empty group 1 has no block


def test_grouped_k_one_block_per_group_matches_colwise_gemm():
    rng = np.random.default_rng(6)
    offs = np.array([100, 100, 228, 300], np.int32)
    M, N, K = 300, 72, 40
    qa, sa = bw.quantize_blockwise_tokens(bits(rng, (M, N), 1e-3), offs, 0)
    qb, sb = bw.quantize_blockwise_tokens(bits(rng, (M, K)), offs, 0)
    got = bw.mm_grouped_k_blockwise(qa, sa, qb, sb, offs, 0, 0)
    full = lambda s: np.insert(s, 1, 1.0, axis=0)         # the empty group: any scale (no tokens)
    want = oracle.mm_grouped_k(qa, full(sa), qb, full(sb), offs, 0, 0)
    assert np.allclose(got, want, rtol=1e-14, atol=0)
    assert not got[1].any()


def test_grouped_k_blocks_sum_by_hand():
    """One group of 256 tokens in two blocks with different scales; exact codes."""
    a = np.zeros((256, 1))
    b = np.zeros((256, 1))
    a[3, 0], a[200, 0] = 2.0, 0.25
    b[3, 0], b[200, 0] = 1.0, 8.0
    qa, sa = bw.quantize_blockwise_tokens(round_bf16(a), np.array([256], np.int32), 0)
    qb, sb = bw.quantize_blockwise_tokens(round_bf16(b), np.array([256], np.int32), 0)
    out = bw.mm_grouped_k_blockwise(qa, sa, qb, sb, np.array([256], np.int32), 0, 0)
    assert out[0, 0, 0] == 2.0 * 1.0 + 0.25 * 8.0
