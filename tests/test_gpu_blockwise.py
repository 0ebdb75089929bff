"""GPU parity of blockwise scaling: quantize_blockwise bit-exact against the
oracle (oracle/blockwise.py), grouped_mm_blockwise within the grouped GEMM's
error bounds of the oracle's exact per-block sum."""
import numpy as np
import pytest
import torch

import mxfp8_quantized_moe_amd as fm
from mxfp8_quantized_moe_amd import synth
from oracle import blockwise as bw
from oracle import gemm as og
from oracle.swiglu import round_bf16
from gpu_helpers import DEV, note, bf16_dev, i32_dev, host, assert_bytes_equal, assert_f32_bits_equal
from test_gpu_gemm import check, _out_host, SENT_BF16

pytestmark = pytest.mark.gpu


def make(seed, shape, scale=1.0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * scale
    if outliers and x.size:
        x.reshape(-1)[rng.integers(0, x.size, 5)] *= 40.0
    return round_bf16(x)


@pytest.mark.parametrize("codec", [fm.E4M3FN, fm.E4M3FNUZ])
@pytest.mark.parametrize("shape,br", [((1, 37, 120), 1), ((1, 300, 520), 1), ((2, 65, 8), 1), ((3, 200, 296), 128),
                                      ((2, 129, 136), 128), ((1, 128, 128), 128), ((1, 0, 64), 1),
                                      ((1, 1, 4096), 128)])
def test_quantize_blockwise_parity(codec, shape, br):
    x = make(sum(shape) + br, shape)
    note(f"quantize_blockwise shape={shape} block_rows={br} codec={codec}")
    q, s = fm.quantize_blockwise(bf16_dev(x).view(*shape), br, codec)
    qr, sr = bw.quantize_blockwise(x, br, codec)
    assert_bytes_equal(host(q), qr, "codes")
    assert_f32_bits_equal(host(s), sr, "scales")


def gemm_case(x, w, offs, out_dtype=0, what=""):
    M, K = x.shape
    E, N, _ = w.shape
    note(f"grouped_mm_blockwise {what} M={M} N={N} K={K} E={E} out={out_dtype}")
    qa, sa = fm.quantize_blockwise(bf16_dev(x), 1)
    qb, sb = fm.quantize_blockwise(bf16_dev(w).view(E, N, K), 128)
    odt = torch.bfloat16 if out_dtype == 0 else torch.float32
    out = torch.empty((M, N), dtype=odt, device=DEV)
    if out_dtype == 0:
        out.view(torch.int16).fill_(SENT_BF16)
    else:
        out.fill_(float("nan"))
    fm.grouped_mm_blockwise(qa, sa.view(M, -1), qb, sb, i32_dev(offs), E, M, N, K, out=out, out_dtype=out_dtype)
    raw, got = _out_host(out)
    qa_h, sa_h, qb_h, sb_h = host(qa), host(sa).reshape(M, -1), host(qb), host(sb)
    ref = bw.mm_grouped_m_blockwise(qa_h, sa_h, qb_h, sb_h, offs, 0, 0)
    A = bw.dequantize_blockwise(qa_h[None], sa_h[None], 1, 0)[0]
    B = bw.dequantize_blockwise(qb_h, sb_h, 128, 0)
    check(got, ref, *og.error_bounds_m(A, B, offs, og.ACC_FP8_MFMA), f"blockwise {what}")
    rows_out = np.isnan(ref[:, 0]) if N else np.zeros(M, bool)
    if out_dtype == 0:
        assert np.all(raw[rows_out] == SENT_BF16), "wrote rows outside every group"


def test_blockwise_gemm_ragged_groups():
    counts = synth.random_counts(41, 700, 5)
    offs = synth.offsets_from_counts(counts)
    x = make(42, (720, 400))                      # 20 rows past the last group; K = 3 blocks + 16
    w = make(43, (5, 200, 400), 0.02)
    gemm_case(x, w, offs, what="ragged")


def test_blockwise_gemm_f32_out_and_malformed_offsets():
    x = make(44, (300, 256))
    w = make(45, (4, 136, 256), 0.02)
    gemm_case(x, w, np.array([100, 40, 250, 999], np.int32), out_dtype=1, what="malformed f32")


def test_blockwise_gemm_dense_one_block():
    x = make(46, (256, 128))
    w = make(47, (1, 384, 128), 0.02)
    gemm_case(x, w, np.array([256], np.int32), what="one block")


def test_blockwise_gemm_llama3_forward_sampled():
    """The Llama3-8B forward shape (M = 8192, N = 14336, K = 4096) in the launch the bench times;
    64 rows x 256 columns sampled for the oracle."""
    M, N, K = 8192, 14336, 4096
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    x = torch.randn(M, K, device=DEV, generator=gen).to(torch.bfloat16)
    w = (torch.randn(N, K, device=DEV, generator=gen) * 0.02).to(torch.bfloat16)
    note("grouped_mm_blockwise llama3 forward")
    qa, sa = fm.quantize_blockwise(x, 1)
    qb, sb = fm.quantize_blockwise(w.view(1, N, K), 128)
    out = fm.grouped_mm_blockwise(qa, sa.view(M, -1), qb, sb, i32_dev([M]), 1, M, N, K)
    rows = np.random.default_rng(6).choice(M, 64, replace=False)
    n0 = 128 * 37
    qa_h, sa_h = host(qa)[rows], host(sa).reshape(M, -1)[rows]
    qb_h, sb_h = host(qb)[:, n0:n0 + 256], host(sb)[:, n0 // 128:n0 // 128 + 2]
    ref = bw.mm_grouped_m_blockwise(qa_h, sa_h, qb_h, sb_h, np.array([64], np.int32), 0, 0)
    A = bw.dequantize_blockwise(qa_h[None], sa_h[None], 1, 0)[0]
    B = bw.dequantize_blockwise(qb_h, sb_h, 128, 0)
    got = _out_host(out)[1][rows][:, n0:n0 + 256]
    check(got, ref, *og.error_bounds_m(A, B, np.array([64], np.int32), og.ACC_FP8_MFMA), "blockwise llama3 sampled")


def _deq_tokens(q_t, s, offs, M):
    out = np.zeros(q_t[:, :M].shape)
    for tb, (_, t0, t1) in enumerate(bw.token_blocks(offs, M)):
        out[:, t0:t1] = bw.decode(q_t[:, t0:t1], 0) / s[tb].astype(np.float64)[:, None]
    return out


@pytest.mark.parametrize("codec", [fm.E4M3FN, fm.E4M3FNUZ])
@pytest.mark.parametrize("M,C,offs", [(700, 200, [130, 130, 400, 690]), (512, 64, [512]), (300, 136, [5, 300]),
                                      (129, 8, [0, 129])])
def test_quantize_blockwise_tokens_parity(codec, M, C, offs):
    offs = np.array(offs, np.int32)
    x = make(M + C, (M, C))
    ld = (M + 15) // 16 * 16 + 16
    q_t = torch.full((C, ld), 0xA5, dtype=torch.uint8, device=DEV)
    note(f"quantize_blockwise_tokens M={M} C={C} offs={offs.tolist()} codec={codec}")
    q_t, s = fm.quantize_blockwise_tokens(bf16_dev(x), i32_dev(offs), codec, ld_q=ld, q_t=q_t)
    qr, sr = bw.quantize_blockwise_tokens(x, offs, codec, ld_q=ld, q_init=np.full((C, ld), 0xA5, np.uint8))
    assert_bytes_equal(host(q_t), qr, "codes")
    assert_f32_bits_equal(host(s)[:len(sr)], sr, "scales")


def gemm_k_case(dy, x, offs, out_dtype=0, what=""):
    M, N = dy.shape
    K = x.shape[1]
    E = len(offs)
    note(f"grouped_mm_blockwise_k {what} M={M} N={N} K={K} E={E}")
    qa, sa = fm.quantize_blockwise_tokens(bf16_dev(dy), i32_dev(offs))
    qb, sb = fm.quantize_blockwise_tokens(bf16_dev(x), i32_dev(offs))
    out = fm.grouped_mm_blockwise_k(qa, sa, qb, sb, i32_dev(offs), M, out_dtype=out_dtype)
    _, got = _out_host(out)
    nb = len(bw.token_blocks(offs, M))
    qa_h, sa_h, qb_h, sb_h = host(qa), host(sa)[:nb], host(qb), host(sb)[:nb]
    ref = bw.mm_grouped_k_blockwise(qa_h, sa_h, qb_h, sb_h, offs, 0, 0)
    A, B = _deq_tokens(qa_h, sa_h, offs, M), _deq_tokens(qb_h, sb_h, offs, M)
    check(got, ref, *og.error_bounds_k(A, B, offs, og.ACC_FP8_MFMA), f"blockwise k {what}")


def test_blockwise_gemm_k_ragged_groups():
    offs = np.array([130, 130, 400, 690], np.int32)   # misaligned starts, an empty group, tail tokens
    gemm_k_case(make(51, (700, 200), 1e-3), make(52, (700, 136)), offs, what="ragged")


def test_blockwise_gemm_k_dense_f32():
    gemm_k_case(make(53, (1024, 256), 1e-3), make(54, (1024, 128)), np.array([1024], np.int32), out_dtype=1,
                what="dense f32")


def test_blockwise_gemm_k_llama3_sampled():
    """The Llama3-8B weight gradient (M = 8192 tokens, N = 14336, K = 4096) in the launch the bench times;
    64 rows x 256 columns of dW sampled for the oracle."""
    M, N, K = 8192, 14336, 4096
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    dy = (torch.randn(M, N, device=DEV, generator=gen) * 1e-3).to(torch.bfloat16)
    x = torch.randn(M, K, device=DEV, generator=gen).to(torch.bfloat16)
    offs = np.array([M], np.int32)
    note("grouped_mm_blockwise_k llama3 weight gradient")
    qa, sa = fm.quantize_blockwise_tokens(dy, i32_dev(offs))
    qb, sb = fm.quantize_blockwise_tokens(x, i32_dev(offs))
    out = fm.grouped_mm_blockwise_k(qa, sa, qb, sb, i32_dev(offs), M)
    rows = np.random.default_rng(8).choice(N, 64, replace=False)
    k0 = 128 * 11
    nb = M // 128
    qa_h, sa_h = host(qa)[rows], host(sa)[:nb][:, rows]
    qb_h, sb_h = host(qb)[k0:k0 + 256], host(sb)[:nb][:, k0:k0 + 256]
    ref = bw.mm_grouped_k_blockwise(qa_h, sa_h, qb_h, sb_h, offs, 0, 0)
    A, B = _deq_tokens(qa_h, sa_h, offs, M), _deq_tokens(qb_h, sb_h, offs, M)
    got = _out_host(out)[1][:, rows][:, :, k0:k0 + 256]
    check(got, ref, *og.error_bounds_k(A, B, offs, og.ACC_FP8_MFMA), "blockwise k llama3 sampled")
