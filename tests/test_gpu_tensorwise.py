"""GPU parity of quantize_tensorwise against the oracle (oracle/tensorwise.py):
codes (row-major and transposed), the broadcast scale, and untouched bytes,
all bit-exact."""
import numpy as np
import pytest
import torch

import mxfp8_quantized_moe_amd as fm
from oracle import tensorwise as tw
from oracle.swiglu import round_bf16
from gpu_helpers import DEV, note, bf16_dev, i32_dev, host, assert_bytes_equal, assert_f32_bits_equal

pytestmark = pytest.mark.gpu

CODECS = [fm.E4M3FN, fm.E4M3FNUZ]


def make_x(seed, shape, outlier=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * 2.0
    if outlier is not None and x.size:
        x.reshape(-1)[rng.integers(0, x.size)] = outlier
    return round_bf16(x)


def check(x, codec, ld_pad=16, n_scale=None, what=""):
    """x bf16 bits [B, R, C]: compare both layouts and the scale vector with the oracle."""
    B, R, C = x.shape
    ld_q = (R + ld_pad + 15) // 16 * 16
    n_scale = max(B * R, 1) if n_scale is None else n_scale
    q_t = torch.full((B, C, ld_q), 0xA5, dtype=torch.uint8, device=DEV)
    note(f"quantize_tensorwise {what} B={B} R={R} C={C} ld_q={ld_q} codec={codec} n_scale={n_scale}")
    q, q_t, s = fm.quantize_tensorwise(bf16_dev(x), codec, rowmajor=True, transposed=True, ld_q=ld_q,
                                       n_scale=n_scale, q_t=q_t)
    qr, sr = tw.quantize_tensorwise(x, codec)
    qtr, _ = tw.quantize_tensorwise_transposed(x, codec, ld_q=ld_q, q_init=np.full((B, C, ld_q), 0xA5, np.uint8))
    assert_bytes_equal(host(q), qr.reshape(B * R, C), f"{what} q")
    assert_bytes_equal(host(q_t), qtr, f"{what} q_t")
    assert_f32_bits_equal(host(s), np.full(n_scale, sr, np.float32), f"{what} scale")


SHAPES = [(1, 7, 8), (1, 128, 64), (1, 129, 72), (1, 300, 520), (3, 129, 136), (2, 1000, 8), (1, 1, 4096),
          (4, 33, 1408), (1, 0, 64), (1, 5, 0)]


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("shape", SHAPES)
def test_tensorwise_parity(codec, shape):
    check(make_x(sum(shape) + codec, shape, outlier=37.0), codec, what="shape")


@pytest.mark.parametrize("codec", CODECS)
def test_tensorwise_special_values(codec):
    """All zeros (eps floor), a single huge value, values at the codec's limits."""
    check(np.zeros((1, 40, 64), np.uint16), codec, what="zeros")
    x = np.zeros((1, 40, 64))
    x[0, 3, 5] = 3.0e38
    x[0, 10, :] = 1e-38
    check(round_bf16(x), codec, what="huge")
    x = make_x(9, (1, 64, 64))
    x.reshape(-1)[:4] = round_bf16(np.array([448.0, -448.0, 240.0, -0.0]))
    check(x, codec, what="limits")


def test_tensorwise_layout_options():
    """Row-major only and transposed only; a scale vector longer than the rows; a second, smaller
    call reusing the workspace."""
    x = make_x(3, (2, 200, 96))
    qr, sr = tw.quantize_tensorwise(x, fm.E4M3FN)
    ws = torch.full((int(fm._lib.lib().quantize_tensorwise_workspace_bytes()),), 0x7F, dtype=torch.uint8,
                    device=DEV)
    note("quantize_tensorwise row-major only")
    q, qt, s = fm.quantize_tensorwise(bf16_dev(x), fm.E4M3FN, rowmajor=True, transposed=False, n_scale=777,
                                      workspace=ws)
    assert qt is None
    assert_bytes_equal(host(q), qr.reshape(400, 96), "q")
    assert_f32_bits_equal(host(s), np.full(777, sr, np.float32), "scale")
    note("quantize_tensorwise transposed only")
    q, qt, s = fm.quantize_tensorwise(bf16_dev(x), fm.E4M3FN, rowmajor=False, transposed=True, n_scale=3,
                                      workspace=ws)
    assert q is None
    assert qt.shape == (2, 96, 208)
    assert_bytes_equal(host(qt)[:, :, :200], qr.transpose(0, 2, 1), "q_t")
    small = make_x(4, (1, 50, 32))
    q, _, s = fm.quantize_tensorwise(bf16_dev(small), fm.E4M3FN, workspace=ws)
    qs, ss = tw.quantize_tensorwise(small, fm.E4M3FN)
    assert_bytes_equal(host(q), qs.reshape(50, 32), "second call q")
    assert_f32_bits_equal(host(s), np.full(50, ss, np.float32), "second call scale")


def test_tensorwise_full_size_llama3_x():
    """The Llama3-8B linear layer's activations [8192, 4096] with both layouts, compared in full."""
    x = make_x(11, (1, 8192, 4096), outlier=80.0)
    check(x, fm.E4M3FN, ld_pad=0, what="llama3 X")


def _tw(x_bits, n_scale, transposed=False, ld_q=None):
    B, R, C = (1, *x_bits.shape) if x_bits.ndim == 2 else x_bits.shape
    return fm.quantize_tensorwise(bf16_dev(x_bits).view(B, R, C), fm.E4M3FN, rowmajor=True, transposed=transposed,
                                  ld_q=ld_q, n_scale=n_scale)


def test_tensorwise_recipe_dense_layer_gemms():
    """fwd, dgrad and wgrad of a dense linear layer on tensorwise operands through the unchanged
    grouped GEMM (scales broadcast into its fp32 vectors), against the oracle GEMMs and bounds."""
    from oracle import gemm as og
    from test_gpu_gemm import check, _out_host
    M, H, F2 = 512, 256, 384
    rng = np.random.default_rng(21)
    X = round_bf16(rng.standard_normal((M, H)))
    W = round_bf16(rng.standard_normal((F2, H)) * 0.02)
    DY = round_bf16(rng.standard_normal((M, F2)) * 1e-3)
    offs = np.array([M], np.int32)
    note("tensorwise recipe: quantize X, W, dY")
    qx, qxt, sx = _tw(X, max(M, H), transposed=True)
    qw, qwt, sw = _tw(W, max(F2, H), transposed=True)
    qdy, qdyt, sdy = _tw(DY, max(M, F2), transposed=True)
    acc = og.ACC_FP8_MFMA
    h = lambda t: host(t)
    # forward: X [M, H] x W^T -> [M, F2]
    note("tensorwise recipe: fwd")
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qx, fm.OPD_E4M3FN, sx, qw.view(1, F2, H), fm.OPD_E4M3FN, sw,
                               fm.SCALE_F32, i32_dev(offs), 1, M, F2, H)
    qa, sa, qb, sb = h(qx), h(sx)[:M], h(qw).reshape(1, F2, H), h(sw)[:F2].reshape(1, F2)
    ref = og.mm_grouped_m(qa, sa, qb, sb, offs, 0, 0)
    A = oracle_dec(qa) / sa[:, None].astype(np.float64)
    Bm = oracle_dec(qb) / sb[..., None].astype(np.float64)
    check(_out_host(out)[1], ref, *og.error_bounds_m(A, Bm, offs, acc), "tensorwise fwd")
    # dgrad: dY [M, F2] x W -> [M, H]; W's transposed codes [1, H, F2]
    note("tensorwise recipe: dgrad")
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qdy, fm.OPD_E4M3FN, sdy, qwt.view(1, H, F2), fm.OPD_E4M3FN, sw,
                               fm.SCALE_F32, i32_dev(offs), 1, M, H, F2)
    qa, sa, qb, sb = h(qdy), h(sdy)[:M], h(qwt).reshape(1, H, F2), h(sw)[:H].reshape(1, H)
    ref = og.mm_grouped_m(qa, sa, qb, sb, offs, 0, 0)
    A = oracle_dec(qa) / sa[:, None].astype(np.float64)
    Bm = oracle_dec(qb) / sb[..., None].astype(np.float64)
    check(_out_host(out)[1], ref, *og.error_bounds_m(A, Bm, offs, acc), "tensorwise dgrad")
    # wgrad: dY^T [F2, M] x X^T [H, M] -> [1, F2, H]
    note("tensorwise recipe: wgrad")
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qdyt.view(F2, M), fm.OPD_E4M3FN, sdy, qxt.view(H, M), fm.OPD_E4M3FN,
                               sx, fm.SCALE_F32, i32_dev(offs), 1, M, F2, H)
    qa, sa, qb, sb = h(qdyt).reshape(F2, M), h(sdy)[:F2].reshape(1, F2), h(qxt).reshape(H, M), h(sx)[:H].reshape(1, H)
    ref = og.mm_grouped_k(qa, sa, qb, sb, offs, 0, 0)
    A = oracle_dec(qa) / sa[0][:, None].astype(np.float64)
    Bm = oracle_dec(qb) / sb[0][:, None].astype(np.float64)
    check(_out_host(out)[1], ref, *og.error_bounds_k(A, Bm, offs, acc), "tensorwise wgrad")


def test_tensorwise_recipe_moe_forward():
    """A grouped forward whose 3D expert weights share one tensorwise scale."""
    from oracle import gemm as og
    from test_gpu_gemm import check, _out_host
    from mxfp8_quantized_moe_amd import synth
    E, N, K = 5, 192, 256
    counts = synth.random_counts(31, 900, E)
    offs = synth.offsets_from_counts(counts)
    M = int(offs[-1])
    rng = np.random.default_rng(22)
    X = round_bf16(rng.standard_normal((M, K)))
    W = round_bf16(rng.standard_normal((E, N, K)) * 0.02)
    note("tensorwise recipe: MoE fwd")
    qx, _, sx = _tw(X, M)
    qw, _, sw = _tw(W, E * N)
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qx, fm.OPD_E4M3FN, sx, qw.view(E, N, K), fm.OPD_E4M3FN, sw,
                               fm.SCALE_F32, i32_dev(offs), E, M, N, K)
    qa, sa, qb, sb = host(qx), host(sx), host(qw).reshape(E, N, K), host(sw).reshape(E, N)
    qr, sr = tw.quantize_tensorwise(W, fm.E4M3FN)
    assert_bytes_equal(qb, qr, "3D weight codes")
    assert np.all(sb == sr)
    ref = og.mm_grouped_m(qa, sa, qb, sb, offs, 0, 0)
    A = oracle_dec(qa) / sa[:, None].astype(np.float64)
    Bm = oracle_dec(qb) / sb[..., None].astype(np.float64)
    check(_out_host(out)[1], ref, *og.error_bounds_m(A, Bm, offs, og.ACC_FP8_MFMA), "tensorwise MoE fwd")


def oracle_dec(q):
    import oracle
    return oracle.decode(q, fm.E4M3FN)
