"""GPU parity of the fused SwiGLU + rowwise quantization (forward and backward)
against the oracle (oracle/swiglu.py).

The bf16 activation and gradients are compared with the exact values rounded
once to bf16: the kernels compute in fp32 with their own exponential, so an
element whose exact value lies within a few fp32 ulps of a bf16 rounding
boundary may land one bf16 ulp away.  Bound: 1 ulp, on at most a fraction
2^-11 of the elements (the derivation is in gpu_helpers.assert_within_one_ulp).
Measured rates stay near 1e-5 to 3e-5.
The FP8 codes and scales are an integer decision, taken on the same
bf16 values on both sides: they must equal the oracle's rowwise quantizer
applied to the kernel's own bf16 output, bit for bit."""
import numpy as np
import pytest
import torch

import mxfp8_quantized_moe_amd as fm
import oracle
from oracle import swiglu as sw
from gpu_helpers import (DEV, note, bf16_dev, i32_dev, host, assert_bytes_equal, assert_f32_bits_equal,
                         assert_within_one_ulp)

pytestmark = pytest.mark.gpu

CODECS = [fm.E4M3FN, fm.E4M3FNUZ]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_h1(seed: int, R: int, F: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((R, F)).astype(np.float32) * 3
    u = rng.standard_normal((R, F)).astype(np.float32)
    if R and F:
        # exact zeros, both signs of up, the exponential's overflow region, tiny gates
        sp = np.float32([0.0, -0.0, 100.0, -100.0, 89.5, -89.5, 88.0, -88.0, 1e-30, -1e-30, 20.0, -20.0])
        k = min(F, len(sp))
        g[0, :k] = sp[:k]
        u[0, :k] = np.float32([3.0, -3.0] * 6)[:k]
    if R > 2:
        g[2] = 0.0                                   # an all-zero activation row
    return np.concatenate([bf16_bits(g), bf16_bits(u)], axis=1)


def make_da2(seed: int, R: int, F: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((R, F)).astype(np.float32) * 1e-3)


SHAPES = [(7, 8), (33, 64), (129, 1408), (64, 2048), (17, 8192), (3, 16384), (2, 24576), (300, 520), (0, 64)]


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("shape", SHAPES)
def test_swiglu_forward_parity(codec, shape):
    R, F = shape
    h1 = make_h1(10 + R + F, R, F)
    note(f"swiglu fwd codec={codec} rows={R} F={F}")
    a2, q, s = fm.swiglu_quantize_rowwise(bf16_dev(h1), codec)
    a2h = host(a2)
    assert_within_one_ulp(a2h, sw.swiglu_fwd(h1, F), "a2")
    qr, sr = oracle.quantize_rowwise(a2h, codec)
    assert_bytes_equal(host(q), qr, "a2 codes")
    assert_f32_bits_equal(host(s), sr, "a2 scales")
    note(f"swiglu fwd without codes codec={codec} rows={R} F={F}")
    a2b, qb, sb = fm.swiglu_quantize_rowwise(bf16_dev(h1), codec, codes=False)
    assert qb is None and sb is None
    assert_bytes_equal(host(a2b), a2h, "a2 without codes")


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("shape", SHAPES)
def test_swiglu_backward_parity(codec, shape):
    R, F = shape
    h1 = make_h1(20 + R + F, R, F)
    da2 = make_da2(30 + R + F, R, F)
    note(f"swiglu bwd codec={codec} rows={R} F={F}")
    dh1, q, s = fm.swiglu_backward_quantize_rowwise(bf16_dev(da2), bf16_dev(h1), codec)
    dh1h = host(dh1)
    assert_within_one_ulp(dh1h, sw.swiglu_bwd(da2, h1, F), "dh1")
    qr, sr = oracle.quantize_rowwise(dh1h, codec)
    assert_bytes_equal(host(q), qr, "dh1 codes")
    assert_f32_bits_equal(host(s), sr, "dh1 scales")
    note(f"swiglu bwd without codes codec={codec} rows={R} F={F}")
    dh1b, qb, sb = fm.swiglu_backward_quantize_rowwise(bf16_dev(da2), bf16_dev(h1), codec, codes=False)
    assert qb is None and sb is None
    assert_bytes_equal(host(dh1b), dh1h, "dh1 without codes")


def test_swiglu_strided_h1():
    R, F, LD = 65, 1408, 2 * 1408 + 40
    rng = np.random.default_rng(6)
    wide = bf16_bits(rng.standard_normal((R, LD)).astype(np.float32) * 2)
    h1 = np.ascontiguousarray(wide[:, :2 * F])
    da2 = make_da2(7, R, F)
    wd = bf16_dev(wide)[:, :2 * F]                  # row stride LD > 2F
    note("swiglu strided h1")
    a2, q, s = fm.swiglu_quantize_rowwise(wd, fm.E4M3FN)
    assert_within_one_ulp(host(a2), sw.swiglu_fwd(h1, F), "a2 (strided)")
    qr, sr = oracle.quantize_rowwise(host(a2), fm.E4M3FN)
    assert_bytes_equal(host(q), qr, "a2 codes (strided)")
    dh1, q2, s2 = fm.swiglu_backward_quantize_rowwise(bf16_dev(da2), wd, fm.E4M3FN)
    assert_within_one_ulp(host(dh1), sw.swiglu_bwd(da2, h1, F), "dh1 (strided)")
    qr2, sr2 = oracle.quantize_rowwise(host(dh1), fm.E4M3FN)
    assert_bytes_equal(host(q2), qr2, "dh1 codes (strided)")
    assert_f32_bits_equal(host(s2), sr2, "dh1 scales (strided)")


def test_swiglu_full_size_sampled():
    """DeepSeek-V3-share shape (8192 routed rows, F = 2048) in the launch the
    bench times; rows sampled for the oracle."""
    R, F = 8192, 2048
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    h1 = (torch.randn(R, 2 * F, device=DEV, generator=gen) * 2).to(torch.bfloat16)
    da2 = (torch.randn(R, F, device=DEV, generator=gen) * 1e-3).to(torch.bfloat16)
    note("swiglu full size")
    a2, q, s = fm.swiglu_quantize_rowwise(h1, fm.E4M3FN)
    dh1, qb, sb = fm.swiglu_backward_quantize_rowwise(da2, h1, fm.E4M3FN)
    rows = np.random.default_rng(12).choice(R, 96, replace=False)
    h1h, dah = host(h1)[rows], host(da2)[rows]
    a2h, dh1h = host(a2)[rows], host(dh1)[rows]
    assert_within_one_ulp(a2h, sw.swiglu_fwd(h1h, F), "a2 sampled")
    assert_within_one_ulp(dh1h, sw.swiglu_bwd(dah, h1h, F), "dh1 sampled")
    qr, sr = oracle.quantize_rowwise(a2h, fm.E4M3FN)
    assert_bytes_equal(host(q)[rows], qr, "a2 codes sampled")
    assert_f32_bits_equal(host(s)[rows], sr, "a2 scales sampled")
    qr, sr = oracle.quantize_rowwise(dh1h, fm.E4M3FN)
    assert_bytes_equal(host(qb)[rows], qr, "dh1 codes sampled")
    assert_f32_bits_equal(host(sb)[rows], sr, "dh1 scales sampled")


# ----------------------------------------------------------- SwiGLU fused with both MX forms

def _k4_rows(k4, R, NB):
    G = k4.shape[0]
    return np.ascontiguousarray(k4.transpose(1, 0, 2).reshape(R, 4 * G)[:, :NB])


def _check_mx_forms(t_bits, offs, rule, rows_pad, q, sc, q_t, sc_t, op, what):
    """Both MX forms of the bf16 tensor t (the kernel's own copy) against the oracle: last-dim blocks of the
    rows inside groups, padded row blocks per group (K4 scale layout)."""
    R, C = t_bits.shape
    covered = int(min(max(int(np.clip(offs, 0, R).max()), 0), R))
    ql, sl = oracle.quantize_mx_lastdim(t_bits[:covered], rule)
    assert_bytes_equal(host(q)[:covered], ql, f"{what} last-dim codes")
    assert_bytes_equal(_k4_rows(host(sc), R, C // 32)[:covered], sl.reshape(covered, C // 32), f"{what} last-dim e8m0")
    qt, st, opr = oracle.quantize_mx_rows_grouped(t_bits, offs, rule, rows_pad)
    assert_bytes_equal(host(op), opr, f"{what} padded offsets")
    assert_bytes_equal(host(q_t), qt, f"{what} row-block codes")
    assert_bytes_equal(_k4_rows(host(sc_t), C, rows_pad // 32), st, f"{what} row-block e8m0")


SW_MX_CASES = {
    "ragged": (700, 128, np.array([100, 100, 350, 690], np.int32)),       # an empty group, 10 rows in no group
    "wide": (300, 1408 + 128, np.array([37, 200, 300], np.int32)),
    "one_group": (96, 256, np.array([96], np.int32)),
}
# the forward also takes widths that are not a multiple of 128 (partial column tiles)
SW_MX_FWD_CASES = {**SW_MX_CASES, "narrow": (200, 32, np.array([70, 200], np.int32)),
                   "partial": (130, 1408 + 32, np.array([130], np.int32))}


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("case", list(SW_MX_FWD_CASES))
def test_swiglu_mx_dual_forward(rule, case):
    """A2 computed on the fly: its optional bf16 copy within one ulp of the exact value, both MX forms bit-exact
    against the oracle's quantizers of that copy, and the same codes when no copy is written."""
    R, F, offs = SW_MX_FWD_CASES[case]
    h1 = make_h1(40 + R + F, R, F)
    rows_pad = fm.quantize_mx_rows_bound(R, len(offs)) + 32
    a2 = torch.full((R, F), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    note(f"swiglu fwd + MX dual rule={rule} case={case}")
    _, q, sc, q_t, sc_t, op = fm.swiglu_quantize_mx_dual(bf16_dev(h1), i32_dev(offs), rule=rule, rows_pad=rows_pad,
                                                         a2=a2)
    covered = int(np.clip(offs, 0, R).max())
    a2h = host(a2)
    assert_within_one_ulp(a2h[:covered], sw.swiglu_fwd(h1[:covered], F), "a2 copy")
    assert np.all(a2h[covered:].view(np.int16) == 0x5A5A), "rows in no group must stay untouched"
    _check_mx_forms(a2h, offs, rule, rows_pad, q, sc, q_t, sc_t, op, "a2")
    note(f"swiglu fwd + MX dual without the copy rule={rule} case={case}")
    _, q2, sc2, qt2, sct2, _ = fm.swiglu_quantize_mx_dual(bf16_dev(h1), i32_dev(offs), rule=rule, rows_pad=rows_pad)
    assert_bytes_equal(host(q2)[:covered], host(q)[:covered], "without the copy: last-dim codes")
    assert_bytes_equal(_k4_rows(host(sc2), R, F // 32)[:covered], _k4_rows(host(sc), R, F // 32)[:covered],
                       "without the copy: last-dim e8m0")
    assert_bytes_equal(host(qt2), host(q_t), "without the copy: row-block codes")
    assert_bytes_equal(host(sct2), host(sc_t), "without the copy: row-block e8m0")


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("case", list(SW_MX_CASES))
def test_swiglu_mx_dual_backward(rule, case):
    R, F, offs = SW_MX_CASES[case]
    h1 = make_h1(50 + R + F, R, F)
    da2 = make_da2(60 + R + F, R, F)
    rows_pad = fm.quantize_mx_rows_bound(R, len(offs)) + 32
    dh1 = torch.full((R, 2 * F), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    note(f"swiglu bwd + MX dual rule={rule} case={case}")
    _, q, sc, q_t, sc_t, op = fm.swiglu_backward_quantize_mx_dual(bf16_dev(da2), bf16_dev(h1), i32_dev(offs), rule=rule,
                                                                  rows_pad=rows_pad, dh1=dh1)
    covered = int(np.clip(offs, 0, R).max())
    dh1h = host(dh1)
    assert_within_one_ulp(dh1h[:covered], sw.swiglu_bwd(da2[:covered], h1[:covered], F), "dh1 copy")
    _check_mx_forms(dh1h, offs, rule, rows_pad, q, sc, q_t, sc_t, op, "dh1")


def test_swiglu_mx_dual_llama4_scout_sampled():
    """The Llama4-Scout layer's shapes (16384 routed rows, F = 8192, 16 groups): the fused forward and backward
    against swiglu (bf16 copy, sampled rows) and the separate dual quantizer applied to that copy (whole
    tensors, bit for bit)."""
    from mxfp8_quantized_moe_amd import synth
    w = synth.WORKLOADS[5]
    offs = i32_dev(w.offs)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(55)
    h1 = (torch.randn(w.M, w.F2, device=DEV, generator=gen) * 0.5).to(torch.bfloat16)
    da2 = (torch.randn(w.M, w.F, device=DEV, generator=gen) * 1e-3).to(torch.bfloat16)
    a2 = torch.empty(w.M, w.F, dtype=torch.bfloat16, device=DEV)
    dh1 = torch.empty(w.M, w.F2, dtype=torch.bfloat16, device=DEV)
    note("swiglu + MX dual, Llama4-Scout shapes")
    _, q, sc, qt, sct, _ = fm.swiglu_quantize_mx_dual(h1, offs, a2=a2)
    r = fm.quantize_mx_dual(a2, offs=offs, layout=fm.MX_LAYOUT_K4)
    for g_, w_, n_ in zip((q, sc, qt, sct), r[:4], ("q", "scale", "q_t", "scale_t")):
        assert torch.equal(g_, w_), f"forward {n_} differs from quantize_mx_dual of the copy"
    _, q, sc, qt, sct, _ = fm.swiglu_backward_quantize_mx_dual(da2, h1, offs, dh1=dh1)
    r = fm.quantize_mx_dual(dh1, offs=offs, layout=fm.MX_LAYOUT_K4)
    for g_, w_, n_ in zip((q, sc, qt, sct), r[:4], ("q", "scale", "q_t", "scale_t")):
        assert torch.equal(g_, w_), f"backward {n_} differs from quantize_mx_dual of the copy"
    rows = np.random.default_rng(5).choice(w.M, 64, replace=False)
    h1h, dah = host(h1)[rows], host(da2)[rows]
    assert_within_one_ulp(host(a2)[rows], sw.swiglu_fwd(h1h, w.F), "a2 sampled")
    assert_within_one_ulp(host(dh1)[rows], sw.swiglu_bwd(dah, h1h, w.F), "dh1 sampled")
