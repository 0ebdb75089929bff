"""GPU parity of the grouped GEMMs against the fp64 oracle.

Operands are the GPU's own quantized tensors (their bytes are checked
bit-exactly by test_gpu_quant), fed to both sides, so GEMM and quantization
are tested independently.  Acceptance per element:
  contract:   |out - ref| <= 1e-2 * ||a_row|| * ||b_col||   (dequantized operands)
  diagnostic: |out - ref| <= 2^-8 |ref| + rel * sum|a*b|, rel = K * 2^-23 for
              bf16 MFMA and 2^-10 for the FP8 matrix cores, which keep fewer
              bits than fp32 inside one instruction (test_fp8_mfma_accumulation)
Rows of GROUPED_M outside every group must keep their sentinel; empty groups
of GROUPED_K must be exact zeros.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_quantized_moe_amd as fm
from mxfp8_quantized_moe_amd import synth
from gpu_helpers import DEV, note, bf16_dev, i32_dev, host, bf16_bits_to_f64, e8m0_rows_to_k4

pytestmark = pytest.mark.gpu

SENT_BF16 = 0x7FC1      # a NaN pattern the kernel never writes


def _out_host(t):
    h = host(t)
    if t.dtype == torch.bfloat16:
        return h, bf16_bits_to_f64(h)
    return h.view(np.uint32), h.astype(np.float64)


def check(got, ref, contract, tight, what):
    """got/ref/bounds float64; NaN in ref marks positions that are not compared."""
    fin = ~np.isnan(ref)
    err = np.abs(got[fin] - ref[fin])
    assert not np.any(np.isnan(got[fin])), f"{what}: NaN in output"
    bad_c = err > contract[fin]
    bad_t = err > tight[fin]
    assert not bad_c.any(), f"{what}: {bad_c.sum()} elements beyond the contract bound (max err {err.max():.3e})"
    assert not bad_t.any(), f"{what}: {bad_t.sum()} elements beyond the diagnostic bound (max err {err.max():.3e})"


def gm_case(x_bits, w_bits, offs, codec_a=0, codec_b=0, out_dtype=0, name=""):
    """Quantize on the GPU (rowwise), run GROUPED_M, compare with the oracle."""
    M, K = x_bits.shape
    E, N, _ = w_bits.shape
    note(f"GROUPED_M {name} M={M} N={N} K={K} E={E} codecs={codec_a},{codec_b} out={out_dtype}")
    qa, sa = fm.quantize_rowwise(bf16_dev(x_bits), codec_a)
    qb, sb = fm.quantize_rowwise(bf16_dev(w_bits.reshape(E * N, K)), codec_b)
    odt = torch.bfloat16 if out_dtype == 0 else torch.float32
    out = torch.empty((M, N), dtype=odt, device=DEV)
    if out_dtype == 0:
        out.view(torch.int16).fill_(SENT_BF16)
    else:
        out.fill_(float("nan"))
    fmt = {0: fm.OPD_E4M3FN, 1: fm.OPD_E4M3FNUZ}
    fm.grouped_mm_scaled(fm.GROUPED_M, qa, fmt[codec_a], sa, qb, fmt[codec_b], sb, fm.SCALE_F32,
                         i32_dev(offs), E, M, N, K, out=out, out_dtype=out_dtype)
    raw, got = _out_host(out)
    qa_h, sa_h, qb_h, sb_h = host(qa), host(sa), host(qb).reshape(E, N, K), host(sb).reshape(E, N)
    ref = oracle.mm_grouped_m(qa_h, sa_h, qb_h, sb_h, offs, codec_a, codec_b)
    A = oracle.decode(qa_h, codec_a) / sa_h[:, None].astype(np.float64)
    B = oracle.decode(qb_h, codec_b) / sb_h[..., None].astype(np.float64)
    acc = oracle.ACC_FP8_MFMA if codec_a == 0 and codec_b == 0 else oracle.ACC_FP32
    contract, tight = oracle.error_bounds_m(A, B, offs, acc)
    check(got, ref, contract, tight, f"GROUPED_M {name}")
    rows_out = np.isnan(ref[:, 0]) if N else np.zeros(M, bool)
    if out_dtype == 0:
        assert np.all(raw[rows_out] == SENT_BF16), "wrote rows outside every group"
    else:
        assert np.all(np.isnan(got[rows_out])), "wrote rows outside every group"


GM_CASES = {
    "cfg1": lambda: (synth.make_x(synth.WORKLOADS[1]), synth.make_w1(synth.WORKLOADS[1]), synth.WORKLOADS[1].offs),
    "ragged": lambda: (synth.normal_bf16(11, (700, 384), 1.0, 0.01, 50.0), synth.normal_bf16(12, (9, 320, 384), 0.02),
                       synth.offsets_from_counts(synth.random_counts(13, 680, 9))),
    "dense": lambda: (synth.normal_bf16(14, (600, 512), 1.0), synth.normal_bf16(15, (1, 300, 512), 0.02),
                      np.array([600], np.int32)),
    "malformed": lambda: (synth.normal_bf16(16, (300, 128), 1.0), synth.normal_bf16(17, (4, 64, 128), 0.02),
                          np.array([100, 40, 250, 999], np.int32)),
}


@pytest.mark.parametrize("case", list(GM_CASES))
def test_grouped_m_fp8(case):
    x, w, offs = GM_CASES[case]()
    gm_case(x, w, offs, name=case)


@pytest.mark.parametrize("codecs", [(1, 1), (0, 1), (1, 0)])
def test_grouped_m_fnuz(codecs):
    x, w, offs = GM_CASES["ragged"]()
    gm_case(x, w, offs, *codecs, name="fnuz")


def test_grouped_m_f32_out():
    x, w, offs = GM_CASES["cfg1"]()
    gm_case(x, w, offs, out_dtype=1, name="f32out")


def test_grouped_m_zero_rows():
    note("GROUPED_M M=0")
    out = fm.grouped_mm_scaled(fm.GROUPED_M, torch.empty(0, 64, dtype=torch.uint8, device=DEV), 0,
                               torch.empty(0, device=DEV), torch.zeros(2, 16, 64, dtype=torch.uint8, device=DEV), 0,
                               torch.ones(2, 16, device=DEV), fm.SCALE_F32, i32_dev([0, 0]), 2, 0, 16, 64)
    torch.cuda.synchronize()
    assert out.shape == (0, 16)


# ------------------------------------------------------------------ GROUPED_K

def gk_case(dy_bits, x_bits, offs, codec_a=0, codec_b=0, out_dtype=0, name=""):
    M, N = dy_bits.shape
    K = x_bits.shape[1]
    E = len(offs)
    note(f"GROUPED_K {name} M={M} N={N} K={K} E={E} codecs={codec_a},{codec_b}")
    qa, sa = fm.quantize_colwise(bf16_dev(dy_bits), i32_dev(offs), codec_a)
    qb, sb = fm.quantize_colwise(bf16_dev(x_bits), i32_dev(offs), codec_b)
    fmt = {0: fm.OPD_E4M3FN, 1: fm.OPD_E4M3FNUZ}
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, fmt[codec_a], sa, qb, fmt[codec_b], sb, fm.SCALE_F32,
                               i32_dev(offs), E, M, N, K, out_dtype=out_dtype)
    _, got = _out_host(out)
    qa_h, sa_h, qb_h, sb_h = host(qa), host(sa), host(qb), host(sb)
    ref = oracle.mm_grouped_k(qa_h, sa_h, qb_h, sb_h, offs, codec_a, codec_b)
    lo, hi = oracle.group_bounds(offs, M)
    A = np.zeros((N, M))
    B = np.zeros((K, M))
    for e in range(E):
        A[:, lo[e]:hi[e]] = oracle.decode(qa_h[:, lo[e]:hi[e]], codec_a) / sa_h[e][:, None].astype(np.float64)
        B[:, lo[e]:hi[e]] = oracle.decode(qb_h[:, lo[e]:hi[e]], codec_b) / sb_h[e][:, None].astype(np.float64)
    acc = oracle.ACC_FP8_MFMA if codec_a == 0 and codec_b == 0 else oracle.ACC_FP32
    contract, tight = oracle.error_bounds_k(A, B, offs, acc)
    check(got, ref, contract, tight, f"GROUPED_K {name}")
    for e in range(E):
        if hi[e] == lo[e]:
            assert not np.any(got[e]), "empty group must be exact zeros"


GK_CASES = {
    "cfg1": lambda: (synth.normal_bf16(21, (512, 512), 1e-3), synth.make_x(synth.WORKLOADS[1]),
                     synth.WORKLOADS[1].offs),
    "ragged": lambda: (synth.normal_bf16(22, (1200, 320), 1e-3), synth.normal_bf16(23, (1200, 272), 1.0, 0.01, 50.0),
                       synth.offsets_from_counts(synth.random_counts(24, 1150, 7))),
    "dense": lambda: (synth.normal_bf16(25, (1024, 256), 1e-3), synth.normal_bf16(26, (1024, 512), 1.0),
                      np.array([1024], np.int32)),
}


@pytest.mark.parametrize("case", list(GK_CASES))
def test_grouped_k_fp8(case):
    dy, x, offs = GK_CASES[case]()
    gk_case(dy, x, offs, name=case)


def test_grouped_k_fnuz():
    dy, x, offs = GK_CASES["ragged"]()
    gk_case(dy, x, offs, 1, 1, name="fnuz")


def test_grouped_k_bf16_plus_gw():
    dy, x, offs = GK_CASES["ragged"]()
    M, N = dy.shape
    K = x.shape[1]
    E = len(offs)
    note(f"GROUPED_K bf16 M={M} N={N} K={K}")
    out = fm.grouped_mm_scaled(fm.GROUPED_K, bf16_dev(dy), fm.OPD_BF16, None, bf16_dev(x), fm.OPD_BF16, None,
                               fm.SCALE_NONE, i32_dev(offs), E, M, N, K)
    _, got = _out_host(out)
    ref = oracle.mm_grouped_k_bf16(dy, x, offs)
    lo, hi = oracle.group_bounds(offs, M)
    A = bf16_bits_to_f64(np.ascontiguousarray(dy.T))
    B = bf16_bits_to_f64(np.ascontiguousarray(x.T))
    contract, tight = oracle.error_bounds_k(A, B, offs)
    check(got, ref, contract, tight, "GROUPED_K bf16")


def gw_case(dy, x, offs, out_dtype=0, name=""):
    """bf16 "+GW" GROUPED_K on token-major operands against the fp64 oracle; every
    output element (exact zeros for empty groups) must be written."""
    M, N = dy.shape
    K, E = x.shape[1], len(offs)
    note(f"GROUPED_K bf16 {name} M={M} N={N} K={K} E={E} out={out_dtype}")
    odt = torch.bfloat16 if out_dtype == 0 else torch.float32
    out = torch.empty((E, N, K), dtype=odt, device=DEV)
    if out_dtype == 0:
        out.view(torch.int16).fill_(SENT_BF16)
    else:
        out.fill_(float("nan"))
    fm.grouped_mm_scaled(fm.GROUPED_K, bf16_dev(dy), fm.OPD_BF16, None, bf16_dev(x), fm.OPD_BF16, None,
                         fm.SCALE_NONE, i32_dev(offs), E, M, N, K, out=out, out_dtype=out_dtype)
    _, got = _out_host(out)
    ref = oracle.mm_grouped_k_bf16(dy, x, offs)
    A = bf16_bits_to_f64(np.ascontiguousarray(dy.T))
    B = bf16_bits_to_f64(np.ascontiguousarray(x.T))
    contract, tight = oracle.error_bounds_k(A, B, offs)
    check(got, ref, contract, tight, f"GROUPED_K bf16 {name}")


GW_CASES = {
    # one group whose token count leaves a partial last stage; tiles past N and K
    "tail": lambda: (synth.normal_bf16(40, (1000, 264), 1e-3), synth.normal_bf16(41, (1000, 520), 1.0, 0.01, 30.0),
                     np.array([1000], np.int32)),
    # tiny, single-token and empty groups
    "small": lambda: (synth.normal_bf16(42, (480, 136), 1e-3), synth.normal_bf16(43, (480, 72), 1.0),
                      np.cumsum([0, 1, 7, 16, 0, 63, 64, 65, 1, 0, 150, 113]).astype(np.int32)),
    # decreasing and out-of-range offsets
    "malformed": lambda: (synth.normal_bf16(44, (600, 64), 1e-3), synth.normal_bf16(45, (600, 96), 1.0),
                          np.array([100, 50, 650, 900, -3], np.int32)),
    # more groups than the kernel's group table (the scan path)
    "many_groups": lambda: (synth.normal_bf16(46, (2048, 64), 1e-3), synth.normal_bf16(47, (2048, 64), 1.0),
                            synth.offsets_from_counts(synth.random_counts(48, 2048, 300))),
}


@pytest.mark.parametrize("case", list(GW_CASES))
def test_grouped_k_bf16_gw(case):
    dy, x, offs = GW_CASES[case]()
    gw_case(dy, x, offs, name=case)


def test_grouped_k_bf16_gw_f32_out():
    dy, x, offs = GW_CASES["tail"]()
    gw_case(dy, x, offs, out_dtype=1, name="tail f32")


def test_grouped_k_bf16_gw_full_size_sampled():
    # the Llama3-8B linear's weight gradient kept in BF16: dY [8192, 14336], X [8192, 4096]
    w = synth.WORKLOADS[2]
    dy, x = synth.make_dy(w), synth.make_x(w)
    M, N = dy.shape
    K = x.shape[1]
    offs = np.array([M], np.int32)
    note(f"GROUPED_K bf16 full M={M} N={N} K={K}")
    out = fm.grouped_mm_scaled(fm.GROUPED_K, bf16_dev(dy), fm.OPD_BF16, None, bf16_dev(x), fm.OPD_BF16, None,
                               fm.SCALE_NONE, i32_dev(offs), 1, M, N, K)
    rows = _rows(N, 10, 81)
    got = bf16_bits_to_f64(host(out[:, torch.from_numpy(rows).to(DEV)]))
    del out
    dyr = np.ascontiguousarray(dy[:, rows])
    ref = oracle.mm_grouped_k_bf16(dyr, x, offs)
    A = bf16_bits_to_f64(np.ascontiguousarray(dyr.T))
    B = bf16_bits_to_f64(np.ascontiguousarray(x.T))
    contract, tight = oracle.error_bounds_k(A, B, offs)
    check(got, ref, contract, tight, "GROUPED_K bf16 full")


# ------------------------------------------------------------------ MXFP8

@pytest.mark.parametrize("rule", [0, 1])
def test_grouped_m_mx(rule):
    x = synth.normal_bf16(31, (900, 512), 1.0, 0.01, 30.0)
    w = synth.normal_bf16(32, (5, 288, 512), 0.02)
    offs = synth.offsets_from_counts(synth.random_counts(33, 880, 5))
    M, K = x.shape
    E, N, _ = w.shape
    note(f"GROUPED_M MX rule={rule}")
    qa, xa, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule)
    qb, xb, _ = fm.quantize_mx(bf16_dev(w.reshape(E * N, K)), axis=1, rule=rule)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(SENT_BF16)
    fm.grouped_mm_scaled(fm.GROUPED_M, qa, fm.OPD_E4M3FN, xa, qb, fm.OPD_E4M3FN, xb, fm.SCALE_E8M0, i32_dev(offs),
                         E, M, N, K, out=out)
    raw, got = _out_host(out)
    qa_h, xa_h = host(qa), host(xa)
    qb_h, xb_h = host(qb).reshape(E, N, K), host(xb).reshape(E, N, K // 32)
    ref = oracle.mm_grouped_m_mx(qa_h, xa_h, qb_h, xb_h, offs)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_m(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, "GROUPED_M MX")
    assert np.all(raw[np.isnan(ref[:, 0])] == SENT_BF16)


@pytest.mark.parametrize("rule", [0, 1])
def test_grouped_k_mx(rule):
    dy = synth.normal_bf16(34, (1000, 320), 1e-3)
    x = synth.normal_bf16(35, (1000, 288), 1.0, 0.01, 30.0)
    offs = synth.offsets_from_counts(synth.random_counts(36, 990, 6))
    M, N = dy.shape
    K = x.shape[1]
    E = len(offs)
    Mp = fm.quantize_mx_rows_bound(M, E)
    note(f"GROUPED_K MX rule={rule} Mp={Mp}")
    qa, xa, op = fm.quantize_mx(bf16_dev(dy), axis=0, offs=i32_dev(offs), rule=rule, rows_pad=Mp)
    qb, xb, _ = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=rule, rows_pad=Mp)
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, fm.OPD_E4M3FN, xa, qb, fm.OPD_E4M3FN, xb, fm.SCALE_E8M0, op, E,
                               Mp, N, K)
    _, got = _out_host(out)
    qa_h, xa_h, qb_h, xb_h, op_h = host(qa), host(xa), host(qb), host(xb), host(op)
    ref = oracle.mm_grouped_k_mx(qa_h, xa_h, qb_h, xb_h, op_h)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_k(A, B, op_h, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, "GROUPED_K MX")


# ------------------------------------------------------------------ full size, sampled rows

def _rows(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))


def _check_rows_by_expert(got, rows, offs, M, per_expert_ref, what):
    """Compare sampled output rows, one oracle call per expert that owns sampled rows."""
    lo, hi = oracle.group_bounds(offs, M)
    grp = np.searchsorted(hi, rows, side="right")
    for e in np.unique(grp):
        sel = rows[grp == e]
        ref, contract, tight = per_expert_ref(e, sel)
        check(got[sel], ref, contract, tight, f"{what} expert {e}")


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_grouped_m_full_size_sampled(cfg):
    w = synth.WORKLOADS[cfg]
    x = synth.make_x(w)
    wt = synth.make_w1(w)
    offs = w.offs
    M, K = x.shape
    E, N, _ = wt.shape
    note(f"GROUPED_M full cfg={cfg} M={M} N={N} K={K}")
    qa, sa = fm.quantize_rowwise(bf16_dev(x), 0)
    qb, sb = fm.quantize_rowwise(bf16_dev(wt.reshape(E * N, K)), 0)
    del wt
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, sa, qb, 0, sb, fm.SCALE_F32, i32_dev(offs), E, M, N, K)
    _, got = _out_host(out)
    qa_h, sa_h = host(qa), host(sa)
    qb_h, sb_h = host(qb).reshape(E, N, K), host(sb).reshape(E, N)

    def ref_for(e, sel):
        one = np.array([len(sel)], np.int32)
        ref = oracle.mm_grouped_m(qa_h[sel], sa_h[sel], qb_h[e:e + 1], sb_h[e:e + 1], one, 0, 0)
        A = oracle.decode(qa_h[sel], 0) / sa_h[sel][:, None].astype(np.float64)
        B = oracle.decode(qb_h[e:e + 1], 0) / sb_h[e][None, :, None].astype(np.float64)
        return (ref,) + oracle.error_bounds_m(A, B, one, oracle.ACC_FP8_MFMA)

    _check_rows_by_expert(got, _rows(M, 24, cfg), offs, M, ref_for, f"cfg{cfg}")


def test_grouped_k_full_size_sampled():
    w = synth.WORKLOADS[2]
    dy = synth.make_dy(w)             # [8192, 14336]
    x = synth.make_x(w)               # [8192, 4096]
    offs = np.array([8192], np.int32)
    M, N = dy.shape
    K = x.shape[1]
    note("GROUPED_K full cfg=2")
    qa, sa = fm.quantize_colwise(bf16_dev(dy), i32_dev(offs), 0)
    qb, sb = fm.quantize_colwise(bf16_dev(x), i32_dev(offs), 0)
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, 0, sa, qb, 0, sb, fm.SCALE_F32, i32_dev(offs), 1, M, N, K)
    rows = _rows(N, 12, 7)
    _, got = _out_host(out)
    qa_h, sa_h = host(qa)[rows], host(sa)[:, rows]
    qb_h, sb_h = host(qb), host(sb)
    ref = oracle.mm_grouped_k(qa_h, sa_h, qb_h, sb_h, offs, 0, 0)
    A = oracle.decode(qa_h, 0) / sa_h[0][:, None]
    B = oracle.decode(qb_h, 0) / sb_h[0][:, None]
    contract, tight = oracle.error_bounds_k(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got[:, rows], ref, contract, tight, "cfg2 wgrad")


@pytest.mark.parametrize("layout", ["rows", "k4"])
def test_grouped_m_mx_full_size_sampled(layout):
    w = synth.WORKLOADS[5]
    x = synth.make_x(w)               # [16384, 5120]
    # a 2048-row slice of every expert's W1 keeps the host-side check small
    E, N, K = 16, 2048, 5120
    wt = np.stack([synth.normal_bf16(1000 * synth.tensor_seed(5, synth.T_W1) + e, (N, K), 0.02) for e in range(E)])
    offs = w.offs
    M = x.shape[0]
    note(f"GROUPED_M MX full cfg=5 M={M} N={N} K={K} scales={layout}")
    qa, xa, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0)
    qb, xb, _ = fm.quantize_mx(bf16_dev(wt.reshape(E * N, K)), axis=1, rule=0)
    if layout == "k4":
        _, ya, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0, layout=fm.MX_LAYOUT_K4)
        _, yb, _ = fm.quantize_mx(bf16_dev(wt.reshape(E * N, K)), axis=1, rule=0, layout=fm.MX_LAYOUT_K4)
        out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, ya, qb, 0, yb, fm.SCALE_E8M0_K4, i32_dev(offs), E, M, N, K)
    else:
        out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, xa, qb, 0, xb, fm.SCALE_E8M0, i32_dev(offs), E, M, N, K)
    _, got = _out_host(out)
    qa_h, xa_h = host(qa), host(xa)
    qb_h, xb_h = host(qb).reshape(E, N, K), host(xb).reshape(E, N, K // 32)

    def ref_for(e, sel):
        one = np.array([len(sel)], np.int32)
        ref = oracle.mm_grouped_m_mx(qa_h[sel], xa_h[sel], qb_h[e:e + 1], xb_h[e:e + 1], one)
        A = oracle.decode(qa_h[sel], 0) * np.repeat(oracle.e8m0_decode(xa_h[sel]), 32, axis=-1)
        B = oracle.decode(qb_h[e:e + 1], 0) * np.repeat(oracle.e8m0_decode(xb_h[e:e + 1]), 32, axis=-1)
        return (ref,) + oracle.error_bounds_m(A, B, one, oracle.ACC_FP8_MFMA)

    _check_rows_by_expert(got, _rows(M, 16, 55), offs, M, ref_for, "cfg5 MX")


# ------------------------------------------------------------------ pipeline edge cases
# The FP8/MX kernel streams 128-byte contraction stages through a 2-slot (256-row
# tiles) or 3-slot (128-row tiles, small groups) ring, processes the last stage
# first, and reloads past the end: cover 1..5 stages, lengths that are not a
# multiple of 128, both tile shapes, and the staged fp32 epilogue.

@pytest.mark.parametrize("K", [48, 144, 400, 640])
@pytest.mark.parametrize("tiles", ["wide", "small"])
def test_grouped_m_contraction_lengths(K, tiles):
    if tiles == "wide":     # one group: 256-row tiles
        x = synth.normal_bf16(41, (600, K), 1.0)
        w = synth.normal_bf16(42, (1, 272, K), 0.02)
        offs = np.array([600], np.int32)
    else:                   # small groups: 128-row tiles
        x = synth.normal_bf16(43, (700, K), 1.0, 0.01, 50.0)
        w = synth.normal_bf16(44, (8, 272, K), 0.02)
        offs = synth.offsets_from_counts(synth.random_counts(45, 690, 8))
    gm_case(x, w, offs, name=f"K{K}-{tiles}")


def test_grouped_m_f32_out_wide_tiles():
    x, w, offs = GM_CASES["dense"]()
    w = np.concatenate([w, w[:, :212]], axis=1)       # N = 512: 16-byte aligned fp32 rows
    gm_case(x, w, offs, out_dtype=1, name="f32out-wide")


def test_grouped_k_small_and_empty_groups():
    counts = np.array([1, 0, 2, 17, 128, 0, 255, 300, 3], np.int64)
    M = (int(counts.sum()) + 20 + 15) // 16 * 16       # a multiple of 16; rows past the last group are ignored
    dy = synth.normal_bf16(46, (M, 264), 1e-3)
    x = synth.normal_bf16(47, (M, 200), 1.0, 0.01, 30.0)
    gk_case(dy, x, synth.offsets_from_counts(counts), name="small-groups")



def test_grouped_k_skewed_groups():
    """One group far above the mean (the kernel then runs the groups in decreasing size, every other
    round of the grid backwards), equal sizes (ties keep index order) and empty groups; more tiles
    than one round of the grid."""
    counts = np.array([64, 3000, 0, 64, 130, 1, 700, 64, 0, 2, 300, 33], np.int64)
    assert counts.max() * (counts > 0).sum() > 2 * counts.sum()
    M = (int(counts.sum()) + 15) // 16 * 16        # a multiple of 16; rows past the last group are ignored
    dy = synth.normal_bf16(48, (M, 2104), 1e-3)      # 12 x 9 x 6 tiles of 256: three rounds of 256 CUs
    x = synth.normal_bf16(49, (M, 1400), 1.0, 0.01, 30.0)
    gk_case(dy, x, synth.offsets_from_counts(counts), name="skewed")

def test_grouped_k_f32_out():
    dy, x, offs = GK_CASES["ragged"]()
    gk_case(dy, x, offs, out_dtype=1, name="f32out")


def _gk_mx(dy, x, offs, rule, what):
    M, N = dy.shape
    K = x.shape[1]
    E = len(offs)
    Mp = fm.quantize_mx_rows_bound(M, E)
    note(f"GROUPED_K MX {what} rule={rule} Mp={Mp}")
    qa, xa, op = fm.quantize_mx(bf16_dev(dy), axis=0, offs=i32_dev(offs), rule=rule, rows_pad=Mp)
    qb, xb, _ = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=rule, rows_pad=Mp)
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, fm.OPD_E4M3FN, xa, qb, fm.OPD_E4M3FN, xb, fm.SCALE_E8M0, op, E,
                               Mp, N, K)
    _, got = _out_host(out)
    qa_h, xa_h, qb_h, xb_h, op_h = host(qa), host(xa), host(qb), host(xb), host(op)
    ref = oracle.mm_grouped_k_mx(qa_h, xa_h, qb_h, xb_h, op_h)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_k(A, B, op_h, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, f"GROUPED_K MX {what}")
    return Mp


@pytest.mark.parametrize("rule", [0, 1])
def test_grouped_k_mx_aligned_rows(rule):
    # rows_pad = round_up(960 + 31 * 2, 32) = 1024, a multiple of 128: the 128-byte-stage kernel
    dy = synth.normal_bf16(48, (960, 320), 1e-3)
    x = synth.normal_bf16(49, (960, 288), 1.0, 0.01, 30.0)
    offs = synth.offsets_from_counts(np.array([517, 443]))
    assert _gk_mx(dy, x, offs, rule, "aligned") % 128 == 0


def test_grouped_k_mx_aligned_many_groups():
    counts = np.array([40, 0, 300, 1, 127, 129, 200, 103], np.int64)   # sum 900, bound = 1152
    M = int(counts.sum())
    dy = synth.normal_bf16(50, (M, 256), 1e-3)
    x = synth.normal_bf16(51, (M, 320), 1.0)
    assert _gk_mx(dy, x, synth.offsets_from_counts(counts), 0, "groups") % 128 == 0


def test_grouped_m_mx_unaligned_k():
    # K = 288 is not a multiple of 128: e8m0 rows take the byte-wise stage kernel
    x = synth.normal_bf16(52, (500, 288), 1.0, 0.01, 30.0)
    w = synth.normal_bf16(53, (3, 200, 288), 0.02)
    offs = synth.offsets_from_counts(synth.random_counts(54, 480, 3))
    M, K = x.shape
    E, N, _ = w.shape
    note("GROUPED_M MX K=288")
    qa, xa, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0)
    qb, xb, _ = fm.quantize_mx(bf16_dev(w.reshape(E * N, K)), axis=1, rule=0)
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, xa, qb, 0, xb, fm.SCALE_E8M0, i32_dev(offs), E, M, N, K)
    _, got = _out_host(out)
    qa_h, xa_h = host(qa), host(xa)
    qb_h, xb_h = host(qb).reshape(E, N, K), host(xb).reshape(E, N, K // 32)
    ref = oracle.mm_grouped_m_mx(qa_h, xa_h, qb_h, xb_h, offs)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_m(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, "GROUPED_M MX K=288")


# ------------------------------------------------------------------ e8m0 scales in the K4 layout
# The same products with the scales in the layout whose stage words are contiguous per tile:
# the pipeline reads them with other addresses but the same MFMA sequence, so where the
# row-major scales take the pipeline too the outputs are bit-identical; elsewhere (contraction
# lengths that are not a multiple of 128) they are checked against the oracle.

@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("K", [512, 288])
def test_grouped_m_mx_k4(rule, K):
    x = synth.normal_bf16(61, (900, K), 1.0, 0.01, 30.0)
    w = synth.normal_bf16(62, (5, 288, K), 0.02)
    offs = synth.offsets_from_counts(synth.random_counts(63, 880, 5))
    M = x.shape[0]
    E, N, _ = w.shape
    note(f"GROUPED_M MX K4 rule={rule} K={K}")
    qa, xa, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule)
    qb, xb, _ = fm.quantize_mx(bf16_dev(w.reshape(E * N, K)), axis=1, rule=rule)
    _, ya, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule, layout=fm.MX_LAYOUT_K4)
    _, yb, _ = fm.quantize_mx(bf16_dev(w.reshape(E * N, K)), axis=1, rule=rule, layout=fm.MX_LAYOUT_K4)
    xa_h, xb_h = host(xa), host(xb)
    assert np.array_equal(host(ya), e8m0_rows_to_k4(xa_h)) and np.array_equal(host(yb), e8m0_rows_to_k4(xb_h))
    ref_rows = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, xa, qb, 0, xb, fm.SCALE_E8M0, i32_dev(offs), E, M, N, K)
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, ya, qb, 0, yb, fm.SCALE_E8M0_K4, i32_dev(offs), E, M, N, K)
    raw, got = _out_host(out)
    if K % 128 == 0:       # rows outside every group are left untouched: compare the routed ones
        used = int(offs[-1])
        assert np.array_equal(raw[:used], _out_host(ref_rows)[0][:used]), "K4 and row-major scales differ"
    qa_h = host(qa)
    qb_h, xb3 = host(qb).reshape(E, N, K), xb_h.reshape(E, N, K // 32)
    ref = oracle.mm_grouped_m_mx(qa_h, xa_h, qb_h, xb3, offs)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb3), 32, axis=-1)
    contract, tight = oracle.error_bounds_m(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, f"GROUPED_M MX K4 K={K}")


# Groups averaging at least 512 rows take 256-row tiles.  These sizes put a group's last tile at every
# boundary: remainders (mod 256) of 0, 1, 64, 65, 127, 128, 129, 255, groups under one tile, an empty
# group, one row.
SPLIT_COUNTS = np.array([256, 257, 383, 385, 511, 512, 513, 640, 767, 900, 0, 1, 100, 1023, 2000, 320, 321],
                        np.int64)


@pytest.mark.parametrize("N", [320, 200])           # two column tiles, one
def test_grouped_m_last_tile_sizes(N):
    offs = synth.offsets_from_counts(SPLIT_COUNTS)
    M = int(offs[-1]) + 37                          # rows past the last group keep their sentinel
    x = synth.normal_bf16(81, (M, 512), 1.0, 0.01, 50.0)
    w = synth.normal_bf16(82, (len(SPLIT_COUNTS), N, 512), 0.02)
    assert M // len(SPLIT_COUNTS) >= 512
    gm_case(x, w, offs, name=f"tile boundaries N={N}")



def test_grouped_m_last_tile_sizes_malformed_offsets():
    """A decreasing offset (an empty group) and one past M (clamped), with 256-row tiles."""
    x = synth.normal_bf16(85, (3000, 384), 1.0)
    w = synth.normal_bf16(86, (4, 300, 384), 0.02)
    gm_case(x, w, np.array([1000, 600, 2300, 99999], np.int32), name="tile boundaries, malformed offsets")

@pytest.mark.parametrize("rule", [0, 1])
def test_grouped_m_mx_k4_last_tile_sizes(rule):
    offs = synth.offsets_from_counts(SPLIT_COUNTS)
    M, K = int(offs[-1]), 640
    E, N = len(SPLIT_COUNTS), 288
    x = synth.normal_bf16(83, (M, K), 1.0, 0.01, 30.0)
    w = synth.normal_bf16(84, (E, N, K), 0.02)
    note(f"GROUPED_M MX K4 last tile sizes rule={rule}")
    qa, xa, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule)
    qb, xb, _ = fm.quantize_mx(bf16_dev(w.reshape(E * N, K)), axis=1, rule=rule)
    _, ya, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule, layout=fm.MX_LAYOUT_K4)
    _, yb, _ = fm.quantize_mx(bf16_dev(w.reshape(E * N, K)), axis=1, rule=rule, layout=fm.MX_LAYOUT_K4)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    out.view(torch.int16).fill_(SENT_BF16)
    fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, ya, qb, 0, yb, fm.SCALE_E8M0_K4, i32_dev(offs), E, M, N, K, out=out)
    raw, got = _out_host(out)
    qa_h, xa_h = host(qa), host(xa)
    qb_h, xb3 = host(qb).reshape(E, N, K), host(xb).reshape(E, N, K // 32)
    ref = oracle.mm_grouped_m_mx(qa_h, xa_h, qb_h, xb3, offs)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb3), 32, axis=-1)
    contract, tight = oracle.error_bounds_m(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, "GROUPED_M MX K4 last tile sizes")


@pytest.mark.parametrize("case", ["unaligned", "aligned", "small-groups"])
def test_grouped_k_mx_k4(case):
    if case == "unaligned":       # rows_pad = 1216: the last stage holds one real 32-block
        counts = synth.random_counts(64, 990, 6)
    elif case == "aligned":       # rows_pad = 1024
        counts = np.array([517, 443])
    else:
        counts = np.array([40, 0, 300, 1, 127, 129, 200, 103], np.int64)
    offs = synth.offsets_from_counts(counts)
    M = int(np.sum(counts)) + 10
    dy = synth.normal_bf16(65, (M, 320), 1e-3)
    x = synth.normal_bf16(66, (M, 288), 1.0, 0.01, 30.0)
    N, K, E = dy.shape[1], x.shape[1], len(offs)
    Mp = fm.quantize_mx_rows_bound(M, E)
    note(f"GROUPED_K MX K4 {case} Mp={Mp}")
    qa, xa, op = fm.quantize_mx(bf16_dev(dy), axis=0, offs=i32_dev(offs), rule=0, rows_pad=Mp)
    qb, xb, _ = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=0, rows_pad=Mp)
    _, ya, _ = fm.quantize_mx(bf16_dev(dy), axis=0, offs=i32_dev(offs), rule=0, rows_pad=Mp, layout=fm.MX_LAYOUT_K4)
    _, yb, _ = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=0, rows_pad=Mp, layout=fm.MX_LAYOUT_K4)
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, 0, ya, qb, 0, yb, fm.SCALE_E8M0_K4, op, E, Mp, N, K)
    raw, got = _out_host(out)
    if Mp % 128 == 0:
        ref_rows = fm.grouped_mm_scaled(fm.GROUPED_K, qa, 0, xa, qb, 0, xb, fm.SCALE_E8M0, op, E, Mp, N, K)
        assert np.array_equal(raw, _out_host(ref_rows)[0]), "K4 and row-major scales differ"
    qa_h, xa_h, qb_h, xb_h, op_h = host(qa), host(xa), host(qb), host(xb), host(op)
    ref = oracle.mm_grouped_k_mx(qa_h, xa_h, qb_h, xb_h, op_h)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_k(A, B, op_h, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, f"GROUPED_K MX K4 {case}")


def test_grouped_m_mx_k4_batched_weights():
    # dgrad-style B operand: weights quantized along their rows (batched axis 0), scale rows E * N
    x = synth.normal_bf16(67, (700, 384), 1.0, 0.01, 30.0)
    w = synth.normal_bf16(68, (4, 384, 160), 0.02)             # [E][K][N] -> B phys [E][N][K]
    offs = synth.offsets_from_counts(synth.random_counts(69, 690, 4))
    M, K = x.shape
    E, _, N = w.shape
    note("GROUPED_M MX K4 batched weights")
    qa, ya, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0, layout=fm.MX_LAYOUT_K4)
    qb, yb, _ = fm.quantize_mx(bf16_dev(w), axis=0, rule=0, layout=fm.MX_LAYOUT_K4)
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, ya, qb, 0, yb, fm.SCALE_E8M0_K4, i32_dev(offs), E, M, N, K)
    _, got = _out_host(out)
    _, xa, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0)
    _, xb, _ = fm.quantize_mx(bf16_dev(w), axis=0, rule=0)
    qa_h, xa_h = host(qa), host(xa)
    qb_h, xb_h = host(qb), host(xb)                               # [E][N][K], [E][N][K/32]
    ref = oracle.mm_grouped_m_mx(qa_h, xa_h, qb_h, xb_h, offs)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_m(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, "GROUPED_M MX K4 batched weights")


# ------------------------------------------------------------------ dense wgrad split into rounds
# One group, fp32 scales: with 256 CUs, N = 33 x 256 and K = 16 x 256 make 528 tiles of 256x256,
# two full rounds and a 16-tile remainder, so the output rows split into a 256-row-tile launch
# (N = 8192) and a 128-row-tile tail (N = 256). The full-size Llama3-8B weight gradient takes
# the same path (896 tiles). Checked element by element against the oracle.

@pytest.mark.parametrize("out_dtype", [0, 1])
def test_grouped_k_dense_round_split(out_dtype):
    M, N, K = 256, 33 * 256, 16 * 256
    dy = synth.normal_bf16(71, (M, N), 1e-3)
    x = synth.normal_bf16(72, (M, K), 1.0, 0.01, 30.0)
    gk_case(dy, x, np.array([M], np.int32), out_dtype=out_dtype, name=f"round-split out={out_dtype}")


# ------------------------------------------------------------------ MoE weight gradients at full size, sampled
# The launches the bench times for the W1 weight gradient of the MoE workloads: every expert's
# [N, K] output, checked on sampled output rows n (all experts, all k) against the oracle.

def _dequant_groups(q_t, s, lo, hi, codec=0):
    out = np.zeros(q_t.shape)
    for e in range(len(lo)):
        if hi[e] > lo[e]:
            out[:, lo[e]:hi[e]] = oracle.decode(q_t[:, lo[e]:hi[e]], codec) / s[e][:, None].astype(np.float64)
    return out


@pytest.mark.parametrize("cfg", [3, 4])
def test_grouped_k_moe_full_size_sampled(cfg):
    w = synth.WORKLOADS[cfg]
    dh = synth.make_dh1(w)            # [M, 2F]
    x = synth.make_x(w)               # [M, H]
    offs = w.offs
    M, N = dh.shape
    K, E = x.shape[1], w.E
    note(f"GROUPED_K full cfg={cfg} M={M} N={N} K={K} E={E}")
    o = i32_dev(offs)
    qa, sa = fm.quantize_colwise(bf16_dev(dh), o, 0)
    qb, sb = fm.quantize_colwise(bf16_dev(x), o, 0)
    del dh, x
    ld = qa.shape[1]
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, 0, sa, qb, 0, sb, fm.SCALE_F32, o, E, ld, N, K)
    rows = _rows(N, 8, 70 + cfg)
    got = bf16_bits_to_f64(host(out[:, torch.from_numpy(rows).to(DEV)]))
    del out
    qa_h, sa_h = host(qa)[rows], host(sa)[:, rows]
    qb_h, sb_h = host(qb), host(sb)
    ref = oracle.mm_grouped_k(qa_h, sa_h, qb_h, sb_h, offs, 0, 0)
    lo, hi = oracle.group_bounds(offs, ld)
    A, B = _dequant_groups(qa_h, sa_h, lo, hi), _dequant_groups(qb_h, sb_h, lo, hi)
    contract, tight = oracle.error_bounds_k(A, B, offs, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, f"cfg{cfg} wgrad W1")


def test_grouped_k_mx_k4_full_size_sampled():
    w = synth.WORKLOADS[5]
    dh = synth.make_dh1(w)            # [16384, 16384]
    x = synth.make_x(w)               # [16384, 5120]
    offs = w.offs
    M, N = dh.shape
    K, E = x.shape[1], w.E
    Mp = fm.quantize_mx_rows_bound(M, E)
    note(f"GROUPED_K MX K4 full cfg=5 Mp={Mp} N={N} K={K}")
    o = i32_dev(offs)
    qa, ya, op = fm.quantize_mx(bf16_dev(dh), axis=0, offs=o, rule=0, rows_pad=Mp, layout=fm.MX_LAYOUT_K4)
    qb, yb, _ = fm.quantize_mx(bf16_dev(x), axis=0, offs=o, rule=0, rows_pad=Mp, layout=fm.MX_LAYOUT_K4)
    out = fm.grouped_mm_scaled(fm.GROUPED_K, qa, 0, ya, qb, 0, yb, fm.SCALE_E8M0_K4, op, E, Mp, N, K)
    rows = _rows(N, 6, 77)
    got = bf16_bits_to_f64(host(out[:, torch.from_numpy(rows).to(DEV)]))
    del out
    # the row-major scales of the same tensors for the oracle (the K4 bytes are checked against them elsewhere)
    _, xa, _ = fm.quantize_mx(bf16_dev(dh), axis=0, offs=o, rule=0, rows_pad=Mp)
    _, xb, _ = fm.quantize_mx(bf16_dev(x), axis=0, offs=o, rule=0, rows_pad=Mp)
    del dh, x
    qa_h, xa_h, qb_h, xb_h, op_h = host(qa)[rows], host(xa)[rows], host(qb), host(xb), host(op)
    ref = oracle.mm_grouped_k_mx(qa_h, xa_h, qb_h, xb_h, op_h)
    A = oracle.decode(qa_h, 0) * np.repeat(oracle.e8m0_decode(xa_h), 32, axis=-1)
    B = oracle.decode(qb_h, 0) * np.repeat(oracle.e8m0_decode(xb_h), 32, axis=-1)
    contract, tight = oracle.error_bounds_k(A, B, op_h, oracle.ACC_FP8_MFMA)
    check(got, ref, contract, tight, "cfg5 MX wgrad W1 (K4)")


# ------------------------------------------------------------------ FP8 MFMA accumulation

def _code(v):
    return int(oracle.encode(np.float32([v]), 0)[0])


ACC_CASES = {      # name: (a_k, b_k) pairs of one 64-long contraction (one MFMA k step), the rest zero
    "1 + 2^-13": [(1, 1), (2.0 ** -6, 2.0 ** -7)],
    "1 + 2^-14": [(1, 1), (2.0 ** -7, 2.0 ** -7)],
    "1 + 2^-16": [(1, 1), (2.0 ** -8, 2.0 ** -8)],
    "64 ones": [(1, 1)] * 64,
    "1 + 63 * 2^-14": [(1, 1)] + [(2.0 ** -7, 2.0 ** -7)] * 63,
    "2^16 + 63 * 2^-7": [(256, 256)] + [(2.0 ** -3, 2.0 ** -4)] * 63,
    "cancel, large first": [(448, 448), (-448, 448)] + [(2.0 ** -9, 2.0 ** -9)] * 62,
    "cancel, large last": [(2.0 ** -9, 2.0 ** -9)] * 62 + [(448, 448), (-448, 448)],
}


def test_fp8_mfma_accumulation():
    """One FP8 MFMA k step (64 products, unit scales, fp32 output) on constructed codes whose exact
    sums need more bits than the instruction keeps.  Observed on gfx950: a product 2^-14 or further
    below the largest product of the same instruction can be dropped, where every fp32 summation
    order keeps it (1 + 2^-14 is an fp32 value); 2^-13 is kept.  The result is not an fp32 chain in
    any order, which is why the diagnostic bound of the FP8 paths allows 2^-10 * sum|a*b|; every
    case here stays inside it (and far inside the 1e-2 |a||b| contract)."""
    names = list(ACC_CASES)
    R = len(names)
    A = np.zeros((R, 64), np.uint8)
    B = np.zeros((R, 64), np.uint8)
    for r, nm in enumerate(names):
        for k, (x, y) in enumerate(ACC_CASES[nm]):
            A[r, k], B[r, k] = _code(x), _code(y)
    note("FP8 MFMA accumulation probe")
    qa, qb = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV).view(1, R, 64)
    out = fm.grouped_mm_scaled(fm.GROUPED_M, qa, 0, torch.ones(R, device=DEV), qb, 0, torch.ones(1, R, device=DEV),
                               fm.SCALE_F32, i32_dev([R]), 1, R, R, 64, out_dtype=fm.OUT_F32)
    got = host(out).astype(np.float64).diagonal()
    prod = oracle.decode(A, 0) * oracle.decode(B, 0)
    exact = prod.sum(axis=1)
    absdot = np.abs(prod).sum(axis=1)
    res = dict(zip(names, got))
    assert res["1 + 2^-13"] == 1 + 2.0 ** -13
    assert res["1 + 2^-14"] == 1.0          # dropped inside the instruction
    assert res["1 + 2^-16"] == 1.0
    assert np.float32(np.float32(1.0) + np.float32(2.0 ** -14)) == 1 + 2.0 ** -14   # fp32 would keep it
    assert res["64 ones"] == 64.0
    err = np.abs(got - exact)
    assert np.all(err <= 2.0 ** -10 * absdot), dict(zip(names, err / absdot))
    assert np.any(err > 0)
