"""GPU parity of the quantization kernels against the CPU oracle: bit-exact
codes and scales, through the C ABI (via the thin Python binding).

Small cases span several tiles and ragged tails; full-size cases use the
workloads' real shapes and compare sampled rows/columns (each row's or
column's result depends only on its own reduction set, so the oracle can
compute a sample independently).
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_quantized_moe_amd as fm
from mxfp8_quantized_moe_amd import synth
from gpu_helpers import (DEV, note, bf16_dev, i32_dev, filled_u8, filled_f32, host, assert_bytes_equal, e8m0_rows_to_k4,
                         assert_f32_bits_equal)

pytestmark = pytest.mark.gpu

CODECS = [fm.E4M3FN, fm.E4M3FNUZ]


def special_input(seed, shape, frac=0.02, factor=60.0, sigma=1.0):
    x = synth.normal_bf16(seed, shape, sigma, frac, factor)
    flat = x.reshape(-1)
    n = flat.size
    if n >= 8:
        flat[:4] = synth.f32_to_bf16_bits(np.float32([0.0, 2.0 ** -130, -(2.0 ** -133), -0.0]))
        flat[n // 2] = synth.f32_to_bf16_bits(np.float32([1e30]))[0]
    return x


# ------------------------------------------------------------------- codec

@pytest.mark.parametrize("codec", CODECS)
def test_device_encoder_matches_oracle(codec):
    fmax = oracle.FMAX[codec]
    mags = oracle.decode_table(codec)[: (0x7E if codec == 0 else 0x7F) + 1]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    probes = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                             mags.astype(np.float32)])
    fm_bits = int(np.float32(fmax).view(np.uint32))
    sweep = np.arange(0, fm_bits + 1, 4099, dtype=np.uint32).view(np.float32)
    y = np.concatenate([probes, sweep, np.float32([fmax, 0.0, -0.0, 1e-45, 2.0 ** -126])])
    y = np.concatenate([y, -y]).astype(np.float32)
    y = y[np.abs(y) <= fmax]
    note(f"encode_f32 codec={codec} n={y.size}")
    q = host(fm.encode_f32(torch.from_numpy(y).to(DEV), codec))
    assert_bytes_equal(q, oracle.encode(y, codec), f"encode codec {codec}")


# ------------------------------------------------------------------- rowwise

ROW_SHAPES = [(512, 256), (2048, 256), (7, 8), (33, 24), (5, 4104), (3, 16400), (100, 4096), (2, 131072),
              (257, 520), (0, 64), (3, 0)]


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_rowwise_parity(codec, shape):
    R, C = shape
    x = special_input(1000 + R + C, shape)
    if R > 4:
        x[R // 3] = 0                                      # an all-zero row
    note(f"rowwise codec={codec} shape={shape}")
    q, s = fm.quantize_rowwise(bf16_dev(x), codec)
    qr, sr = oracle.quantize_rowwise(x, codec)
    assert_bytes_equal(host(q), qr, "codes")
    assert_f32_bits_equal(host(s), sr, "scales")


@pytest.mark.parametrize("codec", CODECS)
def test_rowwise_strided_rows(codec):
    x = special_input(77, (129, 392))
    xd = bf16_dev(x)[:, :264]                             # row stride 392 > cols 264
    note(f"rowwise strided codec={codec}")
    q, s = fm.quantize_rowwise(xd, codec)
    qr, sr = oracle.quantize_rowwise(np.ascontiguousarray(x[:, :264]), codec)
    assert_bytes_equal(host(q), qr, "codes")
    assert_f32_bits_equal(host(s), sr, "scales")


def _lookup_edge_offsets():
    """Offsets at the boundary of the quantizers' group lookup: one wave handles at most 64 groups, a
    workgroup scan more.  64 and 65 ragged groups with empty ones, and 64 malformed offsets (a decrease,
    one past the rows, one negative)."""
    g64 = synth.offsets_from_counts(synth.random_counts(11, 1900, 64, 0.25))
    g65 = synth.offsets_from_counts(synth.random_counts(12, 1900, 65, 0.25))
    bad = g64.copy()
    bad[10] = bad[9] - 5
    bad[30] = 2100
    bad[40] = -1
    return {"groups64": (2000, 136, g64), "groups65": (2000, 136, g65), "groups64_malformed": (2000, 136, bad)}


LOOKUP_EDGE_CASES = _lookup_edge_offsets()


# ------------------------------------------------------------------- colwise

GROUP_CASES = {
    "cfg1": (512, 256, synth.offsets_from_counts(synth.routing_counts(1))),
    "ragged": (3000, 136, synth.offsets_from_counts(synth.random_counts(5, 2950, 9))),
    "tall": (2100, 64, np.array([2100], np.int32)),
    "malformed": (700, 72, np.array([100, 50, 650, 900, -3], np.int32)),
    "tiny": (37, 8, np.array([0, 5, 5, 36], np.int32)),
    # more than 128 chunks of 512 rows in one group: the two-pass kernels
    "very_tall": (70000, 64, np.array([70000], np.int32)),
    # more chunk slots than the single pass holds (2000 mostly empty groups): the two-pass kernels
    "many_groups": (1024, 1024, synth.offsets_from_counts(synth.random_counts(6, 1024, 2000, 0.5))),
    **LOOKUP_EDGE_CASES,
}


@pytest.fixture(params=[0, 128, 256, 512], ids=["chunks_auto", "chunks128", "chunks256", "chunks512"])
def chunk_rows(request):
    """The single-pass colwise chunk height: chosen per call, or forced to 128, 256 or 512 rows."""
    f = fm._lib.lib().fp8moe_set_colwise_chunk_rows
    prev = f(request.param)
    yield request.param
    f(prev)


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("case", list(GROUP_CASES))
def test_colwise_grouped_parity(codec, case, chunk_rows):
    M, C, offs = GROUP_CASES[case]
    x = special_input(2000 + M, (M, C))
    ld_q = (M + 16 + 15) // 16 * 16
    note(f"colwise grouped codec={codec} case={case} chunk rows={chunk_rows}")
    q_t = filled_u8((C, ld_q))
    sc = filled_f32((len(offs), C))
    fm.quantize_colwise(bf16_dev(x), i32_dev(offs), codec, q_t=q_t, scale=sc, ld_q=ld_q)
    sentinel = np.full((C, ld_q), 0xA5, np.uint8)
    qr, sr = oracle.quantize_colwise_grouped(x, offs, codec, q_init=sentinel, ld_q=ld_q)
    assert_bytes_equal(host(q_t), qr, "codes")
    assert_f32_bits_equal(host(sc), sr, "scales")


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("shape", [(3, 700, 72), (4, 100, 64), (2, 1, 8), (1, 1030, 136),
                                   (2, 4096, 72), (2, 4097, 72), (5, 1536, 200), (1, 65600, 16)])
def test_colwise_batched_parity(codec, shape, chunk_rows):
    x = special_input(3000 + sum(shape), shape)
    B, R, C = shape
    ld_q = (R + 15) // 16 * 16 + 16
    note(f"colwise batched codec={codec} shape={shape} chunk rows={chunk_rows}")
    q_t = filled_u8((B, C, ld_q))
    sc = filled_f32((B, C))
    fm.quantize_colwise(bf16_dev(x), None, codec, q_t=q_t, scale=sc, ld_q=ld_q)
    qr, sr = oracle.quantize_colwise_batched(x, codec)
    got = host(q_t)
    assert_bytes_equal(got[:, :, :R], qr, "codes")
    assert np.all(got[:, :, R:] == 0xA5), "wrote past the rows"
    assert_f32_bits_equal(host(sc), sr, "scales")


def test_colwise_batched_back_to_back_calls():
    # The batched single pass exchanges column maxima between chunks through
    # memory the library keeps across calls: a call must see none of the
    # previous call's maxima, here larger than its own by 2^10.
    shape = (3, 1800, 136)
    big = special_input(4100, shape, sigma=1024.0)
    small = special_input(4101, shape)
    for k, x in enumerate([big, small, big[:2, :900], small[:2, :900]]):
        note(f"colwise batched back-to-back call {k} shape={x.shape}")
        q_t, sc = fm.quantize_colwise(bf16_dev(x), None, fm.E4M3FN)
        qr, sr = oracle.quantize_colwise_batched(x, fm.E4M3FN)
        assert_bytes_equal(host(q_t)[:, :, :x.shape[1]], qr, f"codes call {k}")
        assert_f32_bits_equal(host(sc), sr, f"scales call {k}")


def test_colwise_deterministic_across_runs():
    M, C, offs = GROUP_CASES["ragged"]
    x = bf16_dev(special_input(99, (M, C)))
    o = i32_dev(offs)
    note("colwise determinism")
    a = [host(t) for t in fm.quantize_colwise(x, o, fm.E4M3FN)]
    b = [host(t) for t in fm.quantize_colwise(x, o, fm.E4M3FN)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


# ------------------------------------------------------------------- MXFP8

@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("shape", [(64, 96), (1000, 5120), (3, 32), (0, 64)])
def test_mx_lastdim_parity(rule, shape):
    x = special_input(4000 + shape[0], shape, 0.01, 30.0)
    note(f"mx lastdim rule={rule} shape={shape}")
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule)
    qr, sr = oracle.quantize_mx_lastdim(x, rule)
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), sr, "e8m0")


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("shape", [(2, 544, 72), (3, 32, 8), (1, 1024, 128)])
def test_mx_rows_batched_parity(rule, shape):
    x = special_input(5000 + sum(shape), shape, 0.01, 30.0)
    note(f"mx rows batched rule={rule} shape={shape}")
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=0, rule=rule)
    qr, sr = oracle.quantize_mx_rows_batched(x, rule)
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), sr, "e8m0")


@pytest.mark.parametrize("shape", [(64, 96), (1000, 5120), (3, 32), (0, 64), (40, 288)])
def test_mx_lastdim_k4_layout(shape):
    x = special_input(4100 + shape[0], shape, 0.01, 30.0)
    R, C = shape
    note(f"mx lastdim K4 shape={shape}")
    sc = filled_u8(fm.mx_k4_shape(R, C // 32))
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0, scale=sc, layout=fm.MX_LAYOUT_K4)
    qr, sr = oracle.quantize_mx_lastdim(x, 0)
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), e8m0_rows_to_k4(sr.reshape(R, C // 32)), "e8m0 K4")


@pytest.mark.parametrize("shape", [(2, 544, 72), (3, 32, 8), (1, 1024, 128)])
def test_mx_rows_batched_k4_layout(shape):
    x = special_input(5100 + sum(shape), shape, 0.01, 30.0)
    B, R, C = shape
    note(f"mx rows batched K4 shape={shape}")
    sc = filled_u8(fm.mx_k4_shape(B * C, R // 32))
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=0, rule=1, scale=sc, layout=fm.MX_LAYOUT_K4)
    qr, sr = oracle.quantize_mx_rows_batched(x, 1)
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), e8m0_rows_to_k4(sr.reshape(B * C, R // 32)), "e8m0 K4")


MX_GROUP_CASES = {
    "ragged": (1300, 136, synth.offsets_from_counts(synth.random_counts(8, 1290, 7))),
    "cfg1": (512, 256, synth.offsets_from_counts(synth.routing_counts(1))),
    "malformed": (300, 64, np.array([40, 20, 300, 500], np.int32)),
    "one_row": (1, 8, np.array([1], np.int32)),
    **LOOKUP_EDGE_CASES,
}


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("case", list(MX_GROUP_CASES))
def test_mx_rows_grouped_parity(rule, case):
    M, C, offs = MX_GROUP_CASES[case]
    x = special_input(6000 + M, (M, C), 0.01, 30.0)
    rows_pad = fm.quantize_mx_rows_bound(M, len(offs)) + 64      # extra tail beyond the bound
    note(f"mx rows grouped rule={rule} case={case} rows_pad={rows_pad}")
    q = filled_u8((C, rows_pad))
    sc = filled_u8((C, rows_pad // 32))
    q, sc, op = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=rule, rows_pad=rows_pad,
                               q=q, scale=sc)
    qr, sr, opr = oracle.quantize_mx_rows_grouped(x, offs, rule, rows_pad)
    assert_bytes_equal(host(op), opr, "padded offsets")
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), sr, "e8m0")


@pytest.mark.parametrize("case", list(MX_GROUP_CASES))
def test_mx_rows_grouped_k4_layout(case):
    M, C, offs = MX_GROUP_CASES[case]
    x = special_input(6100 + M, (M, C), 0.01, 30.0)
    rows_pad = fm.quantize_mx_rows_bound(M, len(offs)) + 32      # a tail, and NB not a multiple of 4
    note(f"mx rows grouped K4 case={case} rows_pad={rows_pad}")
    sc = filled_u8(fm.mx_k4_shape(C, rows_pad // 32))
    q, sc, op = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=0, rows_pad=rows_pad, scale=sc,
                               layout=fm.MX_LAYOUT_K4)
    qr, sr, opr = oracle.quantize_mx_rows_grouped(x, offs, 0, rows_pad)
    assert_bytes_equal(host(op), opr, "padded offsets")
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), e8m0_rows_to_k4(sr), "e8m0 K4")


@pytest.mark.parametrize("rule", [0, 1])
def test_mx_cast_every_bf16_value(rule):
    """The MX cast runs on gfx950's scaled converter.  For block exponents X across the whole range
    (-127 .. 119: the e8m0 extremes, the subnormal-maximum clamp, both sides of 0, the largest bf16), every
    bf16 magnitude up to the block maximum, with both signs, is cast in blocks whose first element pins
    that maximum; this covers the values that land in (448, 512) under the FLOOR rule (the converter's NaN
    range, mapped back to +-448), subnormal results and signed zeros.  Bit-exact against the oracle."""
    Xs = [-127, -126, -125, -120, -100, -60, -20, -9, -8, -1, 0, 1, 8, 30, 60, 100, 117, 118, 119]
    blocks = []
    for X in Xs:
        field = X + 135
        if field < 1:
            continue
        # FLOOR: any significand gives X; CEIL: a significand up to 0x60 (1.75) keeps X
        pilot = (field << 7) | (0x7F if rule == 0 else 0x60)
        mags = np.arange(0, pilot + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | 0x8000])
        n = (vals.size + 30) // 31
        body = np.zeros(n * 31, np.uint16)
        body[:vals.size] = vals
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = pilot
        blk[:, 1:] = body.reshape(n, 31)
        blocks.append(blk)
    allb = np.concatenate(blocks)
    allb = np.concatenate([allb, np.zeros(((-allb.shape[0]) % 4, 32), np.uint16)])   # whole rows of 4 blocks
    x = allb.reshape(-1, 128)
    note(f"mx cast sweep rule={rule}: {x.size} values")
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule)
    qr, sr = oracle.quantize_mx_lastdim(x, rule)
    assert_bytes_equal(host(sc), sr, "e8m0")
    assert_bytes_equal(host(q), qr, "codes")
    note(f"mx cast sweep rule={rule}: row blocks")
    xt = np.ascontiguousarray(x[: x.shape[0] // 32 * 32].reshape(-1, 32, 128)[:4].transpose(0, 2, 1))   # blocks down columns
    qt, sct, _ = fm.quantize_mx(bf16_dev(xt), axis=0, rule=rule)
    qtr, strr = oracle.quantize_mx_rows_batched(xt, rule)
    assert_bytes_equal(host(sct), strr, "row-block e8m0")
    assert_bytes_equal(host(qt), qtr, "row-block codes")


# ------------------------------------------------------------------- MXFP8, both forms from one read

def _dual_check(x, xq, offs, rule, layout, rows_pad, what):
    """quantize_mx_dual against the oracle's last-dim and row-block quantizers (and so against the two
    quantize_mx calls it stands for), with sentinels in every output."""
    q, sc, q_t, sc_t = _dual_outputs(x.shape, offs is not None, layout, rows_pad)
    note(f"mx dual {what} rule={rule} layout={layout} shape={x.shape}")
    outs = fm.quantize_mx_dual(xq, None if offs is None else i32_dev(offs), rule=rule, rows_pad=rows_pad, q=q,
                               scale=sc, q_t=q_t, scale_t=sc_t, layout=layout)
    _dual_verify(x, offs, rule, layout, rows_pad, outs, what)


def _dual_outputs(x_shape, grouped, layout, rows_pad):
    """Sentinel-filled outputs of the dual MX quantizers for a [B, R, C] (not grouped) or [R, C] tensor."""
    k4 = layout == fm.MX_LAYOUT_K4
    if not grouped:
        B, R, C = x_shape
        rows_total, scale_t_rows, nb_t = B * R, B * C, R // 32
        q_t = filled_u8((B, C, R))
    else:
        (R, C), B = x_shape, 1
        rows_total, scale_t_rows, nb_t = R, C, rows_pad // 32
        q_t = filled_u8((C, rows_pad))
    q = filled_u8((rows_total, C))
    sc = filled_u8(fm.mx_k4_shape(rows_total, C // 32) if k4 else (rows_total, C // 32))
    sc_t = filled_u8(fm.mx_k4_shape(scale_t_rows, nb_t) if k4 else (scale_t_rows, nb_t))
    return q, sc, q_t, sc_t


def _dual_verify(x, offs, rule, layout, rows_pad, outs, what):
    """Both MX forms `outs` = (q, sc, q_t, sc_t, offs_pad) of the host tensor x against the oracle's last-dim
    and row-block quantizers; last-dim rows past the last group must keep their sentinel."""
    q, sc, q_t, sc_t, op = outs
    k4 = layout == fm.MX_LAYOUT_K4
    if offs is None:
        B, R, C = x.shape
        rows_total, scale_t_rows, nb_t = B * R, B * C, R // 32
    else:
        (R, C), B = x.shape, 1
        rows_total, scale_t_rows, nb_t = R, C, rows_pad // 32
    x2 = x.reshape(rows_total, C)
    if offs is None:
        covered = rows_total
        qtr, str_ = oracle.quantize_mx_rows_batched(x, rule)
        str_ = str_.reshape(scale_t_rows, nb_t)
    else:
        covered = int(min(max(int(np.clip(offs, 0, R).max()), 0), R))
        qtr, str_, opr = oracle.quantize_mx_rows_grouped(x, offs, rule, rows_pad)
        assert_bytes_equal(host(op), opr, f"{what} padded offsets")
    assert_bytes_equal(host(q_t), qtr, f"{what} row-block codes")
    assert_bytes_equal(host(sc_t), e8m0_rows_to_k4(str_) if k4 else str_, f"{what} row-block e8m0")
    ql, sl = oracle.quantize_mx_lastdim(x2[:covered], rule)
    qh = host(q)
    assert_bytes_equal(qh[:covered], ql, f"{what} last-dim codes")
    assert np.all(qh[covered:] == 0xA5), f"{what}: rows past the last group must stay untouched"
    if k4:
        full = np.full((rows_total, C // 32), 0xA5, np.uint8)
        full[:covered] = sl.reshape(covered, C // 32)
        want = e8m0_rows_to_k4(full)
        got = host(sc)
        if covered < rows_total:          # the untouched rows' K4 bytes, padding included, keep the sentinel
            want[:, covered:, :] = 0xA5
        assert_bytes_equal(got, want, f"{what} last-dim e8m0 K4")
    else:
        assert_bytes_equal(host(sc)[:covered], sl.reshape(covered, C // 32), f"{what} last-dim e8m0")
        assert np.all(host(sc)[covered:] == 0xA5)


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("layout", [fm.MX_LAYOUT_ROWS, fm.MX_LAYOUT_K4])
@pytest.mark.parametrize("shape", [(2, 64, 96), (3, 288, 160), (1, 32, 32), (2, 544, 224), (4, 1024, 512)])
def test_mx_dual_batched(rule, layout, shape):
    """Batched (weights): last-dim blocks of x viewed [B*R, C] and row blocks per batch item.  Widths give
    1 to 16 blocks per row, odd block counts (a tile's second block past the end) and block counts of 1, 2
    and 3 modulo 4 (the K4 stage padding)."""
    x = special_input(7000 + sum(shape), shape, 0.01, 30.0)
    _dual_check(x, bf16_dev(x), None, rule, layout, None, "batched")


MX_DUAL_GROUP_CASES = {
    "ragged": (1300, 160, synth.offsets_from_counts(synth.random_counts(8, 1290, 7))),   # 10 rows in no group
    "cfg1": (512, 256, synth.offsets_from_counts(synth.routing_counts(1))),
    "malformed": (300, 64, np.array([40, 20, 300, 500], np.int32)),
    "one_row": (1, 32, np.array([1], np.int32)),
    "wide": (700, 5120, synth.offsets_from_counts(synth.random_counts(9, 700, 16))),
    **{k: (M, 160, o) for k, (M, C, o) in LOOKUP_EDGE_CASES.items()},
}


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("layout", [fm.MX_LAYOUT_ROWS, fm.MX_LAYOUT_K4])
@pytest.mark.parametrize("case", list(MX_DUAL_GROUP_CASES))
def test_mx_dual_grouped(rule, layout, case):
    """Grouped (activations): last-dim blocks of the rows inside groups and padded row blocks per group."""
    M, C, offs = MX_DUAL_GROUP_CASES[case]
    x = special_input(7100 + M + C, (M, C), 0.01, 30.0)
    rows_pad = fm.quantize_mx_rows_bound(M, len(offs)) + 32
    _dual_check(x, bf16_dev(x), offs, rule, layout, rows_pad, case)


def test_mx_dual_llama4_scout_weights_sampled():
    """W2 of the Llama4-Scout layer ([16, 5120, 8192]) in the dual form, against the two quantize_mx calls
    it replaces (bit for bit, whole tensors) and the oracle on sampled rows and columns."""
    w = synth.WORKLOADS[5]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    x = (torch.randn(w.E, w.H, w.F, device=DEV, generator=gen) * 0.02).to(torch.bfloat16)
    note("mx dual Llama4-Scout W2 full size")
    q, sc, q_t, sc_t, _ = fm.quantize_mx_dual(x, layout=fm.MX_LAYOUT_K4)
    q1, s1, _ = fm.quantize_mx(x.view(w.E * w.H, w.F), axis=1, layout=fm.MX_LAYOUT_K4)
    q2, s2, _ = fm.quantize_mx(x, axis=0, layout=fm.MX_LAYOUT_K4)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(sc, s1), "last-dim form differs from quantize_mx(axis=1)"
    assert torch.equal(q_t, q2) and torch.equal(sc_t, s2), "row-block form differs from quantize_mx(axis=0)"
    xh = host(x)
    rows = _sample(w.E * w.H, 64, 11)
    ql, sl = oracle.quantize_mx_lastdim(xh.reshape(-1, w.F)[rows], 0)
    assert_bytes_equal(host(q)[rows], ql, "last-dim codes sampled")


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("rule,layout", [(0, fm.MX_LAYOUT_K4), (1, fm.MX_LAYOUT_ROWS)])
@pytest.mark.parametrize("shape", [(700, 2, 5, 320), (96, 1, 3, 32), (0, 2, 4, 64)])
def test_moe_permute_mx_dual(weighted, rule, layout, shape):
    """The gather into moe_route's grouped layout fused with both MX forms: the same bytes as the oracle's
    gather (or, with router weights, the routed-row gradients of the oracle's combine backward) quantized by
    the oracle's MX quantizers; the optional bf16 copy equals the gathered rows; rows past the last group
    keep their sentinels.  Dropped slots (ids -1) leave zero rows."""
    from oracle import route as rt
    T, k, E, C = shape
    rng = np.random.default_rng(T + 7 * k + C + 2 * weighted)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 10:
        ids[rng.random((T, k)) < 0.03] = -1
    x = synth.normal_bf16(9100 + T + C, (T, C), 1.0, 0.01, 30.0)
    counts, offs, dest, src = fm.moe_route(i32_dev(ids), E, 1)
    R = src.numel()
    w = (rng.random((T, k)) + 0.05).astype(np.float32) if weighted else None
    rows_pad = fm.quantize_mx_rows_bound(R, E) + 32
    q, sc, q_t, sc_t = _dual_outputs((R, C), True, layout, rows_pad)
    xg = torch.full((R, C), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    note(f"moe_permute_quantize_mx_dual T={T} k={k} E={E} C={C} rows={R} weighted={weighted} rule={rule}")
    got = fm.moe_permute_quantize_mx_dual(bf16_dev(x), src, k, offs, weights=None if w is None else
                                          torch.from_numpy(w).to(DEV), rule=rule, rows_pad=rows_pad, xg=xg, q=q,
                                          scale=sc, q_t=q_t, scale_t=sc_t, layout=layout)
    src_h, dest_h, offs_h = host(src), host(dest), host(offs)
    if w is None:
        ref = rt.permute(x, src_h, k)
    else:
        ref, _ = rt.combine_backward(x, np.zeros((R, C), np.uint16), src_h, dest_h, w, T, k)
    covered = int(offs_h[-1]) if E else 0
    xg_h = host(got[0])
    assert_bytes_equal(xg_h[:covered], ref[:covered], "gathered rows (bf16 copy)")
    assert np.all(xg_h.view(np.uint16)[covered:] == 0x5A5A), "copy rows past the last group untouched"
    _dual_verify(ref, offs_h, rule, layout, rows_pad, got[1:], f"permute mx dual weighted={weighted}")


# ------------------------------------------------------------------- full-size, sampled

def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))


@pytest.mark.parametrize("cfg,tensor", [(2, "dy"), (2, "w1"), (3, "w1"), (4, "x")])
def test_rowwise_full_size_sampled(cfg, tensor):
    w = synth.WORKLOADS[cfg]
    x = {"dy": synth.make_dy, "x": synth.make_x, "w1": synth.make_w1}[tensor](w)
    x = x.reshape(-1, x.shape[-1])
    note(f"rowwise full cfg={cfg} {tensor} {x.shape}")
    q, s = fm.quantize_rowwise(bf16_dev(x), fm.E4M3FN)
    rows = _sample(x.shape[0], 48, cfg)
    qh, sh = host(q), host(s)
    qr, sr = oracle.quantize_rowwise(x[rows], fm.E4M3FN)
    assert_bytes_equal(qh[rows], qr, "codes")
    assert_f32_bits_equal(sh[rows], sr, "scales")


@pytest.mark.parametrize("cfg,tensor", [(2, "dy"), (3, "x"), (4, "dy"), (4, "a2")])
def test_colwise_grouped_full_size_sampled(cfg, tensor):
    w = synth.WORKLOADS[cfg]
    x = {"dy": synth.make_dy, "x": synth.make_x, "a2": synth.make_a2}[tensor](w)
    offs = w.offs
    note(f"colwise full cfg={cfg} {tensor} {x.shape}")
    q_t, sc = fm.quantize_colwise(bf16_dev(x), i32_dev(offs), fm.E4M3FN)
    cols = _sample(x.shape[1], 12, cfg + 10)
    qh, sh = host(q_t), host(sc)
    qr, sr = oracle.quantize_colwise_grouped(np.ascontiguousarray(x[:, cols]), offs, fm.E4M3FN)
    assert_bytes_equal(qh[cols], qr, "codes")
    assert_f32_bits_equal(sh[:, cols], sr, "scales")


@pytest.mark.parametrize("tensor", ["w1", "w2"])
def test_colwise_batched_full_size_sampled(tensor):
    w = synth.WORKLOADS[4]
    x = synth.make_w1(w) if tensor == "w1" else synth.make_w2(w)  # [32, 4096, 7168] / [32, 7168, 2048]
    note(f"colwise batched full cfg=4 {tensor} {x.shape}")
    q_t, sc = fm.quantize_colwise(bf16_dev(x), None, fm.E4M3FN)
    cols = _sample(x.shape[2], 8, 44)
    qh, sh = host(q_t), host(sc)
    qr, sr = oracle.quantize_colwise_batched(np.ascontiguousarray(x[:, :, cols]), fm.E4M3FN)
    assert_bytes_equal(qh[:, cols], qr, "codes")
    assert_f32_bits_equal(sh[:, cols], sr, "scales")


def test_mx_full_size_sampled():
    w = synth.WORKLOADS[5]
    x = synth.make_dy(w)                                          # [16384, 5120]
    offs = w.offs
    note(f"mx full cfg=5 dy {x.shape}")
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=0)
    rows = _sample(x.shape[0], 32, 5)
    qr, sr = oracle.quantize_mx_lastdim(x[rows], 0)
    assert_bytes_equal(host(q)[rows], qr, "codes lastdim")
    assert_bytes_equal(host(sc)[rows], sr, "e8m0 lastdim")
    rows_pad = fm.quantize_mx_rows_bound(x.shape[0], len(offs))
    q, sc, op = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=0, rows_pad=rows_pad)
    cols = _sample(x.shape[1], 8, 6)
    qr, sr, opr = oracle.quantize_mx_rows_grouped(np.ascontiguousarray(x[:, cols]), offs, 0, rows_pad)
    assert_bytes_equal(host(op), opr, "padded offsets")
    assert_bytes_equal(host(q)[cols], qr, "codes rows")
    assert_bytes_equal(host(sc)[cols], sr, "e8m0 rows")


# ------------------------------------------------------------------- edge cases

def _subnormal_bf16(seed, shape):
    """bf16 patterns of nonzero subnormals only (exponent field 0), random signs."""
    rng = np.random.default_rng(seed)
    mant = rng.integers(1, 128, size=shape).astype(np.uint16)
    sign = (rng.random(shape) < 0.5).astype(np.uint16) << np.uint16(15)
    return (mant | sign).astype(np.uint16)


@pytest.mark.parametrize("rule", [0, 1])
def test_mx_all_subnormal_blocks(rule):
    """Blocks made only of bf16 subnormals: the shared exponent clamps at -127 (e8m0 code 0) and
    x * 2^127 stays non-zero, so no code of a non-zero input may be zero (no flush to zero)."""
    R, C = 64, 256
    x = _subnormal_bf16(71, (R, C))
    x[5, 32:64] = 0                  # one all-zero block beside them
    x[9, :32] = 1                    # the smallest subnormal, 2^-133, everywhere in a block
    note(f"mx all-subnormal rule={rule}")
    q, sc, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule)
    qr, sr = oracle.quantize_mx_lastdim(x, rule)
    assert_bytes_equal(host(q), qr, "codes")
    assert_bytes_equal(host(sc), sr, "e8m0")
    assert not host(sc).any(), "subnormal blocks take X = -127 (code 0)"
    nz = x.reshape(R, C) & 0x7FFF != 0
    assert np.all(host(q)[nz] & 0x7F != 0), "a subnormal input was flushed to a zero code"
    _, sk, _ = fm.quantize_mx(bf16_dev(x), axis=1, rule=rule, layout=fm.MX_LAYOUT_K4)
    assert_bytes_equal(host(sk), e8m0_rows_to_k4(sr), "e8m0 K4")
    xb = x.reshape(2, 32, C)         # row blocks, batched
    q, sc, _ = fm.quantize_mx(bf16_dev(xb), axis=0, rule=rule)
    qr, sr = oracle.quantize_mx_rows_batched(xb, rule)
    assert_bytes_equal(host(q), qr, "row-block codes")
    assert_bytes_equal(host(sc), sr, "row-block e8m0")
    offs = np.array([20, 20, 64], np.int32)          # grouped, with an empty group and padding
    Mp = fm.quantize_mx_rows_bound(R, 3)
    q, sc, op = fm.quantize_mx(bf16_dev(x), axis=0, offs=i32_dev(offs), rule=rule, rows_pad=Mp)
    qr, sr, opr = oracle.quantize_mx_rows_grouped(x, offs, rule, Mp)
    assert_bytes_equal(host(q), qr, "grouped codes")
    assert_bytes_equal(host(sc), sr, "grouped e8m0")
    assert_bytes_equal(host(op), opr, "padded offsets")


@pytest.mark.parametrize("codec", CODECS)
def test_colwise_wait_fallback_bit_exact(codec, chunk_rows):
    """With a poll budget of 0 every chunk of a multi-chunk group recomputes its group's column
    maxima from x (the path a chunk takes when its peers do not publish in time); every kernel
    still exits normally and the result is the same, bit for bit."""
    lib = fm._lib.lib()
    M, C = 3000, 200
    x = special_input(7100 + codec, (M, C))
    offs = np.array([1300, 1300, 2950], np.int32)    # groups of 1300 and 1650 rows (3-4 chunks), an empty one
    qr, sr = oracle.quantize_colwise_grouped(x, offs, codec)
    xb = special_input(7200 + codec, (2, 1100, 64))
    qbr, sbr = oracle.quantize_colwise_batched(xb, codec)
    prev = lib.fp8moe_set_colwise_poll_budget(0)
    try:
        note(f"colwise with no polls codec={codec}")
        q, s = fm.quantize_colwise(bf16_dev(x), i32_dev(offs), codec)
        qb, sb = fm.quantize_colwise(bf16_dev(xb), None, codec, ld_q=1104)
        qh, qbh = host(q), host(qb)
    finally:
        lib.fp8moe_set_colwise_poll_budget(prev)
    assert_bytes_equal(qh[:, :2950], qr[:, :2950], "codes")
    assert_f32_bits_equal(host(s), sr, "scales")
    assert_bytes_equal(qbh[:, :, :1100], qbr, "batched codes")
    assert_f32_bits_equal(host(sb), sbr, "batched scales")


def _routed(T, k, E, C, seed, drop=0.03, one_expert=False):
    """Token rows, their routing (GPU moe_route, pad 1) and router weights for the gathered quantizers."""
    rng = np.random.default_rng(seed)
    ids = (np.zeros((T, k)) if one_expert else rng.integers(0, E, size=(T, k))).astype(np.int32)
    if T > 10 and drop:
        ids[rng.random((T, k)) < drop] = -1
    x = synth.normal_bf16(seed + 1, (T, C), 1.0, 0.01, 30.0)
    w = (rng.random((T, k)) + 0.05).astype(np.float32)
    return x, w, fm.moe_route(i32_dev(ids), E, 1)


def _gathered_ref(x, w, src, dest, k):
    from oracle import route as rt
    T, C = x.shape
    if w is None:
        return rt.permute(x, src, k)
    return rt.combine_backward(x, np.zeros((src.size, C), np.uint16), src, dest, w, T, k)[0]


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("shape", [(700, 2, 5, 136), (3000, 1, 4, 64), (96, 6, 8, 200)])
def test_moe_permute_colwise(weighted, codec, shape, chunk_rows):
    """The gather into moe_route's grouped layout fused with the colwise quantizer: the same bytes as the
    oracle's gather (with router weights: the routed-row gradients of its combine backward) followed by
    its grouped colwise quantizer, on every single-pass chunk height."""
    T, k, E, C = shape
    x, w, (counts, offs, dest, src) = _routed(T, k, E, C, 9300 + T + C + codec)
    R = src.numel()
    ld_q = (R + 15) // 16 * 16 + 16
    note(f"moe_permute_quantize_colwise T={T} k={k} E={E} C={C} weighted={weighted} codec={codec} "
         f"chunk rows={chunk_rows}")
    q_t, sc = filled_u8((C, ld_q)), filled_f32((E, C))
    fm.moe_permute_quantize_colwise(bf16_dev(x), src, k, offs, weights=torch.from_numpy(w).to(DEV) if weighted
                                    else None, codec=codec, q_t=q_t, scale=sc, ld_q=ld_q)
    g = _gathered_ref(x, w if weighted else None, host(src), host(dest), k)
    qr, sr = oracle.quantize_colwise_grouped(g, host(offs), codec, q_init=np.full((C, ld_q), 0xA5, np.uint8),
                                             ld_q=ld_q)
    assert_bytes_equal(host(q_t), qr, "codes")
    assert_f32_bits_equal(host(sc), sr, "scales")


@pytest.mark.parametrize("weighted", [False, True])
def test_moe_permute_colwise_other_paths(weighted):
    """The gathered colwise quantizer on its other paths, bit for bit: the fallback a chunk takes when its
    peers do not publish in time (poll budget 0, so every multi-chunk group re-reads its rows through the
    gather) and the two-pass kernels (one group of 70000 rows, more than 128 chunks)."""
    lib = fm._lib.lib()
    x, w, (counts, offs, dest, src) = _routed(3000, 2, 3, 72, 9400)
    ref = oracle.quantize_colwise_grouped(_gathered_ref(x, w if weighted else None, host(src), host(dest), 2),
                                          host(offs), 0)
    wd = torch.from_numpy(w).to(DEV) if weighted else None
    prev = lib.fp8moe_set_colwise_poll_budget(0)
    try:
        note(f"moe_permute_quantize_colwise with no polls weighted={weighted}")
        q, s = fm.moe_permute_quantize_colwise(bf16_dev(x), src, 2, offs, weights=wd)
        qh, sh = host(q), host(s)
    finally:
        lib.fp8moe_set_colwise_poll_budget(prev)
    used = int(host(offs)[-1])
    assert_bytes_equal(qh[:, :used], ref[0][:, :used], "codes (fallback)")
    assert_f32_bits_equal(sh, ref[1], "scales (fallback)")
    xt, wt, (ct, ot, dt, st_) = _routed(70000, 1, 1, 64, 9500, drop=0.0, one_expert=True)
    note(f"moe_permute_quantize_colwise two-pass weighted={weighted}")
    q, s = fm.moe_permute_quantize_colwise(bf16_dev(xt), st_, 1, ot, weights=torch.from_numpy(wt).to(DEV)
                                           if weighted else None)
    qr, sr = oracle.quantize_colwise_grouped(_gathered_ref(xt, wt if weighted else None, host(st_), host(dt), 1),
                                             host(ot), 0)
    assert_bytes_equal(host(q)[:, :70000], qr[:, :70000], "codes (two-pass)")
    assert_f32_bits_equal(host(s), sr, "scales (two-pass)")


def test_colwise_graph_replays():
    """A call captured into a HIP graph and replayed with new inputs (eager calls in between, which
    advance the single-pass kernel's tag) gives the oracle's result on every replay."""
    M, C = 2000, 136
    offs = np.array([700, 700, 1900], np.int32)
    xs = bf16_dev(special_input(7300, (M, C)))
    ws = bf16_dev(special_input(7301, (3, 640, 64)))
    od = i32_dev(offs)
    q, s = filled_u8((C, M)), filled_f32((3, C))
    qw, sw = filled_u8((3, 64, 640)), filled_f32((3, 64))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up off the default stream, as capture requires
        fm.quantize_colwise(xs, od, 0, q_t=q, scale=s)
        fm.quantize_colwise(ws, None, 0, q_t=qw, scale=sw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("colwise graph capture")
    with torch.cuda.graph(g):
        fm.quantize_colwise(xs, od, 0, q_t=q, scale=s)
        fm.quantize_colwise(ws, None, 0, q_t=qw, scale=sw)
    for rep in range(4):
        xh = special_input(7310 + rep, (M, C), sigma=4.0 ** rep)
        wh = special_input(7320 + rep, (3, 640, 64), sigma=0.5 ** rep)
        xs.copy_(bf16_dev(xh))
        ws.copy_(bf16_dev(wh))
        fm.quantize_colwise(bf16_dev(special_input(7330 + rep, (M, C))), od, 0)    # eager call in between
        torch.cuda.synchronize()
        note(f"colwise graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        qr, sr = oracle.quantize_colwise_grouped(xh, offs, 0)
        assert_bytes_equal(host(q)[:, :1900], qr[:, :1900], f"replay {rep} codes")
        assert_f32_bits_equal(host(s), sr, f"replay {rep} scales")
        qwr, swr = oracle.quantize_colwise_batched(wh, 0)
        assert_bytes_equal(host(qw), qwr, f"replay {rep} batched codes")
        assert_f32_bits_equal(host(sw), swr, f"replay {rep} batched scales")


@pytest.mark.parametrize("codec", CODECS)
def test_device_encoder_monotone_exhaustive(codec):
    """Every fp32 value in [0, fmax], encoded on the device: codes never decrease as the value
    grows, and -y encodes as y with the sign bit (e4m3fnuz: a zero code stays 0x00).  With the
    midpoint probes of test_device_encoder_matches_oracle (every rounding boundary +-1 ulp) this
    fixes the encoder on every input: between two boundaries a monotone encoder is constant."""
    fm_bits = int(np.float32(oracle.FMAX[codec]).view(np.uint32))
    chunk = 1 << 27
    last = -1
    note(f"encoder sweep codec={codec} values={fm_bits + 1}")
    for start in range(0, fm_bits + 1, chunk):
        stop = min(start + chunk, fm_bits + 1)
        y = torch.arange(start, stop, dtype=torch.int32, device=DEV).view(torch.float32)
        qp = fm.encode_f32(y, codec).to(torch.int32)
        qn = fm.encode_f32(-y, codec).to(torch.int32)
        assert bool((qp[1:] >= qp[:-1]).all()), f"codes decrease inside [{start}, {stop})"
        assert int(qp[0]) >= last, f"codes decrease at bit pattern {start}"
        assert int(qp.max()) <= (0x7E if codec == 0 else 0x7F) and int(qp.min()) >= 0
        want_n = qp | 0x80 if codec == 0 else torch.where(qp == 0, qp, qp | 0x80)
        assert bool((qn == want_n).all()), f"negative values inside [{start}, {stop})"
        last = int(qp[-1])
        del y, qp, qn
    assert last == (0x7E if codec == 0 else 0x7F)
    torch.cuda.synchronize()


def test_default_codec_on_gfx950():
    """fp8moe_default_codec picks the OCP e4m3fn codec on gfx950 (its FP8 matrix cores take it)."""
    import ctypes
    out = ctypes.c_int(-1)
    assert fm._lib.lib().fp8moe_default_codec(torch.cuda.current_device(), ctypes.byref(out)) == 0
    assert out.value == fm.E4M3FN
    assert fm.default_codec() == fm.E4M3FN
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
