"""GPU parity of the routing kernels (moe_route, moe_permute, moe_permute_rowwise,
moe_combine, moe_combine_backward) against the oracle (oracle/route.py).

Everything here is integer or byte work, or an fp32 sum in a fixed order of
round-to-nearest operations: all outputs must match the oracle bit for bit.
The one exception is the router-weight gradient of moe_combine_backward, an
fp32 dot product in the kernel's own order, accepted within fp32 summation
error of the exact sum."""
import numpy as np
import pytest
import torch

import mxfp8_quantized_moe_amd as fm
from mxfp8_quantized_moe_amd import synth
from oracle import route as rt
from oracle.swiglu import round_bf16
from gpu_helpers import (DEV, note, bf16_dev, i32_dev, host, assert_bytes_equal, assert_f32_bits_equal,
                         filled_u8, filled_f32)

pytestmark = pytest.mark.gpu


def check_route(ids: np.ndarray, E: int, pad: int, what: str):
    note(f"moe_route {what}: tokens={ids.shape[0]} topk={ids.shape[1]} E={E} pad={pad}")
    got = fm.moe_route(i32_dev(ids), E, pad)
    ref = rt.route(ids, E, pad)
    for name, g, r in zip(("counts", "offs", "dest", "src"), got, ref):
        assert_bytes_equal(host(g), r, f"{what} {name}")
    return got, ref


SMALL = [
    (np.array([[2, 0, 1], [1, 2, 4], [0, 0, 3], [4, 1, 2], [2, 3, 0], [1, 1, 4], [3, 2, 0]]), 5, 1),
    (np.array([[2, 0, 1], [1, 2, 4], [0, 0, 3], [4, 1, 2], [2, 3, 0], [1, 1, 4], [3, 2, 0]]), 5, 4),
    (np.array([[0, 7], [-1, 2], [2, 2], [5, 1]]), 6, 2),          # ids 7 and -1 drop their slots
    (np.zeros((9, 2), dtype=np.int32), 3, 8),                      # one expert takes everything
    (np.zeros((0, 4), dtype=np.int32), 8, 32),                     # no tokens: all padding-free, src all -1
    (np.arange(12).reshape(12, 1) % 4, 4, 1),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_route_small(case):
    ids, E, pad = SMALL[case]
    check_route(np.asarray(ids, np.int32), E, pad, f"small{case}")


# tokens x topk spanning several 256-slot blocks and a ragged tail; experts up to the maximum
RANDOM = [(1000, 6, 64, 1), (1000, 6, 64, 32), (777, 2, 7, 16), (3001, 1, 1, 1), (513, 8, 256, 128),
          (2048, 4, 1024, 1), (2048, 4, 1024, 32), (255, 1, 1000, 3), (4099, 3, 33, 5)]


@pytest.mark.parametrize("shape", RANDOM)
def test_route_random(shape):
    T, k, E, pad = shape
    rng = np.random.default_rng(T * 31 + k * 7 + E + pad)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 10:
        ids[rng.random((T, k)) < 0.01] = -1                          # dropped slots
        ids[3, 0] = E                                               # an id past the last expert
    check_route(ids, E, pad, "random")


def test_route_skewed_and_runs():
    """Long runs of one expert inside a wave and across blocks; most experts empty."""
    T, k, E = 5000, 2, 40
    ids = np.full((T, k), 17, np.int32)
    ids[::97, 1] = 3
    ids[2000:2600] = 39
    check_route(ids, E, 16, "skewed")


@pytest.mark.parametrize("cfg,E,pad", [(3, 64, 1), (3, 64, 32), (4, 32, 1), (4, 32, 128)])
def test_route_workload_routing(cfg, E, pad):
    """The DeepSeek-MoE-16B (8192 tokens top-6 over 64 experts) and DeepSeek-V3
    share (8192 tokens top-1 over 32 experts) routings, in the launch the bench times."""
    check_route(synth.routing_ids(cfg), E, pad, f"workload{cfg}")


def test_route_repeated_calls_reuse_buffers():
    """Stale outputs and workspace from an earlier, larger call do not leak into a smaller one."""
    rng = np.random.default_rng(5)
    big = rng.integers(0, 16, size=(3000, 4)).astype(np.int32)
    small = rng.integers(0, 16, size=(300, 4)).astype(np.int32)
    rows_big = fm.moe_route_rows_bound(big.size, 16, 8)
    out = (torch.full((16,), -5, dtype=torch.int32, device=DEV), torch.full((16,), -5, dtype=torch.int32, device=DEV),
           torch.full((big.size,), -5, dtype=torch.int32, device=DEV),
           torch.full((rows_big,), -5, dtype=torch.int32, device=DEV))
    ws = torch.full((1 << 20,), 0x7F, dtype=torch.uint8, device=DEV)
    note("moe_route repeated calls")
    fm.moe_route(i32_dev(big), 16, 8, out=out, workspace=ws)
    rows_small = fm.moe_route_rows_bound(small.size, 16, 8)
    sub = (out[0], out[1], out[2][:small.size], out[3][:rows_small])
    fm.moe_route(i32_dev(small), 16, 8, out=sub, workspace=ws)
    for name, g, r in zip(("counts", "offs", "dest", "src"), sub, rt.route(small, 16, 8)):
        assert_bytes_equal(host(g), r, f"second call {name}")


def bf16_random(rng, shape, scale=1.0):
    return round_bf16(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("shape", [(7, 3, 5, 4, 8), (1000, 6, 64, 32, 136), (300, 1, 16, 1, 2048),
                                   (129, 8, 256, 16, 24), (0, 2, 4, 16, 64)])
def test_permute_and_combine(shape):
    T, k, E, pad, C = shape
    rng = np.random.default_rng(T + C)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 10:
        ids[rng.random((T, k)) < 0.02] = -1
    x = bf16_random(rng, (T, C))
    (counts, offs, dest, src), (_, _, dref, sref) = check_route(ids, E, pad, "permute/combine")
    note(f"moe_permute T={T} k={k} C={C} rows={src.numel()}")
    xg = fm.moe_permute(bf16_dev(x), src, k)
    assert_bytes_equal(host(xg), rt.permute(x, sref, k), "xg")
    yg = bf16_random(rng, (src.numel(), C), 3.0)
    w = rng.random((T, k)).astype(np.float32)
    note(f"moe_combine T={T} k={k} C={C}")
    y = fm.moe_combine(bf16_dev(yg), dest, torch.from_numpy(w).to(DEV), k)
    assert_bytes_equal(host(y), rt.combine(yg, dref, w, T, k), "y")


def test_combine_ignores_out_of_range_dest():
    """A dest at or past rows_in contributes nothing (as a dropped slot)."""
    rng = np.random.default_rng(9)
    T, k, C, R = 40, 3, 64, 100
    dest = rng.integers(0, R, size=T * k).astype(np.int32)
    dest[::7] = R + 3
    dest[1::11] = -1
    yg = bf16_random(rng, (R, C))
    w = rng.random((T, k)).astype(np.float32)
    note("moe_combine out-of-range dest")
    y = fm.moe_combine(bf16_dev(yg), i32_dev(dest), torch.from_numpy(w).to(DEV), k)
    ref_dest = np.where(dest >= R, -1, dest)
    assert_bytes_equal(host(y), rt.combine(yg, ref_dest, w, T, k), "y")


@pytest.mark.parametrize("cfg,E,C", [(3, 64, 2048), (4, 32, 7168)])
def test_workload_permute_combine_sampled(cfg, E, C):
    """Full-size permute and combine on the workloads' routing and hidden sizes
    (MX padding of 32); grouped rows and tokens sampled for the oracle."""
    ids = synth.routing_ids(cfg)
    T, k = ids.shape
    gen = torch.Generator(device=DEV)
    gen.manual_seed(cfg)
    x = torch.randn(T, C, device=DEV, generator=gen).to(torch.bfloat16)
    counts, offs, dest, src = fm.moe_route(i32_dev(ids), E, 32)
    note(f"workload {cfg} permute/combine full size")
    xg = fm.moe_permute(x, src, k)
    w = torch.rand(T, k, device=DEV, generator=gen)
    y = fm.moe_combine(xg, dest, w, k)
    srch, desth, xh, wh = host(src), host(dest), host(x), host(w)
    rng = np.random.default_rng(cfg)
    rows = rng.choice(src.numel(), 512, replace=False)
    want = np.where((srch[rows] >= 0)[:, None], xh[np.clip(srch[rows], 0, None) // k], 0).astype(np.uint16)
    assert_bytes_equal(host(xg)[rows], want, "xg sampled")
    toks = rng.choice(T, 256, replace=False)
    d = desth.reshape(T, k)[toks]                               # [n, k]
    xgh = host(xg)
    yg_sub = xgh[np.clip(d, 0, None).ravel()]
    dest_sub = np.where(d.ravel() >= 0, np.arange(d.size), -1).astype(np.int32)
    assert_bytes_equal(host(y)[toks], rt.combine(yg_sub, dest_sub, wh[toks], len(toks), k), "y sampled")


@pytest.mark.parametrize("codec", [fm.E4M3FN, fm.E4M3FNUZ])
@pytest.mark.parametrize("shape", [(9, 3, 5, 4, 32), (1000, 6, 64, 32, 2048), (300, 1, 16, 128, 7168), (0, 2, 4, 16, 64)])
def test_permute_quantized(codec, shape):
    """Gather of rowwise codes and scales: bit-exact against the oracle, and equal to quantizing the
    gathered bf16 rows on the device."""
    import oracle
    T, k, E, pad, C = shape
    rng = np.random.default_rng(T + C + codec)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 10:
        ids[rng.random((T, k)) < 0.02] = -1
    x = bf16_random(rng, (T, C), 2.0)
    counts, offs, dest, src = fm.moe_route(i32_dev(ids), E, pad)
    xd = bf16_dev(x)
    note(f"moe_permute_quantized T={T} k={k} C={C} codec={codec}")
    q, s = fm.quantize_rowwise(xd, codec)
    qg, sg = fm.moe_permute_quantized(q, s, src, k, codec)
    qr, sr = rt.permute_quantized(host(q), host(s), host(src), k, codec)
    assert_bytes_equal(host(qg), qr, "qg")
    assert_bytes_equal(host(sg).view(np.uint32), sr.view(np.uint32), "scale_g")
    q2, s2 = fm.quantize_rowwise(fm.moe_permute(xd, src, k), codec)
    assert_bytes_equal(host(qg), host(q2), "qg vs quantize after permute")
    assert_bytes_equal(host(sg).view(np.uint32), host(s2).view(np.uint32), "scale_g vs quantize after permute")
    q_or, s_or = oracle.quantize_rowwise(x, codec)
    assert_bytes_equal(host(q), q_or, "token codes")


@pytest.mark.parametrize("codec", [fm.E4M3FN, fm.E4M3FNUZ])
@pytest.mark.parametrize("shape,keep", [((9, 3, 5, 4, 32), True), ((1000, 6, 64, 32, 2048), True),
                                        ((300, 1, 16, 128, 7168), False), ((40, 2, 3, 8, 16392), True),
                                        ((77, 2, 4, 1, 136), False), ((0, 2, 4, 16, 64), True)])
def test_permute_rowwise(codec, shape, keep):
    """Fused gather + rowwise quantization: the gathered rows bit-exact against the oracle's permute, the
    codes and scales against the oracle's rowwise quantizer of those rows (padding rows: zero codes and the
    all-zero row's scale); rows of 16392 columns take the streaming cast."""
    import oracle
    T, k, E, pad, C = shape
    rng = np.random.default_rng(T + C + codec + 11)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 10:
        ids[rng.random((T, k)) < 0.02] = -1
    x = bf16_random(rng, (T, C), 2.0)
    if T > 5:
        x[4] = 0                                                    # an all-zero token
    counts, offs, dest, src = fm.moe_route(i32_dev(ids), E, pad)
    R = src.numel()
    xg0 = torch.full((R, C), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16) if keep else None
    note(f"moe_permute_rowwise T={T} k={k} C={C} rows={R} codec={codec} keep={keep}")
    xg, qg, sg = fm.moe_permute_rowwise(bf16_dev(x), src, k, codec, xg=xg0, keep_bf16=keep,
                                        qg=filled_u8((R, C)), scale_g=filled_f32((R,)))
    xg_ref = rt.permute(x, host(src), k)
    if keep:
        assert_bytes_equal(host(xg), xg_ref, "xg")
    else:
        assert xg is None
    q_ref, s_ref = oracle.quantize_rowwise(xg_ref, codec)
    assert_bytes_equal(host(qg), q_ref, "qg")
    assert_f32_bits_equal(host(sg), s_ref, "scale_g")


def check_combine_backward(ids, E, pad, C, codec, codes, seed, what):
    import oracle
    T, k = ids.shape
    rng = np.random.default_rng(seed)
    (counts, offs, dest, src), (_, _, dref, sref) = check_route(ids, E, pad, what)
    R = src.numel()
    dy = bf16_random(rng, (T, C), 1e-3)
    yg = bf16_random(rng, (R, C), 2.0)
    w = (rng.random((T, k)) + 0.05).astype(np.float32)
    note(f"moe_combine_backward {what}: T={T} k={k} C={C} rows={R} codec={codec} codes={codes}")
    dyg, q, s, dw = fm.moe_combine_backward(
        bf16_dev(dy), bf16_dev(yg), dest, src, torch.from_numpy(w).to(DEV), k, codec, codes=codes,
        dyg=torch.full((R, C), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16),
        q=filled_u8((R, C)) if codes else None, scale=filled_f32((R,)) if codes else None,
        dweights=filled_f32((T * k,)))
    dyg_ref, dw_ref = rt.combine_backward(dy, yg, sref, dref, w, T, k)
    assert_bytes_equal(host(dyg), dyg_ref, f"{what} dyg")
    if codes:
        q_ref, s_ref = oracle.quantize_rowwise(dyg_ref, codec)
        assert_bytes_equal(host(q), q_ref, f"{what} codes")
        assert_f32_bits_equal(host(s), s_ref, f"{what} scales")
    else:
        assert q is None and s is None
    # dw: exact bf16 products, fp32 sums in the kernel's order: within C * 2^-24 * sum |products|
    dyf = oracle.bf16_to_f32(dy).astype(np.float64)
    ygf = oracle.bf16_to_f32(yg).astype(np.float64)
    ok = dref >= 0
    mag = np.zeros(T * k)
    mag[ok] = np.einsum("sc,sc->s", np.abs(dyf[np.nonzero(ok)[0] // k]), np.abs(ygf[dref[ok]]))
    err = np.abs(host(dw).astype(np.float64) - dw_ref)
    bound = C * 2.0 ** -24 * mag
    assert np.all(err <= bound), f"{what} dw: worst excess {np.max(err - bound):.3e}"
    assert np.all(host(dw)[~ok] == 0.0), f"{what}: dropped slots must get dw = 0"


@pytest.mark.parametrize("codec", [fm.E4M3FN, fm.E4M3FNUZ])
@pytest.mark.parametrize("shape", [(7, 3, 5, 4, 8), (1000, 6, 64, 32, 2048), (300, 1, 16, 1, 7168),
                                   (129, 8, 256, 16, 24), (50, 2, 3, 8, 16384), (0, 2, 4, 16, 64)])
def test_combine_backward(codec, shape):
    """Routed-row gradients bit-exact (and their rowwise codes), router-weight gradients within fp32 summation
    error, padding rows zero, dropped slots zero."""
    T, k, E, pad, C = shape
    rng = np.random.default_rng(T + C + 3)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if T > 10:
        ids[rng.random((T, k)) < 0.02] = -1
    check_combine_backward(ids, E, pad, C, codec, True, T + 7, f"random{shape}")
    if C <= 2048:
        check_combine_backward(ids, E, pad, C, codec, False, T + 8, f"random{shape} no codes")


@pytest.mark.parametrize("cfg,E,C", [(3, 64, 2048), (4, 32, 7168)])
def test_combine_backward_workload(cfg, E, C):
    """The DeepSeek-MoE-16B and DeepSeek-V3-share routings at their hidden sizes."""
    check_combine_backward(synth.routing_ids(cfg), E, 1, C, fm.E4M3FN, True, cfg, f"workload{cfg}")


def test_combine_without_weights():
    """Null weights sum a token's routed rows (the backward's input gradient), as the oracle's unit weights."""
    rng = np.random.default_rng(21)
    T, k, E, C = 500, 6, 64, 2048
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[3, 2] = -1
    (counts, offs, dest, src), (_, _, dref, sref) = check_route(ids, E, 1, "unit weights")
    yg = bf16_random(rng, (src.numel(), C), 3.0)
    note("moe_combine without weights")
    y = fm.moe_combine(bf16_dev(yg), dest, None, k)
    assert_bytes_equal(host(y), rt.combine(yg, dref, None, T, k), "y")
