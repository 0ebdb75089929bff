"""Pins of the SwiGLU oracle (oracle/swiglu.py) to things other than itself:
closed forms, special values, finite differences of the forward for the
backward, torch's fp32 -> bf16 conversion for the rounding, and pure-Python
loops for the gate/up layout."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import swiglu as sw


def f32_bits_to_bf16_bits_torch(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_bits(x: np.ndarray) -> np.ndarray:
    """fp32-exact values -> bf16 bits (values chosen bf16-exact by the caller)."""
    return f32_bits_to_bf16_bits_torch(np.asarray(x, dtype=np.float32))


def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 2.0 ** -126, 2.0 ** -130, -(2.0 ** -133), 65504.0])])
    assert np.array_equal(sw.round_bf16(x.astype(np.float64)), f32_bits_to_bf16_bits_torch(x))


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties go to 1 + 2^-6.
    got = sw.round_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]))
    assert got.tolist() == [0x3F80, 0x3F82, 0xBF80]
    # just above a tie rounds up
    assert sw.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81


def test_sigmoid_closed_forms():
    g = np.array([0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0])
    s = sw._sigmoid(g)
    assert s[0] == 0.5 and abs(s[1] - 0.75) < 1e-15 and abs(s[2] - 0.25) < 1e-15
    assert s[3] == 1.0 and s[4] == 0.0


def test_forward_special_values():
    F = 4
    g = np.float32([0.0, 1.0, -30.0, 40.0])
    u = np.float32([3.0, 0.0, 2.0, 0.5])
    h1 = np.concatenate([to_bits(g), to_bits(u)])[None, :]
    a = oracle.bf16_to_f32(sw.swiglu_fwd(h1, F))[0]
    assert a[0] == 0.0                      # silu(0) = 0
    assert a[1] == 0.0                      # up = 0
    want = -30.0 / (1.0 + math.exp(30.0)) * 2.0                  # silu(-30) * 2, about -5.6e-12
    assert abs(a[2] - want) <= abs(want) * 2.0 ** -8
    assert a[3] == 20.0                     # sigmoid(40) rounds away: 40 * 0.5


def test_forward_closed_form_log3():
    # sigmoid(ln 3) = 3/4, so silu(ln 3) * u = 0.75 ln3 u; the bf16 input ln3 is
    # inexact, so use the bf16 value of ln 3 itself as the gate
    g_bits = to_bits(np.float32([math.log(3.0)]))
    g = float(oracle.bf16_to_f32(g_bits)[0])
    u = 2.0
    h1 = np.concatenate([g_bits, to_bits(np.float32([u]))])[None, :]
    want = g / (1.0 + math.exp(-g)) * u
    got = float(oracle.bf16_to_f32(sw.swiglu_fwd(h1, 1))[0, 0])
    assert abs(got - want) <= abs(want) * 2.0 ** -8


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(1)
    g = rng.uniform(-6, 6, 5000)
    u = rng.uniform(-3, 3, 5000)
    da = rng.uniform(-2, 2, 5000)
    dg, du = sw.swiglu_grads_exact(g, u, da)
    h = 1e-6
    fd_g = (sw.swiglu_exact(g + h, u) - sw.swiglu_exact(g - h, u)) / (2 * h) * da
    fd_u = (sw.swiglu_exact(g, u + h) - sw.swiglu_exact(g, u - h)) / (2 * h) * da
    assert np.max(np.abs(dg - fd_g)) < 1e-7 * (1 + np.max(np.abs(dg)))
    assert np.max(np.abs(du - fd_u)) < 1e-7 * (1 + np.max(np.abs(du)))


@pytest.mark.parametrize("which", ["fwd", "bwd"])
def test_brute_force_layout(which):
    rng = np.random.default_rng(2)
    R, F = 3, 5
    h1 = to_bits(rng.standard_normal((R, 2 * F)).astype(np.float32))
    da2 = to_bits(rng.standard_normal((R, F)).astype(np.float32))
    hv = oracle.bf16_to_f32(h1).astype(np.float64)
    dv = oracle.bf16_to_f32(da2).astype(np.float64)
    if which == "fwd":
        got = oracle.bf16_to_f32(sw.swiglu_fwd(h1, F))
        for r in range(R):
            for c in range(F):
                gg, uu = hv[r, c], hv[r, F + c]
                want = gg / (1.0 + math.exp(-gg)) * uu
                assert abs(got[r, c] - want) <= abs(want) * 2.0 ** -8 + 1e-30
    else:
        got = oracle.bf16_to_f32(sw.swiglu_bwd(da2, h1, F))
        for r in range(R):
            for c in range(F):
                gg, uu, d = hv[r, c], hv[r, F + c], dv[r, c]
                s = 1.0 / (1.0 + math.exp(-gg))
                wg = d * uu * s * (1.0 + gg * (1.0 - s))
                wu = d * gg * s
                assert abs(got[r, c] - wg) <= abs(wg) * 2.0 ** -8 + 1e-30
                assert abs(got[r, F + c] - wu) <= abs(wu) * 2.0 ** -8 + 1e-30


def test_quantized_forms_are_the_rowwise_recipe():
    rng = np.random.default_rng(3)
    R, F = 6, 16
    h1 = to_bits(rng.standard_normal((R, 2 * F)).astype(np.float32))
    da2 = to_bits((rng.standard_normal((R, F)) * 1e-3).astype(np.float32))
    for codec in (oracle.E4M3FN, oracle.E4M3FNUZ):
        a2, q, s = sw.swiglu_quantize_rowwise(h1, F, codec)
        q2, s2 = oracle.quantize_rowwise(a2, codec)
        assert np.array_equal(q, q2) and np.array_equal(s, s2)
        # every code decodes to within half a step of a2 * s (the rowwise recipe's bound)
        dec = oracle.decode(q, codec) / s[:, None]
        assert np.all(np.abs(dec) <= np.abs(oracle.bf16_to_f32(a2)).max(axis=1, keepdims=True) * (1 + 2 ** -3))
        dh1, qb, sb = sw.swiglu_backward_quantize_rowwise(da2, h1, F, codec)
        assert dh1.shape == (R, 2 * F) and qb.shape == (R, 2 * F) and sb.shape == (R,)
