"""Pins of the tensorwise oracle (oracle/tensorwise.py) against things other
than itself: the rowwise quantizer on a one-row view (a special case the
recipe reduces to), closed-form scales and codes, the all-zero tensor, the
invariance of the codes under a split into rows of equal maxima, and a
pure-Python transposition."""
import numpy as np
import pytest

import oracle
from oracle import tensorwise as tw
from oracle.swiglu import round_bf16

CODECS = [oracle.E4M3FN, oracle.E4M3FNUZ]


def bits(rng, shape, scale=1.0):
    return round_bf16(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("codec", CODECS)
def test_equals_rowwise_on_one_row(codec):
    """A tensor viewed as one row: tensorwise must give the rowwise quantizer's codes and scale."""
    rng = np.random.default_rng(0)
    x = bits(rng, (37, 24), 3.0)
    q, s = tw.quantize_tensorwise(x, codec)
    qr, sr = oracle.quantize_rowwise(x.reshape(1, -1), codec)
    assert np.array_equal(q.reshape(1, -1), qr)
    assert np.float32(s).view(np.uint32) == sr[0].view(np.uint32)


@pytest.mark.parametrize("codec", CODECS)
def test_closed_form_scale_and_extremes(codec):
    """amax = 2 exactly: s = fmax / 2; +-2 map to the largest finite codes, 0 to the zero code."""
    x = np.zeros((3, 8), np.float64)
    x[0, 1], x[2, 5], x[1, 3] = 2.0, -2.0, 0.5
    q, s = tw.quantize_tensorwise(round_bf16(x), codec)
    fmax = oracle.FMAX[codec]
    assert s == np.float32(fmax / 2.0)
    top = oracle.encode(np.float32([fmax, -fmax]), codec)
    assert q[0, 1] == top[0] and q[2, 5] == top[1]
    assert q[1, 3] == oracle.encode(np.float32([fmax / 4.0]), codec)[0]
    assert q[0, 0] == oracle.encode(np.float32([0.0]), codec)[0]


@pytest.mark.parametrize("codec", CODECS)
def test_all_zero_and_empty(codec):
    """No nonzero element: the eps floor, s = fmax / 1e-12, and zero codes."""
    q, s = tw.quantize_tensorwise(np.zeros((4, 16), np.uint16), codec)
    assert s == np.float32(np.float32(oracle.FMAX[codec]) / np.float32(1e-12))
    assert np.all(q == oracle.encode(np.float32([0.0]), codec)[0])
    q0, s0 = tw.quantize_tensorwise(np.zeros((0, 16), np.uint16), codec)
    assert q0.shape == (0, 16) and s0 == s


def test_rowwise_agrees_when_every_row_has_the_tensor_max():
    """If every row's max equals the tensor's max, rowwise and tensorwise coincide row by row."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 40))
    x[np.arange(9), rng.integers(0, 40, 9)] = 7.5 * rng.choice([-1.0, 1.0], 9)
    xb = round_bf16(x)
    q, s = tw.quantize_tensorwise(xb, oracle.E4M3FN)
    qr, sr = oracle.quantize_rowwise(xb, oracle.E4M3FN)
    assert np.array_equal(q, qr) and np.all(sr == s)


def test_scale_is_the_coarser_one():
    """One outlier: the tensorwise scale equals the smallest rowwise scale (the outlier's row)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 64))
    x[5, 9] = 300.0
    xb = round_bf16(x)
    _, s = tw.quantize_tensorwise(xb, oracle.E4M3FN)
    _, sr = oracle.quantize_rowwise(xb, oracle.E4M3FN)
    assert s == sr.min() == sr[5]


def test_transposed_layout_loops():
    rng = np.random.default_rng(3)
    B, R, C, LD = 2, 5, 8, 9
    x = bits(rng, (B, R, C))
    init = np.full((B, C, LD), 0xA5, np.uint8)
    qt, s = tw.quantize_tensorwise_transposed(x, oracle.E4M3FN, ld_q=LD, q_init=init)
    q, s2 = tw.quantize_tensorwise(x, oracle.E4M3FN)
    assert s == s2
    for b in range(B):
        for c in range(C):
            for r in range(LD):
                want = q[b, r, c] if r < R else 0xA5
                assert qt[b, c, r] == want
