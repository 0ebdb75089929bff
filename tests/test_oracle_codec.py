"""Pins for the oracle's FP8 / e8m0 codecs (CPU only).

The oracle is checked against things other than itself: torch's independent
float8 dtypes (decode of all 256 codes, RNE casts of clamped values), closed
forms (largest finite values, smallest subnormals), two independent encoders,
monotonicity and round trips, and a pure-Python search for the MX exponent.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3FN, E4M3FNUZ

TORCH_DT = {E4M3FN: torch.float8_e4m3fn, E4M3FNUZ: torch.float8_e4m3fnuz}


def torch_decode(codec):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(TORCH_DT[codec]).to(torch.float64).numpy()


def torch_encode(y32: np.ndarray, codec) -> np.ndarray:
    """torch's fp32 -> float8 cast (round to nearest even; does not saturate,
    so callers pass values already inside [-fmax, fmax])."""
    return torch.from_numpy(np.ascontiguousarray(y32, np.float32)).to(TORCH_DT[codec]).view(torch.uint8).numpy()


@pytest.mark.parametrize("codec", [E4M3FN, E4M3FNUZ])
def test_decode_table_matches_torch(codec):
    ours = oracle.decode_table(codec)
    ref = torch_decode(codec)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])


def test_nan_codes_and_limits():
    fn, fnuz = oracle.decode_table(E4M3FN), oracle.decode_table(E4M3FNUZ)
    assert set(np.flatnonzero(np.isnan(fn))) == {0x7F, 0xFF}
    assert set(np.flatnonzero(np.isnan(fnuz))) == {0x80}
    # the largest finite values: 240 is printed in the e4m3fnuz property table; 448 is OCP e4m3
    assert np.nanmax(fn) == 448.0 == oracle.FMAX[E4M3FN] == torch.finfo(torch.float8_e4m3fn).max
    assert np.nanmax(fnuz) == 240.0 == oracle.FMAX[E4M3FNUZ] == torch.finfo(torch.float8_e4m3fnuz).max
    assert fn[0x7E] == 448.0 and fnuz[0x7F] == 240.0
    # smallest subnormals 2^-9 and 2^-10; zero codes
    assert fn[1] == 2.0 ** -9 and fnuz[1] == 2.0 ** -10
    assert fn[0] == 0.0 and math.copysign(1.0, fn[0x80]) == -1.0 and fn[0x80] == 0.0
    assert fnuz[0] == 0.0


def _midpoint_probes(codec):
    """All midpoints between consecutive magnitudes, +-1 fp32 ulp, both signs, plus the codes."""
    mags = oracle.decode_table(codec)[: (0x7E if codec == E4M3FN else 0x7F) + 1]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)          # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    vals = np.concatenate([mids, up, dn, mags.astype(np.float32)])
    vals = vals[np.abs(vals) <= oracle.FMAX[codec]]
    return np.concatenate([vals, -vals]).astype(np.float32)


@pytest.mark.parametrize("codec", [E4M3FN, E4M3FNUZ])
def test_encode_midpoints_match_torch(codec):
    y = _midpoint_probes(codec)
    ref = torch_encode(y, codec)
    assert np.array_equal(oracle.encode_nearest(y, codec), ref)
    assert np.array_equal(oracle.encode_arith(y, codec), ref)


@pytest.mark.parametrize("codec", [E4M3FN, E4M3FNUZ])
def test_encoders_agree_on_fp32_sweep(codec):
    """Strided sweep over every fp32 bit pattern in [0, fmax] (both signs).
    FP8MOE_EXHAUSTIVE=1 makes it every pattern (minutes)."""
    fm_bits = int(np.float32(oracle.FMAX[codec]).view(np.uint32))
    step = 1 if os.environ.get("FP8MOE_EXHAUSTIVE") == "1" else 9973
    chunk = 1 << 24
    for start in range(0, fm_bits + 1, chunk * step):
        bits = np.arange(start, min(start + chunk * step, fm_bits + 1), step, dtype=np.uint32)
        y = bits.view(np.float32)
        for s in (y, -y):
            a = oracle.encode_nearest(s, codec)
            b = oracle.encode_arith(s, codec)
            assert np.array_equal(a, b)
    # and against torch on a random sample of the same range
    rng = np.random.default_rng(7)
    bits = rng.integers(0, fm_bits + 1, size=200_000, dtype=np.uint32)
    y = bits.view(np.float32) * np.where(rng.random(bits.size) < 0.5, -1, 1).astype(np.float32)
    assert np.array_equal(oracle.encode(y, codec), torch_encode(y, codec))


@pytest.mark.parametrize("codec", [E4M3FN, E4M3FNUZ])
def test_encode_roundtrip_and_monotone(codec):
    tab = oracle.decode_table(codec)
    finite = np.flatnonzero(~np.isnan(tab))
    v = tab[finite].astype(np.float32)
    q = oracle.encode(v, codec)
    assert np.array_equal(oracle.decode(q, codec), tab[finite])
    # monotone: sorted inputs decode to a non-decreasing sequence
    y = np.sort(np.random.default_rng(3).uniform(-oracle.FMAX[codec], oracle.FMAX[codec], 100_000)).astype(np.float32)
    d = oracle.decode(oracle.encode(y, codec), codec)
    assert np.all(np.diff(d) >= 0)
    # round to nearest: the chosen value is no farther than any other finite value
    err = np.abs(d - y.astype(np.float64))
    mags = np.unique(np.abs(tab[finite]))
    idx = np.searchsorted(mags, np.abs(y.astype(np.float64)))
    lo = mags[np.clip(idx - 1, 0, mags.size - 1)]
    hi = mags[np.clip(idx, 0, mags.size - 1)]
    best = np.minimum(np.abs(np.abs(y) - lo), np.abs(np.abs(y) - hi))
    assert np.all(err <= best)


def test_encode_spot_values_and_signed_zero():
    assert oracle.encode(np.float32([232.0, 432.0, 7.5 * 2 ** -9]), E4M3FN).tolist() == [0x76, 0x7E, 0x08]
    assert oracle.encode(np.float32([232.0, 7.5 * 2 ** -10]), E4M3FNUZ).tolist() == [0x7E, 0x08]
    tiny = np.float32([-1e-30, -0.0, 0.0])
    assert oracle.encode(tiny, E4M3FN).tolist() == [0x80, 0x80, 0x00]
    assert oracle.encode(tiny, E4M3FNUZ).tolist() == [0x00, 0x00, 0x00]
    # torch agrees on the sign of zero for both codecs
    assert torch_encode(tiny, E4M3FN).tolist() == [0x80, 0x80, 0x00]
    assert torch_encode(tiny, E4M3FNUZ).tolist() == [0x00, 0x00, 0x00]


def test_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        oracle.encode(np.float32([449.0]), E4M3FN)
    with pytest.raises(ValueError):
        oracle.encode(np.float32([241.0]), E4M3FNUZ)


def test_e8m0_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = oracle.e8m0_decode(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[:255], ref[:255])


def _floor_rule_py(amax: float) -> int:
    if amax == 0.0:
        return -127
    return max(-127, min(127, math.floor(math.log2(amax)) - 8))


def _ceil_rule_py(amax: float) -> int:
    if amax == 0.0:
        return -127
    X = -127
    while amax * 2.0 ** -X > 448.0:      # smallest X that keeps the block inside +-448
        X += 1
    return X


def test_mx_exponent_rules_brute_force():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F7FFFFF, size=4000, dtype=np.uint32)
    vals = list(bits.view(np.float32).astype(np.float64))
    vals += [0.0, 50.0, 60.0, 1.76, 448.0, 449.0, 2.0 ** -130, 2.0 ** -149, 1.75, 1.75 * 2 ** 10,
             float(np.nextafter(np.float32(1.75), np.float32(2.0)))]
    vals += [2.0 ** k for k in range(-149, 128)]
    amax = np.array(vals, dtype=np.float64)
    Xf = oracle.mx_shared_exponent(amax, oracle.MX_FLOOR_OCP)
    Xc = oracle.mx_shared_exponent(amax, oracle.MX_CEIL)
    assert [int(v) for v in Xf] == [_floor_rule_py(a) for a in vals]
    assert [int(v) for v in Xc] == [_ceil_rule_py(a) for a in vals]
    # examples: amax 50 -> code 124 both; 60 -> floor 124, ceil 125; 1.76 -> 119/120;
    # 448 -> 127 both; 449 -> 127/128; 2^-130 -> code 0
    ex = np.array([50.0, 60.0, 1.76, 448.0, 449.0, 2.0 ** -130])
    assert (oracle.mx_shared_exponent(ex, 0) + 127).tolist() == [124, 124, 119, 127, 127, 0]
    assert (oracle.mx_shared_exponent(ex, 1) + 127).tolist() == [124, 125, 120, 127, 128, 0]


# ------------------------------------------------------- planted mistakes
# Each plausible mistake in the encoder must fail one of the pins above.

def _ties_away(y, codec):
    q = oracle.encode_nearest(y, codec)
    tab = oracle.decode_table(codec)
    a = np.abs(np.asarray(y, np.float64))
    d = np.abs(tab[q])
    bump = (a > d) & (np.isin(a, ((tab[:-1] + tab[1:]) / 2)))
    return np.where(bump, q + 1, q).astype(np.uint8)


def _fnuz_signed_zero(y, codec):
    q = oracle.encode_nearest(y, codec)
    return np.where(np.signbit(y), q | 0x80, q).astype(np.uint8)


@pytest.mark.parametrize("mutant,codec", [(_ties_away, E4M3FN), (_ties_away, E4M3FNUZ),
                                          (_fnuz_signed_zero, E4M3FNUZ)])
def test_planted_encoder_mistakes_are_caught(mutant, codec):
    y = _midpoint_probes(codec)
    y = np.concatenate([y, np.float32([-1e-30, -0.0])])
    assert not np.array_equal(mutant(y, codec), torch_encode(y, codec))
