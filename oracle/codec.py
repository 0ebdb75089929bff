"""FP8 e4m3fn / e4m3fnuz and e8m0 codecs, from their bit layouts.

TEST INFRASTRUCTURE ONLY (see the package header).

Formats
-------
* e4m3fn (OCP 8-bit float, the format the pages call NVIDIA's): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; subnormals when the exponent
  field is 0; codes 0x7F/0xFF are NaN; there is no infinity; zero is signed.
  Largest finite magnitude 448 (code 0x7E).  [P4 "FNUZ" section: e4m3fn has a
  different maximum than e4m3fnuz; 448 is the OCP specification's value.]
* e4m3fnuz (AMD Instinct): the same field widths with exponent bias 8, largest
  finite magnitude 240 (code 0x7F), no NaN or infinity among the finite codes,
  and a single unsigned zero.  [P1 "AMD FP8 format in TorchAO" evidence
  bullet, e4m3fnuz property table; P1 glossary entry "FNUZ"; P3 "Az AMD
  FP8-formátumának támogatása"; P4 "Тихая порча градиентов: проблема формата
  FNUZ".]  Reading: code 0x80 (the would-be negative zero) decodes to NaN, the
  library convention; the encoder below never emits it, so every encoded
  output is NaN-free as the pages state.
* e8m0 (MX shared scale): 8-bit unsigned exponent, value 2**(code - 127),
  code 0xFF is NaN.  One code per 1x32 block of e4m3 data.  [P2 Details,
  MXFP8 data/scale layout diagram.]

Encoding is round-to-nearest, ties to the even code (mantissa LSB 0), of a
value already clamped to [-fmax, fmax] (the saturating clamp precedes the
cast; [P4 "Три уровня оптимизации Triton-ядер": absmax, scale, clip, cast]).
Two independent encoders are provided; the tests require them to agree.
"""
from __future__ import annotations

import numpy as np

E4M3FN = 0
E4M3FNUZ = 1

# Largest finite magnitudes.  240 is printed in [P1]'s e4m3fnuz property table
# and in [P3]/[P4]'s FNUZ sections; 448 is the OCP e4m3 value.
FMAX = {E4M3FN: 448.0, E4M3FNUZ: 240.0}

_BIAS = {E4M3FN: 7, E4M3FNUZ: 8}
# Largest magnitude code (positive half): fn reserves 0x7F for NaN.
_TOP_CODE = {E4M3FN: 0x7E, E4M3FNUZ: 0x7F}

MX_FLOOR_OCP = 0
MX_CEIL = 1


def _check_codec(codec: int) -> None:
    if codec not in (E4M3FN, E4M3FNUZ):
        raise ValueError(f"unknown FP8 codec {codec}")


def decode_table(codec: int) -> np.ndarray:
    """Value of each of the 256 codes as float64 (NaN codes -> nan)."""
    _check_codec(codec)
    bias = _BIAS[codec]
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0:
            mag = (m / 8.0) * 2.0 ** (1 - bias)
        else:
            mag = (1.0 + m / 8.0) * 2.0 ** (e - bias)
        out[c] = sign * mag
    if codec == E4M3FN:
        out[0x7F] = np.nan
        out[0xFF] = np.nan
    else:
        out[0x80] = np.nan
    return out


def decode(q: np.ndarray, codec: int) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return decode_table(codec)[np.asarray(q, dtype=np.uint8)]


def _magnitudes(codec: int) -> np.ndarray:
    """Representable magnitudes in increasing code order, codes 0.._TOP_CODE."""
    return decode_table(codec)[: _TOP_CODE[codec] + 1]


def _apply_sign(mag_code: np.ndarray, y: np.ndarray, codec: int) -> np.ndarray:
    neg = np.signbit(y)
    if codec == E4M3FN:
        # signed zero: a negative input keeps its sign bit even when it rounds to 0
        sign = np.where(neg, 0x80, 0)
    else:
        # unsigned zero: the sign bit is set only on a non-zero magnitude
        sign = np.where(neg & (mag_code != 0), 0x80, 0)
    return (mag_code | sign).astype(np.uint8)


def encode_nearest(y, codec: int) -> np.ndarray:
    """Encoder A: nearest representable magnitude by search over the midpoints.

    ``y`` must already lie in [-fmax, fmax] (finite).  Works in float64, in
    which every fp32 input and every midpoint between two FP8 values is exact.
    """
    _check_codec(codec)
    y = np.asarray(y)
    a = np.abs(y.astype(np.float64))
    if np.any(a > FMAX[codec]) or np.any(~np.isfinite(a)):
        raise ValueError("encode expects finite values clamped to [-fmax, fmax]")
    mags = _magnitudes(codec)
    mids = (mags[:-1] + mags[1:]) / 2.0
    idx = np.searchsorted(mids, a, side="left")      # count of midpoints strictly below a
    at_mid = (idx < mids.size) & (mids[np.minimum(idx, mids.size - 1)] == a)
    # at a midpoint between codes idx and idx+1, take the even one
    idx = np.where(at_mid & (idx % 2 == 1), idx + 1, idx)
    return _apply_sign(idx.astype(np.int64), y, codec)


def encode_arith(y, codec: int) -> np.ndarray:
    """Encoder B: exponent/mantissa arithmetic with frexp and round-half-even."""
    _check_codec(codec)
    y = np.asarray(y)
    a = np.abs(y.astype(np.float64))
    if np.any(a > FMAX[codec]) or np.any(~np.isfinite(a)):
        raise ValueError("encode expects finite values clamped to [-fmax, fmax]")
    bias = _BIAS[codec]
    min_normal = 2.0 ** (1 - bias)
    quantum_sub = 2.0 ** (1 - bias - 3)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < min_normal
    # subnormal range: integer multiple of the subnormal step (8 -> the smallest normal)
    code[sub] = np.rint(a[sub] / quantum_sub).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        frac, ex = np.frexp(a[nrm])          # a = frac * 2**ex, frac in [0.5, 1)
        e_unb = ex.astype(np.int64) - 1      # a = sig * 2**e_unb, sig in [1, 2)
        sig = frac * 2.0
        mant = np.rint((sig - 1.0) * 8.0).astype(np.int64)
        carry = mant == 8
        mant = np.where(carry, 0, mant)
        e_unb = np.where(carry, e_unb + 1, e_unb)
        code[nrm] = ((e_unb + bias) << 3) | mant
    return _apply_sign(code, y, codec)


encode = encode_nearest


def e8m0_decode(code) -> np.ndarray:
    """e8m0 code -> float64 scale 2**(code-127); 0xFF -> nan."""
    c = np.asarray(code, dtype=np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 0xFF, np.nan, out)


def mx_shared_exponent(amax, rule: int) -> np.ndarray:
    """Shared block exponent X (int64, in [-127, 127]) from a block's |x| max.

    [P2 Details, MXFP8 data/scale layout diagram] fixes only e4m3 data with one
    e8m0 scale per 1x32 block.  Readings:
      * MX_FLOOR_OCP (default): X = floor(log2 amax) - 8, the OCP MX rule for
        e4m3 elements (8 = exponent of e4m3fn's largest normal binade);
        elements above 448 * 2**X saturate in the clamp.
      * MX_CEIL: the smallest X with amax * 2**-X <= 448 (no element clips).
      * amax == 0 -> X = -127 (code 0).  X is clamped to [-127, 127].
    """
    a = np.asarray(amax, dtype=np.float64)
    frac, ex = np.frexp(a)                   # a = frac * 2**ex
    e = ex.astype(np.int64) - 1              # floor(log2 a) for a > 0
    if rule == MX_FLOOR_OCP:
        X = e - 8
    elif rule == MX_CEIL:
        X = e - 8 + (frac * 2.0 > 1.75).astype(np.int64)
    else:
        raise ValueError(f"unknown MX rule {rule}")
    X = np.where(a == 0.0, -127, X)
    return np.clip(X, -127, 127)
