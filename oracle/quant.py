"""Dynamic FP8 quantization: absmax -> scale -> apply -> clamp -> cast.

TEST INFRASTRUCTURE ONLY (see the package header).

The step order is the one the pages give for the fused quantization kernels:
a row or column absolute maximum, the scale derived from it, the scale
applied, the result clipped, then cast to FP8.  [P3 "A Triton-kernelok
csökkentették a kvantálás költségét"; P4 "Три уровня оптимизации
Triton-ядер"; P1 glossary entry on Triton kernel fusion.]

Granularities: one scale per row (activations, and expert weights viewed as
[E*N, K] so that each expert output column n of W_e^T gets its own scale), one
scale per (group, column) for the backward operands that contract over tokens,
and one e8m0 scale per 1x32 block for MXFP8.  [P1 Details, MoE paragraph:
expert weight column scales, activation row scales, routing offsets; P4 "MoE:
почему DeepSeek-V3 ломал пайплайн"; P4 "Скейлы: от тензора до микроблока";
P2 Details, MXFP8 layout diagram and the wgrad contracting-dimension note.]

Readings (the pages give no formula, epsilon, rounding mode or layout):
  S1  the fp32 scale is a multiplier, s = fmax / max(amax, eps), stored as is.
  S2  the division is IEEE fp32 round-to-nearest-even.
  S3  eps = fp32(1e-12): an all-zero or empty reduction set gets s = fmax/eps.
  S4  y = fp32(x * s) rounded once, then clamped to [-fmax, fmax], then encoded
      (round-to-nearest-even): two roundings, in that order.
  S10 no flush of subnormals anywhere (bf16 inputs or fp32 intermediates).
  S12 colwise outputs are written transposed: 2D [M, C] -> phys [C, M]
      (ld_q >= M bytes per column); 3D [E, R, C] -> phys [E, C, R].
  S13 group e covers rows [hi_{e-1}, hi_e) where hi_e is the running maximum
      of offs clamped to [0, M] (hi_{-1} = 0): groups are disjoint, a
      decreasing entry yields an empty group, and rows past the last group
      are not written.
  S17 MX along rows restarts blocks at every group start, pads each group to a
      multiple of 32 rows with zero codes (the pad counts as +0 in the block
      maximum) and lays the groups out back to back at padded offsets; the
      columns past the last padded group, up to the caller's allocation, get
      data 0x00 and scale 0x00.
"""
from __future__ import annotations

import numpy as np

from .codec import FMAX, E4M3FN, encode, mx_shared_exponent

EPS = np.float32(1e-12)


def _assert_ieee_subnormals() -> None:
    tiny = np.float32(2.0 ** -140)
    if not (tiny * np.float32(1.0)) > 0 or not (np.float32(2.0 ** -126) / np.float32(4.0)) > 0:
        raise RuntimeError("numpy runs with flush-to-zero/denormals-are-zero; the oracle needs IEEE subnormals")


_assert_ieee_subnormals()


def bf16_to_f32(x_bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _scale_from_amax(amax_f32: np.ndarray, codec: int) -> np.ndarray:
    """S1-S3: s = fp32(fmax) / max(amax, eps), IEEE fp32 division."""
    a = np.maximum(amax_f32.astype(np.float32), EPS)
    with np.errstate(over="raise", divide="raise", invalid="raise"):
        return (np.float32(FMAX[codec]) / a).astype(np.float32)


def _apply_clamp_cast(x32: np.ndarray, s32: np.ndarray, codec: int) -> np.ndarray:
    """S4: y = fp32(x*s), clamp to [-fmax, fmax], then round to the nearest FP8 code."""
    with np.errstate(over="ignore"):
        y = (x32 * s32).astype(np.float32)
    fm = np.float32(FMAX[codec])
    y = np.minimum(np.maximum(y, -fm), fm)
    return encode(y, codec)


def group_bounds(offs, M: int):
    """S13: (lo, hi) int64 arrays of the disjoint row range of each group."""
    o = np.clip(np.asarray(offs, dtype=np.int64), 0, M)
    hi = np.maximum.accumulate(o) if o.size else o
    lo = np.concatenate([np.zeros(1, dtype=np.int64), hi[:-1]]) if o.size else o
    return lo, hi


# ----------------------------------------------------------------- rowwise

def quantize_rowwise(x_bits: np.ndarray, codec: int):
    """One scale per row over the last dim.  x [R, C] bf16 -> q [R, C] u8, s [R] f32."""
    x = bf16_to_f32(x_bits)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = _scale_from_amax(amax, codec)
    q = _apply_clamp_cast(x, s[:, None], codec)
    return q, s


# ----------------------------------------------------------------- colwise

def quantize_colwise_grouped(x_bits: np.ndarray, offs, codec: int, q_init=None, ld_q=None):
    """One scale per (group, column) over the group's rows; output transposed.

    x [M, C] bf16, offs [E] int32 -> q phys [C, ld_q] u8 (ld_q >= M, default M),
    s [E, C] f32.  Rows outside every group are left as in ``q_init``.
    """
    x = bf16_to_f32(x_bits)
    M, C = x.shape
    ld_q = M if ld_q is None else ld_q
    q = np.zeros((C, ld_q), np.uint8) if q_init is None else q_init.copy()
    lo, hi = group_bounds(offs, M)
    E = lo.size
    s = np.empty((E, C), np.float32)
    for e in range(E):
        xe = x[lo[e]:hi[e]]                        # [Me, C]
        amax = np.abs(xe).max(axis=0) if xe.shape[0] else np.zeros(C, np.float32)
        s[e] = _scale_from_amax(amax, codec)
        q[:, lo[e]:hi[e]] = _apply_clamp_cast(xe, s[e][None, :], codec).T
    return q, s


def quantize_colwise_batched(x_bits: np.ndarray, codec: int):
    """Per batch item (expert) e and column c, one scale over the R rows.

    x [E, R, C] bf16 -> q phys [E, C, R] u8, s [E, C] f32.
    """
    x = bf16_to_f32(x_bits)
    E, R, C = x.shape
    amax = np.abs(x).max(axis=1) if R else np.zeros((E, C), np.float32)   # [E, C]
    s = _scale_from_amax(amax, codec)
    q = _apply_clamp_cast(x, s[:, None, :], codec)                      # [E, R, C]
    return np.ascontiguousarray(q.transpose(0, 2, 1)), s


# ----------------------------------------------------------------- MXFP8

def _mx_blocks(xb32: np.ndarray, rule: int):
    """Quantize blocks laid out along the last axis (size 32).

    xb32 [..., 32] fp32 -> codes [..., 32] u8 (e4m3fn), e8m0 [...] u8.
    """
    amax = np.abs(xb32).max(axis=-1)
    X = mx_shared_exponent(amax, rule)                 # int64
    inv = np.ldexp(np.float32(1.0), -X).astype(np.float32)   # 2**-X, exact in fp32
    q = _apply_clamp_cast(xb32, inv[..., None], E4M3FN)
    return q, (X + 127).astype(np.uint8)


def quantize_mx_lastdim(x_bits: np.ndarray, rule: int):
    """1x32 blocks along the last dim.  x [R, C] (C % 32 == 0) -> q [R, C], e8m0 [R, C/32]."""
    x = bf16_to_f32(x_bits)
    R, C = x.shape
    assert C % 32 == 0
    q, sc = _mx_blocks(x.reshape(R, C // 32, 32), rule)
    return q.reshape(R, C), sc


def quantize_mx_rows_batched(x_bits: np.ndarray, rule: int):
    """32x1 blocks along rows, per batch item.  x [E, R, C] (R % 32 == 0) ->
    q phys [E, C, R], e8m0 phys [E, C, R/32]."""
    x = bf16_to_f32(x_bits)
    E, R, C = x.shape
    assert R % 32 == 0
    xt = np.ascontiguousarray(x.transpose(0, 2, 1))            # [E, C, R]
    q, sc = _mx_blocks(xt.reshape(E, C, R // 32, 32), rule)
    return q.reshape(E, C, R), sc


def mx_rows_bound(rows: int, n_groups: int) -> int:
    """Host-known upper bound of the padded row count: round_up(rows + 31*E, 32)."""
    return ((rows + 31 * n_groups + 31) // 32) * 32


def quantize_mx_rows_grouped(x_bits: np.ndarray, offs, rule: int, rows_pad: int):
    """32x1 blocks along rows restarting at each group, groups padded to 32 (S17).

    x [M, C] bf16 -> q phys [C, rows_pad] u8, e8m0 phys [C, rows_pad/32] u8,
    offs_pad [E] int32 (inclusive cumulative padded row counts).
    """
    x = bf16_to_f32(x_bits)
    M, C = x.shape
    assert rows_pad % 32 == 0
    lo, hi = group_bounds(offs, M)
    E = lo.size
    q = np.zeros((C, rows_pad), np.uint8)
    sc = np.zeros((C, rows_pad // 32), np.uint8)
    offs_pad = np.zeros(E, np.int32)
    p = 0
    for e in range(E):
        me = int(hi[e] - lo[e])
        mp = (me + 31) // 32 * 32
        if p + mp > rows_pad:
            raise ValueError("rows_pad is smaller than the padded group total")
        if mp:
            blk = np.zeros((C, mp), np.float32)                 # +0 pad
            blk[:, :me] = x[lo[e]:hi[e]].T
            qe, se = _mx_blocks(blk.reshape(C, mp // 32, 32), rule)
            q[:, p:p + mp] = qe.reshape(C, mp)
            sc[:, p // 32:(p + mp) // 32] = se
        p += mp
        offs_pad[e] = p
    return q, sc, offs_pad
