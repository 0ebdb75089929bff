"""Blockwise FP8 scaling: one fp32 scale per fixed tile, and the grouped GEMM
over blockwise-scaled operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages list blockwise scaling (a scale per fixed-size tile) between rowwise
and MXFP8, and name blockwise kernels for MI300/MI350 [P4 "Скейлы: от тензора
до микроблока"; P3, the four scaling strategies], without the tile shape.
Readings, also in the design notes:
  B1  tiles: 1 x 128 (along the contraction) for activations, 128 x 128 for
      weights; the last tile of a row or column range may be partial.
  B2  each tile follows the rowwise recipe (S1-S4 of oracle.quant) with the
      tile's elements as the reduction set: s = fmax / max(amax, eps).
  B3  GROUPED_M: out[m, n] = sum over 128-wide contraction blocks kb of
      (exact dot of the codes over kb) / (sa[m, kb] * sb[e, n // 128, kb]),
      e the group of row m.
"""
from __future__ import annotations

import numpy as np

from .codec import decode
from .quant import _apply_clamp_cast, _scale_from_amax, bf16_to_f32, group_bounds

BLOCK = 128


def quantize_blockwise(x_bits: np.ndarray, block_rows: int, codec: int):
    """x [B, R, C] bf16 -> (q [B, R, C] u8, s [B, ceil(R/block_rows), ceil(C/128)] f32) (B1, B2)."""
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    B, R, C = x.shape
    nr, nc = -(-R // block_rows), -(-C // BLOCK)
    q = np.zeros((B, R, C), np.uint8)
    s = np.zeros((B, nr, nc), np.float32)
    for b in range(B):
        for i in range(nr):
            for j in range(nc):
                tile = x[b, i * block_rows:(i + 1) * block_rows, j * BLOCK:(j + 1) * BLOCK]
                amax = np.abs(tile).max() if tile.size else np.float32(0.0)
                s[b, i, j] = _scale_from_amax(np.asarray([amax], np.float32), codec)[0]
                q[b, i * block_rows:(i + 1) * block_rows, j * BLOCK:(j + 1) * BLOCK] = \
                    _apply_clamp_cast(tile, s[b, i, j], codec)
    return q, s


def mm_grouped_m_blockwise(qa, sa, qb, sb, offs, a_codec: int, b_codec: int) -> np.ndarray:
    """B3.  qa [M, K] u8, sa [M, KB], qb [E, N, K] u8, sb [E, NB, KB] -> [M, N] float64
    (NaN on rows outside every group)."""
    M, K = qa.shape
    E, N, _ = qb.shape
    KB = -(-K // BLOCK)
    A = decode(qa, a_codec)
    out = np.full((M, N), np.nan)
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        Bm = decode(qb[e], b_codec)
        acc = np.zeros((hi[e] - lo[e], N))
        for kb in range(KB):
            ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
            dot = A[lo[e]:hi[e], ks] @ Bm[:, ks].T                    # exact: FP8 products summed in fp64
            col_scale = np.repeat(sb[e][:, kb].astype(np.float64), BLOCK)[:N]
            acc += dot / (sa[lo[e]:hi[e], kb].astype(np.float64)[:, None] * col_scale[None, :])
        out[lo[e]:hi[e]] = acc
    return out


def dequantize_blockwise(q, s, block_rows: int, codec: int) -> np.ndarray:
    """q [B, R, C] u8, s [B, nr, nc] -> the values q / s as float64 (for error bounds)."""
    B, R, C = q.shape
    sf = np.repeat(np.repeat(s.astype(np.float64), block_rows, axis=1), BLOCK, axis=2)[:, :R, :C]
    return decode(q, codec) / sf
