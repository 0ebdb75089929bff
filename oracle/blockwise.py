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
  B4  for the weight gradient, which contracts over tokens, both token-major
      operands take 1 x 128 tiles along the tokens (one scale per column and
      128-token block); the blocks restart at every group start, so a block
      never spans two experts, and the last block of a group may be partial.
  B5  GROUPED_K: out[e, n, k] = sum over the token blocks tb of group e of
      (exact dot over tb) / (sa[tb, n] * sb[tb, k]).
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


def token_blocks(offs, M: int):
    """The 128-token blocks of the groups, restarting at each group start: a list of (group, lo, hi)
    in group order (B4)."""
    lo, hi = group_bounds(offs, M)
    out = []
    for e in range(lo.size):
        for t0 in range(int(lo[e]), int(hi[e]), BLOCK):
            out.append((e, t0, min(t0 + BLOCK, int(hi[e]))))
    return out


def quantize_blockwise_tokens(x_bits: np.ndarray, offs, codec: int, ld_q: int | None = None, q_init=None):
    """B4: x [M, C] bf16 (token-major) -> (q_t phys [C, ld_q] u8, s [TB, C] f32), one scale per column
    and 128-token block of a group (blocks restart at each group start); codes transposed as the
    colwise quantizer lays them out; tokens of no group are left as in q_init."""
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    M, C = x.shape
    ld_q = M if ld_q is None else ld_q
    q = np.zeros((C, ld_q), np.uint8) if q_init is None else np.array(q_init, dtype=np.uint8, copy=True)
    blocks = token_blocks(offs, M)
    s = np.zeros((len(blocks), C), np.float32)
    for i, (_, t0, t1) in enumerate(blocks):
        xb = x[t0:t1]
        s[i] = _scale_from_amax(np.abs(xb).max(axis=0), codec)
        q[:, t0:t1] = _apply_clamp_cast(xb, s[i][None, :], codec).T
    return q, s


def mm_grouped_k_blockwise(qa_t, sa, qb_t, sb, offs, a_codec: int, b_codec: int) -> np.ndarray:
    """B5, GROUPED_K: qa_t phys [N, M], sa [TB, N], qb_t phys [K, M], sb [TB, K] -> [E, N, K] float64:
    per group, the sum over its token blocks of (exact dot over the block) / (sa[tb, n] * sb[tb, k])."""
    N, M = qa_t.shape
    K = qb_t.shape[0]
    E = len(offs)
    A = decode(qa_t, a_codec)
    B = decode(qb_t, b_codec)
    out = np.zeros((E, N, K))
    for tb, (e, t0, t1) in enumerate(token_blocks(offs, M)):
        dot = A[:, t0:t1] @ B[:, t0:t1].T
        out[e] += dot / (sa[tb].astype(np.float64)[:, None] * sb[tb].astype(np.float64)[None, :])
    return out
