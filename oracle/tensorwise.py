"""Tensorwise FP8 quantization: one scale for the whole tensor.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The coarsest of the scaling granularities the pages list: a single scale for
a whole tensor, faster and coarser than one per row [P4 "Скейлы: от тензора до
микроблока"; P4 FAQ on which granularity to start with; P3, the four scaling
strategies TorchAO and TorchTitan support].  The pages give no formula for it;
the readings, also in the design notes:
  T1  the scale and the cast follow the rowwise recipe (S1-S4 of oracle.quant)
      with every element of the tensor as the one reduction set:
      s = fmax / max(amax, eps), y = fp32(x * s), clamp, encode.
  T2  the grouped GEMM takes the tensor's scale as its fp32 per-row /
      per-column scales with every entry equal, so its output is the rowwise
      epilogue's acc / (sa * sb) with scalar sa, sb.
  T3  the backward GEMMs take a transposed copy of the same codes (one scale,
      so the codes do not depend on the layout), laid out as the colwise
      quantizer's (S12): [B, R, C] -> phys [B, C, ld_q], ld_q >= R; bytes past
      R in each output row are left as they were.
"""
from __future__ import annotations

import numpy as np

from .quant import _apply_clamp_cast, _scale_from_amax, bf16_to_f32


def quantize_tensorwise(x_bits: np.ndarray, codec: int):
    """x bf16 of any shape -> (q u8 of the same shape, s f32 scalar) (T1)."""
    x = bf16_to_f32(x_bits)
    amax = np.abs(x).max() if x.size else np.float32(0.0)
    s = _scale_from_amax(np.asarray([amax], np.float32), codec)[0]
    return _apply_clamp_cast(x, s, codec), np.float32(s)


def quantize_tensorwise_transposed(x_bits: np.ndarray, codec: int, ld_q: int | None = None, q_init=None):
    """x [B, R, C] bf16 -> (q_t phys [B, C, ld_q] u8, s) (T3); q_t[b, c, r] = q[b, r, c] for r < R."""
    x = np.asarray(x_bits, dtype=np.uint16)
    B, R, C = x.shape
    ld_q = R if ld_q is None else ld_q
    q, s = quantize_tensorwise(x, codec)
    out = np.zeros((B, C, ld_q), np.uint8) if q_init is None else np.array(q_init, dtype=np.uint8, copy=True)
    out[:, :, :R] = q.transpose(0, 2, 1)
    return out, s
