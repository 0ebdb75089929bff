"""Grouped GEMM references for forward, dgrad and wgrad.

TEST INFRASTRUCTURE ONLY (see the package header).

Each linear layer runs three GEMMs: forward, the gradient w.r.t. the input
(dgrad) and the gradient w.r.t. the weight (wgrad).  [P3 "Az AMD
FP8-formátumának támogatása"; P4 "Что такое FP8-обучение".]  In an MoE layer
the 2D routed activations meet 3D per-expert weights through a group-offsets
tensor, with per-row activation scales and per-expert column weight scales.
[P1 Details, MoE paragraph; P4 "MoE: почему DeepSeek-V3 ломал пайплайн";
P2 Details, MoE forward diagram.]  wgrad contracts over the token dimension.
[P2 Details, contracting-dimension note.]

Two grouping modes:
  GROUPED_M (fwd, dgrad): out[m, n] = sum_k A[m, k] * B[e, n, k] for m in group e.
  GROUPED_K (wgrad):      out[e, n, k] = sum_{m in group e} A[n, m] * B[k, m].

Operands are the dequantized values: dec(q) / s for fp32 multiplier scales,
dec(q) * 2**X for e8m0 block scales, the exact value for bf16.  Each
dequantized FP8 value is exact in fp64.  With fp32 scales the kernel's
product of the raw codes, sum dec(a)*dec(b), is exact in fp64 for every
contraction length used here (each e4m3fn product is a multiple of 2**-18 below
2**18; each e4m3fnuz product a multiple of 2**-20 below 2**16; fewer than 2**17
terms fit in 53 bits), so the reference computes that exact sum with a
library matmul and then divides by sa*sb in fp64.  With e8m0 scales, each
32-wide block partial is exact and the scaled sum has relative error below
2**-53 * n.

Readings: S13 groups (see ``quant.group_bounds``); GROUPED_M leaves rows that
fall in no group unwritten (NaN in the reference); GROUPED_K writes exact zeros
for an empty group; S19 the kernel output is bf16 by default.
"""
from __future__ import annotations

import numpy as np

from .codec import decode, e8m0_decode
from .quant import bf16_to_f32, group_bounds

__all__ = ["group_bounds", "mm_grouped_m", "mm_grouped_k", "mm_grouped_m_mx",
           "mm_grouped_k_mx", "mm_grouped_k_bf16", "error_bounds_m", "error_bounds_k",
           "ACC_FP32", "ACC_FP8_MFMA"]


def mm_grouped_m(qa, sa, qb, sb, offs, a_codec: int, b_codec: int) -> np.ndarray:
    """GROUPED_M with fp32 multiplier scales.

    qa [M, K] u8, sa [M] f32, qb [E, N, K] u8, sb [E, N] f32 -> [M, N] float64
    (NaN on rows outside every group).
    """
    M, K = qa.shape
    E, N, Kb = qb.shape
    assert Kb == K
    A = decode(qa, a_codec)
    out = np.full((M, N), np.nan)
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        B = decode(qb[e], b_codec)                               # [N, K]
        dot = A[lo[e]:hi[e]] @ B.T                               # exact sum of exact products
        out[lo[e]:hi[e]] = dot / (sa[lo[e]:hi[e]].astype(np.float64)[:, None]
                                  * sb[e].astype(np.float64)[None, :])
    return out


def mm_grouped_k(qa_t, sa, qb_t, sb, offs, a_codec: int, b_codec: int) -> np.ndarray:
    """GROUPED_K with fp32 multiplier scales.

    qa_t phys [N, M] u8, sa [E, N], qb_t phys [K, M] u8, sb [E, K] -> [E, N, K] float64.
    """
    N, M = qa_t.shape
    K, Mb = qb_t.shape
    assert Mb == M
    E = sa.shape[0]
    out = np.zeros((E, N, K))
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        A = decode(qa_t[:, lo[e]:hi[e]], a_codec)               # [N, Me]
        B = decode(qb_t[:, lo[e]:hi[e]], b_codec)               # [K, Me]
        out[e] = (A @ B.T) / (sa[e].astype(np.float64)[:, None] * sb[e].astype(np.float64)[None, :])
    return out


def _mx_dequant_lastdim(q, sc):
    """q [..., C] e4m3fn codes, sc [..., C/32] e8m0 -> fp64 values dec(q) * 2**X."""
    v = decode(q, 0)
    f = e8m0_decode(sc)
    return v * np.repeat(f, 32, axis=-1)


def mm_grouped_m_mx(qa, xa, qb, xb, offs) -> np.ndarray:
    """GROUPED_M with e8m0 block scales along K.

    qa [M, K], xa [M, K/32], qb [E, N, K], xb [E, N, K/32] -> [M, N] float64.
    """
    M, K = qa.shape
    E, N, _ = qb.shape
    A = _mx_dequant_lastdim(qa, xa)
    out = np.full((M, N), np.nan)
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        B = _mx_dequant_lastdim(qb[e], xb[e])
        out[lo[e]:hi[e]] = A[lo[e]:hi[e]] @ B.T
    return out


def mm_grouped_k_mx(qa_t, xa, qb_t, xb, offs_pad) -> np.ndarray:
    """GROUPED_K with e8m0 block scales along the (padded) token dim.

    qa_t phys [N, Mp], xa [N, Mp/32], qb_t phys [K, Mp], xb [K, Mp/32],
    offs_pad [E] (multiples of 32) -> [E, N, K] float64.
    """
    N, Mp = qa_t.shape
    K, _ = qb_t.shape
    E = len(offs_pad)
    A = _mx_dequant_lastdim(qa_t, xa)
    B = _mx_dequant_lastdim(qb_t, xb)
    out = np.zeros((E, N, K))
    lo, hi = group_bounds(offs_pad, Mp)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        out[e] = A[:, lo[e]:hi[e]] @ B[:, lo[e]:hi[e]].T
    return out


def mm_grouped_k_bf16(a_bits, b_bits, offs) -> np.ndarray:
    """GROUPED_K on unquantized bf16, token-major operands (the recipe that keeps
    the weight-gradient GEMM in BF16 [P1 Details, Figure 1 "+GW" bar; P3
    "Gyorsulás sűrű és MoE-modelleken"; P4 FAQ on which scaling to start with]).

    a [M, N] bf16, b [M, K] bf16 -> [E, N, K] float64 (bf16 products are exact in fp64).
    """
    A = bf16_to_f32(a_bits).astype(np.float64)
    B = bf16_to_f32(b_bits).astype(np.float64)
    M, N = A.shape
    K = B.shape[1]
    E = len(offs)
    out = np.zeros((E, N, K))
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        out[e] = A[lo[e]:hi[e]].T @ B[lo[e]:hi[e]]
    return out


# ------------------------------------------------------------ acceptance bounds

# Relative accumulation error allowed by the diagnostic bound, per unit of sum|a*b|:
#  * "fp32": sequential IEEE fp32 accumulation of exact products, K * 2**-23.
#  * "fp8_mfma": 2**-10.  The FP8 matrix-core instructions add the products of
#    one instruction with less than fp32 precision (measured on gfx950 over
#    these tests: |err| / sum|a*b| at most about 1.4e-4 = 2**-12.8); 2**-10
#    leaves a margin and is still about 1000x below the error of a dropped
#    term or a wrong scale.  By Cauchy-Schwarz, sum|a*b| <= |a||b|, so this
#    diagnostic is always tighter than the 1e-2 |a||b| contract bound.
ACC_FP32 = "fp32"
ACC_FP8_MFMA = "fp8_mfma"


def _bounds(Ad, Bd, K_eff, acc):
    """Contract bound 1e-2*|a_row|*|b_col| and the tighter diagnostic
    2**-8*|ref| + rel_acc*sum|a*b| for dense dequantized Ad [m, K], Bd [n, K]."""
    na = np.sqrt((Ad * Ad).sum(axis=1))
    nb = np.sqrt((Bd * Bd).sum(axis=1))
    contract = 1e-2 * na[:, None] * nb[None, :]
    absdot = np.abs(Ad) @ np.abs(Bd).T
    ref = Ad @ Bd.T
    rel = max(K_eff, 1) * 2.0 ** -23 if acc == ACC_FP32 else 2.0 ** -10
    tight = 2.0 ** -8 * np.abs(ref) + rel * absdot
    return contract, tight


def error_bounds_m(A_deq, B_deq, offs, acc=ACC_FP32):
    """Per-element bounds for GROUPED_M given dequantized A [M, K] and B [E, N, K]."""
    M, K = A_deq.shape
    E, N, _ = B_deq.shape
    contract = np.full((M, N), np.nan)
    tight = np.full((M, N), np.nan)
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        c, t = _bounds(A_deq[lo[e]:hi[e]], B_deq[e], K, acc)
        contract[lo[e]:hi[e]] = c
        tight[lo[e]:hi[e]] = t
    return contract, tight


def error_bounds_k(A_deq_t, B_deq_t, offs, acc=ACC_FP32):
    """Per-element bounds for GROUPED_K given dequantized A phys [N, M] and B phys [K, M]
    (group scales already applied per column range)."""
    N, M = A_deq_t.shape
    K = B_deq_t.shape[0]
    E = len(offs)
    contract = np.zeros((E, N, K))
    tight = np.zeros((E, N, K))
    lo, hi = group_bounds(offs, M)
    for e in range(E):
        if hi[e] == lo[e]:
            continue
        c, t = _bounds(A_deq_t[:, lo[e]:hi[e]], B_deq_t[:, lo[e]:hi[e]], int(hi[e] - lo[e]), acc)
        contract[e] = c
        tight[e] = t
    return contract, tight
