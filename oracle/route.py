"""MoE routing around the grouped GEMMs: token slots grouped by expert into
offsets (optionally padded per group), the rows gathered into that grouped
layout, and the expert outputs combined back per token.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The grouped GEMMs take their rows already grouped by expert, with an
offsets tensor splitting them [P1 Details (the grouped GEMM over an offsets
tensor); P4 "MoE" (tokens routed to experts, grouped GEMMs over the routed
rows); P2 Details (groups padded to the MX block size)].  Readings the pages
leave open, stated here and in the design notes:
  * Slot i = t * topk + j is token t's j-th expert choice.  Within an expert
    the slots keep their slot order (a stable grouping).
  * Each group's row count may be rounded up to a multiple of `pad` (1: no
    padding); padding rows hold zeros and come after the group's rows.
  * An expert id outside [0, E) drops the slot: it is not counted, its
    destination is -1 and it contributes nothing to the combine.
  * combine: y[t] = sum over j = 0 .. topk-1, in that order, of
    w[t, j] * yg[dest[t, j]], each product and each sum an IEEE fp32
    operation (round to nearest), then rounded once to bf16.  Without
    weights every weight is 1 (the backward's sum of the routed copies'
    input gradients).
  * combine's backward, for the loss gradient dy [T, C]: a grouped row r
    holding slot s = src[r] of token t = s // topk receives
    dyg[r] = w[s] * dy[t] (one fp32 product rounded to bf16, as the
    forward's products; zeros for padding rows), and the router weight
    receives dw[s] = <dy[t], yg[dest[s]]> (0 for a dropped slot).  The pages
    fix no precision for dw; it is an fp32 accumulation in the kernel and the
    exact sum here, and tests accept it within fp32 summation error.
"""
from __future__ import annotations

import numpy as np

from .quant import EPS, bf16_to_f32
from .codec import FMAX
from .swiglu import round_bf16


def rows_bound(slots: int, n_experts: int, pad: int) -> int:
    """Most grouped rows a routing can need: every slot plus pad - 1 per group."""
    return slots + n_experts * (pad - 1)


def route(expert_ids: np.ndarray, n_experts: int, pad: int = 1):
    """expert_ids [T, k] -> (counts [E], offs [E] inclusive padded cumsum, dest [T*k], src [rows_bound]).
    src[r] is the slot whose row lands at grouped row r, -1 for padding and unused rows."""
    ids = np.asarray(expert_ids, dtype=np.int64).ravel()
    S = ids.size
    valid = (ids >= 0) & (ids < n_experts)
    counts = np.bincount(ids[valid], minlength=n_experts).astype(np.int64)
    padded = (counts + pad - 1) // pad * pad
    offs = np.cumsum(padded)
    start = offs - padded
    dest = np.full(S, -1, dtype=np.int64)
    order = np.argsort(np.where(valid, ids, n_experts), kind="stable")   # valid slots by expert, slot order kept
    first = np.concatenate([[0], np.cumsum(counts)])
    for e in range(n_experts):
        slots = order[first[e]:first[e + 1]]
        dest[slots] = start[e] + np.arange(counts[e])
    src = np.full(rows_bound(S, n_experts, pad), -1, dtype=np.int64)
    src[dest[valid]] = np.nonzero(valid)[0]
    return (counts.astype(np.int32), offs.astype(np.int32), dest.astype(np.int32), src.astype(np.int32))


def permute(x_bits: np.ndarray, src: np.ndarray, topk: int) -> np.ndarray:
    """x [T, C] bf16 -> xg [len(src), C] bf16: row r is x[src[r] // topk], zeros where src[r] < 0."""
    x = np.asarray(x_bits, dtype=np.uint16)
    src = np.asarray(src, dtype=np.int64)
    out = np.zeros((src.size, x.shape[1]), dtype=np.uint16)
    used = src >= 0
    out[used] = x[src[used] // topk]
    return out


def permute_quantized(q: np.ndarray, s: np.ndarray, src: np.ndarray, topk: int, codec: int):
    """Rowwise-quantized tokens q [T, C] u8, s [T] f32 -> (qg [len(src), C] u8, sg [len(src)] f32): row r
    is token src[r] // topk's codes and scale; a padding row gets zero codes and the scale the rowwise
    recipe gives an all-zero row, fmax / eps.  Quantizing before the gather moves one byte per element
    instead of two, for the T token rows instead of the topk*T grouped rows; with the padding rows
    defined this way it gives the same bits as quantizing the gathered bf16 rows."""
    q = np.asarray(q, dtype=np.uint8)
    src = np.asarray(src, dtype=np.int64)
    used = src >= 0
    qg = np.zeros((src.size, q.shape[1]), dtype=np.uint8)
    qg[used] = q[src[used] // topk]
    sg = np.full(src.size, np.float32(np.float32(FMAX[codec]) / EPS), dtype=np.float32)
    sg[used] = np.asarray(s, dtype=np.float32)[src[used] // topk]
    return qg, sg


def combine(yg_bits: np.ndarray, dest: np.ndarray, weights, tokens: int, topk: int) -> np.ndarray:
    """yg [rows, C] bf16, dest [T*k], weights [T, k] fp32 or None (all 1) -> y [T, C] bf16 (the fp32 order
    above)."""
    yg = bf16_to_f32(np.asarray(yg_bits, dtype=np.uint16))
    dest = np.asarray(dest, dtype=np.int64).reshape(tokens, topk)
    if weights is None:
        weights = np.ones((tokens, topk), dtype=np.float32)
    w = np.asarray(weights, dtype=np.float32).reshape(tokens, topk)
    acc = np.zeros((tokens, yg.shape[1]), dtype=np.float32)
    for j in range(topk):
        d = dest[:, j]
        ok = d >= 0
        term = np.zeros_like(acc)
        term[ok] = w[ok, j][:, None] * yg[d[ok]]          # fp32 products (numpy: IEEE, round to nearest)
        acc = np.where(ok[:, None], acc + term, acc)       # fp32 sums in slot order
    return round_bf16(acc.astype(np.float64))


def combine_backward(dy_bits: np.ndarray, yg_bits: np.ndarray, src: np.ndarray, dest: np.ndarray,
                     weights: np.ndarray, tokens: int, topk: int):
    """Backward of combine (the reading above).  dy [T, C] bf16, yg [rows, C] bf16 (the forward's expert
    outputs), src [rows_out] and dest [T*k] from route, weights [T, k] fp32 ->
    (dyg [rows_out, C] bf16 bits, dw [T*k] fp64)."""
    dy = bf16_to_f32(np.asarray(dy_bits, dtype=np.uint16))
    yg = bf16_to_f32(np.asarray(yg_bits, dtype=np.uint16)).astype(np.float64)
    src = np.asarray(src, dtype=np.int64)
    dest = np.asarray(dest, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float32).reshape(-1)
    S = tokens * topk
    used = (src >= 0) & (src < S)
    s = src[used]
    prod = np.zeros((src.size, dy.shape[1]), dtype=np.float32)
    prod[used] = w[s][:, None] * dy[s // topk]             # fp32 products, round to nearest
    dyg = round_bf16(prod.astype(np.float64))
    dw = np.zeros(S, dtype=np.float64)
    ok = (dest >= 0) & (dest < yg.shape[0])
    slots = np.nonzero(ok)[0]
    dw[slots] = np.einsum("sc,sc->s", dy[slots // topk].astype(np.float64), yg[dest[slots]])
    return dyg, dw
