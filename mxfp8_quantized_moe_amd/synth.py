"""Seeded synthetic inputs for the five MoE/dense workloads.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no step of the quantization or GEMM arithmetic: it only draws random
numbers, rounds them to bf16 storage and builds routing offsets.

Recipe
------
* Generator: ``numpy.random.Generator(PCG64(seed))``; values are
  ``standard_normal(shape, float32) * sigma`` (sigma is a standard deviation).
* Outliers: after the normals, ``mask = random(shape) < frac`` and masked values
  are multiplied by ``factor``.
* fp32 -> bf16 by round-to-nearest-even on the bit pattern (inputs are finite).
* Tensor seed = 100*cfg + t with t in {0: X, 1: W1/W, 2: W2, 3: dY, 4: A2, 5: dH1,
  6: token rows X of the full MoE layer, 7: its output gradient dY, 8: router logits};
  3D weights draw each expert from seed 1000*(100*cfg + t) + e so they can be
  generated one expert at a time.
* Rows are generated already grouped by expert; ``offs`` is the inclusive
  cumulative sum of per-expert row counts (int32).

The shapes and value distributions follow the layers the pages measure
(Llama3-8B linear, DeepSeek-MoE-16B and DeepSeek-V3 expert layers, Llama4-Scout
MXFP8 experts); the synthetic tensors stand in for the real activations,
weights and gradients, which are not available.
"""
from __future__ import annotations

import dataclasses
import numpy as np

T_X, T_W1, T_W2, T_DY, T_A2, T_DH1, T_XT, T_DYT, T_RW = 0, 1, 2, 3, 4, 5, 6, 7, 8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(seed: int, shape, sigma: float, outlier_frac: float = 0.0,
                outlier_factor: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, sigma) values with an optional outlier fraction."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(sigma)
    if outlier_frac > 0.0:
        mask = rng.random(shape) < outlier_frac
        x[mask] *= np.float32(outlier_factor)
    return f32_to_bf16_bits(x)


def expert_weights_bf16(base_seed: int, n_experts: int, rows: int, cols: int,
                        sigma: float) -> np.ndarray:
    """[E, rows, cols] bf16 bits; expert e is drawn from seed 1000*base_seed + e (experts are
    independent streams, drawn on several host threads; the values do not depend on that)."""
    import concurrent.futures as cf
    out = np.empty((n_experts, rows, cols), dtype=np.uint16)

    def one(e):
        out[e] = normal_bf16(1000 * base_seed + e, (rows, cols), sigma)

    with cf.ThreadPoolExecutor(min(8, max(n_experts, 1))) as ex:
        list(ex.map(one, range(n_experts)))
    return out


# ---------------------------------------------------------------- routing

def routing_counts(cfg: int) -> np.ndarray:
    """Per-expert routed row counts for workload ``cfg`` (1..5), int64."""
    rng = np.random.Generator(np.random.PCG64(cfg))
    if cfg == 1:
        return rng.multinomial(512, [1 / 3, 1 / 3, 0.0, 1 / 3]).astype(np.int64)
    if cfg == 2:
        return np.array([8192], dtype=np.int64)
    if cfg == 3:
        # 64 experts, Zipf(1.1) popularity over a random rank order, 8192 tokens
        # each routed to 6 distinct experts (Gumbel top-k sampling without replacement).
        rank = rng.permutation(64) + 1
        p = rank.astype(np.float64) ** -1.1
        p /= p.sum()
        g = rng.gumbel(size=(8192, 64))
        top = np.argsort(-(np.log(p)[None, :] + g), axis=1)[:, :6]
        return np.bincount(top.ravel(), minlength=64).astype(np.int64)
    if cfg == 4:
        # 32 local experts, Zipf(1.2) over a random rank order, the two least
        # popular ranks forced empty, 8192 routed rows.
        rank = rng.permutation(32) + 1
        p = rank.astype(np.float64) ** -1.2
        p[rank >= 31] = 0.0
        p /= p.sum()
        return rng.multinomial(8192, p).astype(np.int64)
    if cfg == 5:
        return rng.multinomial(16384, [1 / 16] * 16).astype(np.int64)
    raise ValueError(f"unknown workload {cfg}")


def routing_ids(cfg: int):
    """Per-token expert ids [tokens, topk] (int32) whose per-expert counts are
    routing_counts(cfg): config 3 keeps its Gumbel top-6 draw; configs 4 and 5
    place their multinomial counts on 8192 (16384) tokens with one expert each,
    in a seeded random token order."""
    if cfg == 3:
        rng = np.random.Generator(np.random.PCG64(cfg))
        rank = rng.permutation(64) + 1
        p = rank.astype(np.float64) ** -1.1
        p /= p.sum()
        g = rng.gumbel(size=(8192, 64))
        return np.argsort(-(np.log(p)[None, :] + g), axis=1)[:, :6].astype(np.int32)
    if cfg in (4, 5):
        counts = routing_counts(cfg)
        ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
        rng = np.random.Generator(np.random.PCG64(10_000 + cfg))
        return rng.permutation(ids).reshape(-1, 1).astype(np.int32)
    raise ValueError(f"per-token routing is generated for configs 3, 4 and 5, not {cfg}")


def tokens_topk(cfg: int):
    """(tokens, experts per token) of the MoE workloads' routing."""
    return {3: (8192, 6), 4: (8192, 1), 5: (16384, 1)}[cfg]


def router_weights(cfg: int) -> np.ndarray:
    """Router weights [tokens, topk] (fp32) of a token's chosen experts, from N(0, 1) logits (seed
    100*cfg + 8): a softmax over the chosen experts' logits when topk > 1, the sigmoid of the
    logit with one expert per token (fp64 arithmetic, rounded once to fp32)."""
    T, k = tokens_topk(cfg)
    rng = np.random.Generator(np.random.PCG64(tensor_seed(cfg, T_RW)))
    z = rng.standard_normal((T, k))
    if k == 1:
        p = 1.0 / (1.0 + np.exp(-z))
    else:
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def offsets_from_counts(counts) -> np.ndarray:
    return np.cumsum(np.asarray(counts, dtype=np.int64)).astype(np.int32)


def random_counts(seed: int, total: int, n_groups: int, empty_frac: float = 0.25) -> np.ndarray:
    """Ragged per-group counts summing to ``total`` with some forced-empty groups (edge-case tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.random(n_groups) + 0.05
    p[rng.random(n_groups) < empty_frac] = 0.0
    if p.sum() == 0.0:
        p[-1] = 1.0
    p /= p.sum()
    return rng.multinomial(total, p).astype(np.int64)


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    E: int            # experts (1 for the dense layer)
    H: int            # hidden size (contraction dim of the first GEMM)
    F2: int           # output size of W1 (2x the expert FFN for fused gate/up)
    F: int            # contraction dim of W2 (0: no W2 in this workload)
    M: int            # routed rows
    x_outliers: tuple
    mx: bool = False

    @property
    def counts(self) -> np.ndarray:
        return routing_counts(self.cfg)

    @property
    def offs(self) -> np.ndarray:
        return offsets_from_counts(self.counts)


WORKLOADS = {
    1: Workload(1, "tiny-moe-4x512x256", E=4, H=256, F2=512, F=0, M=512, x_outliers=(0.01, 50.0)),
    2: Workload(2, "llama3-8b-linear-8192x14336x4096", E=1, H=4096, F2=14336, F=0, M=8192,
                x_outliers=(0.001, 100.0)),
    3: Workload(3, "deepseek-moe-16b-64e-2048x1408", E=64, H=2048, F2=2816, F=1408, M=49152,
                x_outliers=(0.0, 1.0)),
    4: Workload(4, "deepseek-v3-share-32e-7168x2048", E=32, H=7168, F2=4096, F=2048, M=8192,
                x_outliers=(0.005, 50.0)),
    5: Workload(5, "llama4-scout-mxfp8-16e-5120x8192", E=16, H=5120, F2=16384, F=8192, M=16384,
                x_outliers=(0.01, 30.0), mx=True),
}


def tensor_seed(cfg: int, t: int) -> int:
    return 100 * cfg + t


def make_x(w: Workload) -> np.ndarray:
    return normal_bf16(tensor_seed(w.cfg, T_X), (w.M, w.H), 1.0, *w.x_outliers)


def make_a2(w: Workload) -> np.ndarray:
    return normal_bf16(tensor_seed(w.cfg, T_A2), (w.M, w.F), 1.0, *w.x_outliers)


def make_dy(w: Workload) -> np.ndarray:
    # Gradient w.r.t. the layer output: [M, F2] for the dense layer, [M, H] for MoE layers.
    cols = w.F2 if w.F == 0 else w.H
    return normal_bf16(tensor_seed(w.cfg, T_DY), (w.M, cols), 1e-3)


def make_dh1(w: Workload) -> np.ndarray:
    return normal_bf16(tensor_seed(w.cfg, T_DH1), (w.M, w.F2), 1e-3)


def make_tokens(w: Workload) -> np.ndarray:
    """Token rows entering the full MoE layer: [tokens, H], the activation recipe of X."""
    T, _ = tokens_topk(w.cfg)
    return normal_bf16(tensor_seed(w.cfg, T_XT), (T, w.H), 1.0, *w.x_outliers)


def make_dy_tokens(w: Workload) -> np.ndarray:
    """Gradient of the full MoE layer's output: [tokens, H], N(0, 1e-3)."""
    T, _ = tokens_topk(w.cfg)
    return normal_bf16(tensor_seed(w.cfg, T_DYT), (T, w.H), 1e-3)


def make_w1(w: Workload) -> np.ndarray:
    """[E, F2, H] (dense layer: [1, F2, H])."""
    if w.E == 1:
        return normal_bf16(tensor_seed(w.cfg, T_W1), (w.F2, w.H), 0.02)[None]
    return expert_weights_bf16(tensor_seed(w.cfg, T_W1), w.E, w.F2, w.H, 0.02)


def make_w2(w: Workload) -> np.ndarray:
    """[E, H, F]."""
    return expert_weights_bf16(tensor_seed(w.cfg, T_W2), w.E, w.H, w.F, 0.02)
