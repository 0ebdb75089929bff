"""SwiGLU between the two expert GEMMs and its backward, each followed by the
rowwise FP8 quantization of its output.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests,
smoke() and bench's CPU baseline, never by the product path.

The MoE expert MLP applies W1, the SwiGLU activation, then W2; the
activation's output is what the W2 GEMM quantizes, and in the backward the
gradient of W1's output is what the W1 dgrad quantizes [P1 Details (the MoE
layer's grouped GEMMs and their quantized operands); P4 "MoE" (routed experts
between two grouped GEMMs)].  Readings the pages leave open, stated here and
in the design notes:
  * W1's 2F outputs per row are the gate projection (columns [0, F)) followed
    by the up projection (columns [F, 2F)); the activation is
    silu(gate) * up with silu(g) = g * sigmoid(g).
  * The activation and both gradients are bf16 tensors: the exact value of
    each element, rounded once to bf16 (round to nearest, ties to even).
  * Their FP8 form is the rowwise recipe of the existing quantizer over that
    bf16 tensor (one scale per row).
Backward, from the product rule: with s = sigmoid(g),
  d gate = dA * up * s * (1 + g * (1 - s)),   d up = dA * g * s.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_to_f32, quantize_rowwise


def _sigmoid(g: np.ndarray) -> np.ndarray:
    """fp64 logistic function, written so neither branch overflows."""
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns, rounded once to the nearest bf16 value
    (ties to even).  Finite results only (the inputs here stay far below the
    bf16 maximum)."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()                             # zeros keep their sign
    nz = x != 0
    m, e = np.frexp(x[nz])                     # x = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits for normal values (exponent >= -125 in
    # frexp's convention) and a fixed 2^-133 spacing below.
    e_eff = np.maximum(e, -125)
    scaled = np.ldexp(x[nz], 8 - e_eff)         # exact: a power-of-two scaling
    out[nz] = np.ldexp(np.rint(scaled), e_eff - 8)   # rint: half to even
    if not np.all(np.isfinite(out)) or np.any(np.abs(out) > 3.3895313892515355e38):
        raise ValueError("round_bf16: value outside the finite bf16 range")
    f32 = out.astype(np.float32)               # exact: a bf16 value is an fp32 value
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def split_gate_up(h1_bits: np.ndarray, F: int):
    """h1 [R, 2F] bf16 -> (gate, up) as fp64 [R, F] each."""
    h = bf16_to_f32(np.asarray(h1_bits, dtype=np.uint16)).astype(np.float64)
    if h.shape[-1] != 2 * F:
        raise ValueError("h1 must have 2F columns")
    return h[..., :F], h[..., F:]


def swiglu_exact(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u in fp64."""
    return g * _sigmoid(g) * u


def swiglu_grads_exact(g: np.ndarray, u: np.ndarray, da: np.ndarray):
    """(d gate, d up) in fp64 for upstream gradient da of silu(g) * u."""
    s = _sigmoid(g)
    return da * u * s * (1.0 + g * (1.0 - s)), da * g * s


def swiglu_fwd(h1_bits: np.ndarray, F: int) -> np.ndarray:
    """A2 = bf16(silu(gate) * up): [R, 2F] bf16 -> [R, F] bf16 bits."""
    g, u = split_gate_up(h1_bits, F)
    return round_bf16(swiglu_exact(g, u))


def swiglu_bwd(da2_bits: np.ndarray, h1_bits: np.ndarray, F: int) -> np.ndarray:
    """dH1 = [bf16(d gate) | bf16(d up)]: dA2 [R, F], H1 [R, 2F] -> [R, 2F] bf16 bits."""
    g, u = split_gate_up(h1_bits, F)
    da = bf16_to_f32(np.asarray(da2_bits, dtype=np.uint16)).astype(np.float64)
    dg, du = swiglu_grads_exact(g, u, da)
    return np.concatenate([round_bf16(dg), round_bf16(du)], axis=-1)


def swiglu_quantize_rowwise(h1_bits: np.ndarray, F: int, codec: int):
    """(A2 bf16 bits, q, scale): the activation, then its rowwise FP8 form."""
    a2 = swiglu_fwd(h1_bits, F)
    q, s = quantize_rowwise(a2, codec)
    return a2, q, s


def swiglu_backward_quantize_rowwise(da2_bits: np.ndarray, h1_bits: np.ndarray, F: int, codec: int):
    """(dH1 bf16 bits, q, scale): the gradient of W1's output, then its rowwise FP8 form."""
    dh1 = swiglu_bwd(da2_bits, h1_bits, F)
    q, s = quantize_rowwise(dh1, codec)
    return dh1, q, s
