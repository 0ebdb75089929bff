"""MI355X-native FP8 MoE quantization + grouped GEMM (thin Python binding).

Every function here marshals torch tensors to device pointers and calls the
C ABI of libfp8moe.so (include/fp8moe.h) on the current HIP stream; every step
of the computation runs in the library's HIP kernels.  Outputs not supplied
by the caller are allocated with torch (device memory plumbing only).  There is
no CPU or eager fallback: a missing library or a rejected argument raises.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (E4M3FN, E4M3FNUZ, MX_FLOOR_OCP, MX_CEIL, MX_LAYOUT_ROWS, MX_LAYOUT_K4, GROUPED_M, GROUPED_K,
                   OPD_E4M3FN, OPD_E4M3FNUZ, OPD_BF16, SCALE_F32, SCALE_E8M0, SCALE_NONE, SCALE_E8M0_K4,
                   OUT_BF16, OUT_F32,
                   Fp8MoeError)

__all__ = ["quantize_rowwise", "quantize_colwise", "quantize_mx", "quantize_mx_rows_bound",
           "grouped_mm_scaled", "encode_f32", "default_codec", "E4M3FN", "E4M3FNUZ", "MX_FLOOR_OCP",
           "MX_CEIL", "MX_LAYOUT_ROWS", "MX_LAYOUT_K4", "GROUPED_M", "GROUPED_K", "OPD_E4M3FN", "OPD_E4M3FNUZ",
           "OPD_BF16", "SCALE_F32", "SCALE_E8M0", "SCALE_NONE", "SCALE_E8M0_K4", "OUT_BF16", "OUT_F32",
           "mx_k4_shape", "quantize_mx_dual", "swiglu_quantize_mx_dual", "swiglu_backward_quantize_mx_dual",
           "moe_permute_quantize_mx_dual", "moe_permute_quantize_colwise",
           "Fp8MoeError", "swiglu_quantize_rowwise",
           "swiglu_backward_quantize_rowwise", "moe_route", "moe_route_noalloc", "moe_route_rows_bound", "moe_route_workspace_bytes", "moe_permute", "moe_combine",
           "moe_permute_rowwise", "moe_combine_backward",
           "quantize_tensorwise", "moe_permute_quantized", "quantize_blockwise", "grouped_mm_blockwise",
           "quantize_blockwise_tokens", "grouped_mm_blockwise_k"]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _bits(x: torch.Tensor) -> torch.Tensor:
    """bf16 tensors pass as their 16-bit patterns; int16/uint16 pass through."""
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError(f"expected bf16 (or its 16-bit pattern), got {x.dtype}")


def quantize_rowwise(x, codec=E4M3FN, q=None, scale=None, stream=None):
    """x [R, C] bf16 (row stride may exceed C) -> (q uint8 [R, C], scale f32 [R])."""
    x = _bits(x)
    R, C = x.shape
    if x.numel() and x.stride(1) != 1:
        raise ValueError("quantize_rowwise needs unit stride along the last dim")
    ld_x = x.stride(0) if x.numel() else C
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((R,), dtype=torch.float32, device=x.device) if scale is None else scale
    _lib.check("quantize_rowwise", _lib.lib().quantize_rowwise(
        _ptr(x), R, C, ld_x, codec, _ptr(q), _ptr(scale), _stream(stream)))
    return q, scale


def quantize_colwise(x, offs=None, codec=E4M3FN, q_t=None, scale=None, ld_q=None, stream=None):
    """Grouped 2D: x [M, C] + offs [E] -> (q_t uint8 phys [C, ld_q], scale [E, C]).
    Batched 3D: x [B, R, C] -> (q_t uint8 phys [B, C, ld_q], scale [B, C]).
    ld_q defaults to the row count rounded up to a multiple of 16 (the ABI's alignment)."""
    x = _bits(x).contiguous()
    if offs is not None:
        M, C = x.shape
        B, R, E = 1, M, offs.numel()
        ld_q = ld_q or (M + 15) // 16 * 16
        q_t = torch.empty((C, ld_q), dtype=torch.uint8, device=x.device) if q_t is None else q_t
        scale = torch.empty((E, C), dtype=torch.float32, device=x.device) if scale is None else scale
    else:
        B, R, C = x.shape
        E = 0
        ld_q = ld_q or (R + 15) // 16 * 16
        q_t = torch.empty((B, C, ld_q), dtype=torch.uint8, device=x.device) if q_t is None else q_t
        scale = torch.empty((B, C), dtype=torch.float32, device=x.device) if scale is None else scale
    _lib.check("quantize_colwise", _lib.lib().quantize_colwise(
        _ptr(x), B, R, C, _ptr(offs), E, codec, _ptr(q_t), ld_q, _ptr(scale), _stream(stream)))
    return q_t, scale


def moe_permute_quantize_colwise(x, src, topk, offs, weights=None, codec=E4M3FN, q_t=None, scale=None, ld_q=None,
                                 stream=None):
    """x bf16 [T, C] (token rows, or the output gradient dy), src int32 [R], offs int32 [E] from moe_route,
    weights f32 [T, topk] or None -> (q_t uint8 phys [C, ld_q], scale [E, C]): quantize_colwise of the gathered
    rows x[src[r] // topk] (times weights[src[r]] when given, rounded to bf16), which never go to memory."""
    x = _bits(x).contiguous()
    T, C = x.shape
    R, E = src.numel(), offs.numel()
    if weights is not None:
        weights = weights.contiguous()
        if weights.dtype != torch.float32 or weights.numel() != T * topk:
            raise ValueError("moe_permute_quantize_colwise: weights f32 [T, topk]")
    ld_q = ld_q or (R + 15) // 16 * 16
    q_t = torch.empty((C, ld_q), dtype=torch.uint8, device=x.device) if q_t is None else q_t
    scale = torch.empty((E, C), dtype=torch.float32, device=x.device) if scale is None else scale
    _lib.check("moe_permute_quantize_colwise", _lib.lib().moe_permute_quantize_colwise(
        _ptr(x), T, C, topk, _ptr(src), _ptr(weights), R, _ptr(offs), E, codec, _ptr(q_t), ld_q, _ptr(scale),
        _stream(stream)))
    return q_t, scale


def quantize_mx_rows_bound(rows: int, n_groups: int) -> int:
    return int(_lib.lib().quantize_mx_rows_bound(rows, n_groups))


def mx_k4_shape(rows: int, n_blocks: int):
    """Shape of an e8m0 scale matrix of `rows` rows and `n_blocks` 32-blocks per row in the K4
    layout: [ceil(n_blocks / 4), rows, 4]."""
    return ((n_blocks + 3) // 4, rows, 4)


def quantize_mx(x, axis=1, offs=None, rule=MX_FLOOR_OCP, rows_pad=None, q=None, scale=None,
                offs_pad=None, layout=MX_LAYOUT_ROWS, stream=None):
    """MXFP8.  axis=1: x [R, C] -> (q [R, C], e8m0 [R, C/32], None).
    axis=0 without offs: x [B, R, C] -> (q phys [B, C, R], e8m0 [B, C, R/32], None).
    axis=0 with offs: x [M, C] -> (q phys [C, rows_pad], e8m0 [C, rows_pad/32], offs_pad [E]).
    layout=MX_LAYOUT_K4: e8m0 in the K4 layout instead, shape mx_k4_shape(scale rows, blocks) with
    scale rows R (axis 1), B*C (axis 0 without offs), C (axis 0 with offs)."""
    x = _bits(x).contiguous()
    dev = x.device
    k4 = layout == MX_LAYOUT_K4

    def sc_empty(rows_major_shape, n_rows, n_blocks):
        shape = mx_k4_shape(n_rows, n_blocks) if k4 else rows_major_shape
        return torch.empty(shape, dtype=torch.uint8, device=dev)

    if axis == 1:
        C = x.shape[-1]
        R = x.numel() // max(C, 1)
        q = torch.empty(tuple(x.shape), dtype=torch.uint8, device=dev) if q is None else q
        scale = sc_empty(tuple(x.shape[:-1]) + (C // 32,), R, C // 32) if scale is None else scale
        st = _lib.lib().quantize_mx(_ptr(x), 1, R, C, 1, None, 0, rule, layout, _ptr(q), _ptr(scale), 0, None,
                                    _stream(stream))
        _lib.check("quantize_mx", st)
        return q, scale, None
    if offs is None:
        B, R, C = x.shape
        q = torch.empty((B, C, R), dtype=torch.uint8, device=dev) if q is None else q
        scale = sc_empty((B, C, R // 32), B * C, R // 32) if scale is None else scale
        st = _lib.lib().quantize_mx(_ptr(x), B, R, C, 0, None, 0, rule, layout, _ptr(q), _ptr(scale), R, None,
                                    _stream(stream))
        _lib.check("quantize_mx", st)
        return q, scale, None
    M, C = x.shape
    E = offs.numel()
    rows_pad = rows_pad or quantize_mx_rows_bound(M, E)
    q = torch.empty((C, rows_pad), dtype=torch.uint8, device=dev) if q is None else q
    scale = sc_empty((C, rows_pad // 32), C, rows_pad // 32) if scale is None else scale
    offs_pad = torch.empty((E,), dtype=torch.int32, device=dev) if offs_pad is None else offs_pad
    st = _lib.lib().quantize_mx(_ptr(x), 1, M, C, 0, _ptr(offs), E, rule, layout, _ptr(q), _ptr(scale), rows_pad,
                                _ptr(offs_pad), _stream(stream))
    _lib.check("quantize_mx", st)
    return q, scale, offs_pad


def quantize_mx_dual(x, offs=None, rule=MX_FLOOR_OCP, rows_pad=None, q=None, scale=None, q_t=None, scale_t=None,
                     offs_pad=None, layout=MX_LAYOUT_ROWS, stream=None):
    """Both MXFP8 forms from one read: (q, scale) as quantize_mx(x viewed [B*R, C], axis=1) and
    (q_t, scale_t, offs_pad) as quantize_mx(x, axis=0, offs).  x is [B, R, C] without offs, [M, C] with."""
    x = _bits(x).contiguous()
    dev = x.device
    k4 = layout == MX_LAYOUT_K4

    def sc_empty(rows_major_shape, n_rows, n_blocks):
        shape = mx_k4_shape(n_rows, n_blocks) if k4 else rows_major_shape
        return torch.empty(shape, dtype=torch.uint8, device=dev)

    if offs is None:
        B, R, C = x.shape
        E, rp, offs_pad = 0, R, None
        q_t = torch.empty((B, C, R), dtype=torch.uint8, device=dev) if q_t is None else q_t
        scale_t = sc_empty((B, C, R // 32), B * C, R // 32) if scale_t is None else scale_t
    else:
        (M, C), B = x.shape, 1
        R = M
        E = offs.numel()
        rp = rows_pad or quantize_mx_rows_bound(M, E)
        q_t = torch.empty((C, rp), dtype=torch.uint8, device=dev) if q_t is None else q_t
        scale_t = sc_empty((C, rp // 32), C, rp // 32) if scale_t is None else scale_t
        offs_pad = torch.empty((E,), dtype=torch.int32, device=dev) if offs_pad is None else offs_pad
    q = torch.empty((B * R, C), dtype=torch.uint8, device=dev) if q is None else q
    scale = sc_empty((B * R, C // 32), B * R, C // 32) if scale is None else scale
    st = _lib.lib().quantize_mx_dual(_ptr(x), B, R, C, _ptr(offs), E, rule, layout, _ptr(q), _ptr(scale), _ptr(q_t),
                                     _ptr(scale_t), rp, _ptr(offs_pad), _stream(stream))
    _lib.check("quantize_mx_dual", st)
    return q, scale, q_t, scale_t, offs_pad


def _mx_dual_outputs(R, C, offs, rows_pad, q, scale, q_t, scale_t, offs_pad, layout, dev):
    k4 = layout == MX_LAYOUT_K4
    E = offs.numel()
    rp = rows_pad or quantize_mx_rows_bound(R, E)
    sc_shape = lambda rows_major, n_rows, n_blocks: mx_k4_shape(n_rows, n_blocks) if k4 else rows_major
    q = torch.empty((R, C), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty(sc_shape((R, C // 32), R, C // 32), dtype=torch.uint8, device=dev) if scale is None else scale
    q_t = torch.empty((C, rp), dtype=torch.uint8, device=dev) if q_t is None else q_t
    scale_t = torch.empty(sc_shape((C, rp // 32), C, rp // 32), dtype=torch.uint8, device=dev) \
        if scale_t is None else scale_t
    offs_pad = torch.empty((E,), dtype=torch.int32, device=dev) if offs_pad is None else offs_pad
    return rp, q, scale, q_t, scale_t, offs_pad


def moe_permute_quantize_mx_dual(x, src, topk, offs, weights=None, rule=MX_FLOOR_OCP, rows_pad=None, xg=None,
                                 q=None, scale=None, q_t=None, scale_t=None, offs_pad=None, layout=MX_LAYOUT_K4,
                                 stream=None):
    """x bf16 [T, C] (token rows, or the output gradient dy), src int32 [R], offs int32 [E] from moe_route,
    weights f32 [T, topk] or None -> (xg or None, q [R, C], scale, q_t [C, rows_pad], scale_t, offs_pad): both
    MX forms of the gathered rows x[src[r] // topk] (times weights[src[r]] when given, rounded to bf16);
    xg (bf16 [R, C]) is written only if passed."""
    x = _bits(x).contiguous()
    T, C = x.shape
    R = src.numel()
    if weights is not None:
        weights = weights.contiguous()
        if weights.dtype != torch.float32 or weights.numel() != T * topk:
            raise ValueError("moe_permute_quantize_mx_dual: weights f32 [T, topk]")
    rp, q, scale, q_t, scale_t, offs_pad = _mx_dual_outputs(R, C, offs, rows_pad, q, scale, q_t, scale_t, offs_pad,
                                                            layout, x.device)
    _lib.check("moe_permute_quantize_mx_dual", _lib.lib().moe_permute_quantize_mx_dual(
        _ptr(x), T, C, topk, _ptr(src), _ptr(weights), R, _ptr(offs), offs.numel(), rule, layout, _ptr(xg), _ptr(q),
        _ptr(scale), _ptr(q_t), _ptr(scale_t), rp, _ptr(offs_pad), _stream(stream)))
    return xg, q, scale, q_t, scale_t, offs_pad


def swiglu_quantize_mx_dual(h1, offs, rule=MX_FLOOR_OCP, rows_pad=None, a2=None, q=None, scale=None, q_t=None,
                            scale_t=None, offs_pad=None, layout=MX_LAYOUT_K4, stream=None):
    """h1 [R, 2F] bf16 (gate | up), offs int32 [E] -> (a2 or None, q [R, F], scale, q_t [F, rows_pad], scale_t,
    offs_pad): both MX forms of bf16(silu(gate) * up); a2 (bf16 [R, F]) is written only if passed."""
    h1 = _bits(h1)
    R, F2 = h1.shape
    if F2 % 2 or (h1.numel() and h1.stride(1) != 1):
        raise ValueError("swiglu_quantize_mx_dual needs an even column count and unit column stride")
    F = F2 // 2
    ld = h1.stride(0) if h1.numel() else F2
    rp, q, scale, q_t, scale_t, offs_pad = _mx_dual_outputs(R, F, offs, rows_pad, q, scale, q_t, scale_t, offs_pad,
                                                            layout, h1.device)
    _lib.check("swiglu_quantize_mx_dual", _lib.lib().swiglu_quantize_mx_dual(
        _ptr(h1), R, F, ld, _ptr(offs), offs.numel(), rule, layout, _ptr(a2), _ptr(q), _ptr(scale), _ptr(q_t),
        _ptr(scale_t), rp, _ptr(offs_pad), _stream(stream)))
    return a2, q, scale, q_t, scale_t, offs_pad


def swiglu_backward_quantize_mx_dual(da2, h1, offs, rule=MX_FLOOR_OCP, rows_pad=None, dh1=None, q=None, scale=None,
                                     q_t=None, scale_t=None, offs_pad=None, layout=MX_LAYOUT_K4, stream=None):
    """da2 [R, F], h1 [R, 2F] bf16, offs int32 [E] -> (dh1 or None, q [R, 2F], scale, q_t [2F, rows_pad], scale_t,
    offs_pad): both MX forms of SwiGLU's input gradient; dh1 (bf16 [R, 2F]) is written only if passed."""
    h1 = _bits(h1)
    da2 = _bits(da2).contiguous()
    R, F2 = h1.shape
    if F2 % 2 or (h1.numel() and h1.stride(1) != 1) or tuple(da2.shape) != (R, F2 // 2):
        raise ValueError("swiglu_backward_quantize_mx_dual: h1 [R, 2F] with unit column stride, da2 [R, F]")
    F = F2 // 2
    ld = h1.stride(0) if h1.numel() else F2
    rp, q, scale, q_t, scale_t, offs_pad = _mx_dual_outputs(R, F2, offs, rows_pad, q, scale, q_t, scale_t, offs_pad,
                                                            layout, h1.device)
    _lib.check("swiglu_backward_quantize_mx_dual", _lib.lib().swiglu_backward_quantize_mx_dual(
        _ptr(da2), _ptr(h1), R, F, ld, _ptr(offs), offs.numel(), rule, layout, _ptr(dh1), _ptr(q), _ptr(scale),
        _ptr(q_t), _ptr(scale_t), rp, _ptr(offs_pad), _stream(stream)))
    return dh1, q, scale, q_t, scale_t, offs_pad


def grouped_mm_scaled(mode, a, a_fmt, a_scale, b, b_fmt, b_scale, scale_kind, offs, n_groups, M, N, K,
                      out=None, out_dtype=OUT_BF16, stream=None):
    """See include/fp8moe.h.  GROUPED_M -> out [M, N]; GROUPED_K -> out [E, N, K]."""
    dev = a.device
    if out is None:
        shape = (M, N) if mode == GROUPED_M else (n_groups, N, K)
        out = torch.empty(shape, dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device=dev)
    st = _lib.lib().grouped_mm_scaled(mode, _ptr(a), a_fmt, _ptr(a_scale), _ptr(b), b_fmt, _ptr(b_scale),
                                      scale_kind, _ptr(offs), n_groups, M, N, K, _ptr(out), out_dtype,
                                      _stream(stream))
    _lib.check("grouped_mm_scaled", st)
    return out


def swiglu_quantize_rowwise(h1, codec=E4M3FN, a2=None, q=None, scale=None, stream=None, codes=True):
    """h1 [R, 2F] bf16 (gate | up; row stride may exceed 2F) -> (a2 bf16 [R, F], q uint8 [R, F], scale f32 [R]);
    with codes=False only a2 is computed and q, scale are None."""
    h1 = _bits(h1)
    R, F2 = h1.shape
    if F2 % 2 or (h1.numel() and h1.stride(1) != 1):
        raise ValueError("swiglu_quantize_rowwise needs an even column count and unit column stride")
    F = F2 // 2
    ld = h1.stride(0) if h1.numel() else F2
    a2 = torch.empty((R, F), dtype=torch.bfloat16, device=h1.device) if a2 is None else a2
    if codes:
        q = torch.empty((R, F), dtype=torch.uint8, device=h1.device) if q is None else q
        scale = torch.empty((R,), dtype=torch.float32, device=h1.device) if scale is None else scale
    else:
        q = scale = None
    _lib.check("swiglu_quantize_rowwise", _lib.lib().swiglu_quantize_rowwise(
        _ptr(h1), R, F, ld, codec, _ptr(a2), _ptr(q), _ptr(scale), _stream(stream)))
    return a2, q, scale


def swiglu_backward_quantize_rowwise(da2, h1, codec=E4M3FN, dh1=None, q=None, scale=None, stream=None, codes=True):
    """da2 [R, F] bf16 and h1 [R, 2F] bf16 -> (dh1 bf16 [R, 2F], q uint8 [R, 2F], scale f32 [R]);
    with codes=False only dh1 is computed and q, scale are None."""
    h1 = _bits(h1)
    da2 = _bits(da2).contiguous()
    R, F2 = h1.shape
    if F2 % 2 or (h1.numel() and h1.stride(1) != 1) or tuple(da2.shape) != (R, F2 // 2):
        raise ValueError("swiglu_backward_quantize_rowwise: h1 [R, 2F] with unit column stride, da2 [R, F]")
    F = F2 // 2
    ld = h1.stride(0) if h1.numel() else F2
    dh1 = torch.empty((R, F2), dtype=torch.bfloat16, device=h1.device) if dh1 is None else dh1
    if codes:
        q = torch.empty((R, F2), dtype=torch.uint8, device=h1.device) if q is None else q
        scale = torch.empty((R,), dtype=torch.float32, device=h1.device) if scale is None else scale
    else:
        q = scale = None
    _lib.check("swiglu_backward_quantize_rowwise", _lib.lib().swiglu_backward_quantize_rowwise(
        _ptr(da2), _ptr(h1), R, F, ld, codec, _ptr(dh1), _ptr(q), _ptr(scale), _stream(stream)))
    return dh1, q, scale


def quantize_tensorwise(x, codec=E4M3FN, rowmajor=True, transposed=False, ld_q=None, n_scale=None, q=None,
                        q_t=None, scale=None, workspace=None, stream=None):
    """x bf16 [R, C] or [B, R, C] -> (q u8 [B*R, C] or None, q_t u8 [B, C, ld_q] or None, scale f32 [n_scale]).
    One scale for the whole tensor, repeated n_scale times (default: B*R, the row count); ld_q defaults to R
    rounded up to 16."""
    x = _bits(x).contiguous()
    B, R, C = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    dev = x.device
    if rowmajor and q is None:
        q = torch.empty((B * R, C), dtype=torch.uint8, device=dev)
    if transposed:
        ld_q = (R + 15) // 16 * 16 if ld_q is None else ld_q   # rows of q_t start 16-byte aligned
        if q_t is None:
            q_t = torch.empty((B, C, ld_q), dtype=torch.uint8, device=dev)
    n_scale = max(B * R, 1) if n_scale is None else n_scale
    scale = torch.empty((n_scale,), dtype=torch.float32, device=dev) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(int(_lib.lib().quantize_tensorwise_workspace_bytes()), dtype=torch.uint8, device=dev)
    _lib.check("quantize_tensorwise", _lib.lib().quantize_tensorwise(
        _ptr(x), B, R, C, codec, _ptr(q) if rowmajor else None, _ptr(q_t) if transposed else None,
        ld_q if transposed else 0, _ptr(scale), n_scale, _ptr(workspace), _stream(stream)))
    return (q if rowmajor else None), (q_t if transposed else None), scale


def quantize_blockwise(x, block_rows, codec=E4M3FN, q=None, scale=None, stream=None):
    """x bf16 [R, C] or [B, R, C] -> (q u8 of x's shape, scale f32 [B, ceil(R/block_rows), ceil(C/128)])."""
    x = _bits(x).contiguous()
    B, R, C = (1, *x.shape) if x.dim() == 2 else tuple(x.shape)
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    nr, nc = -(-R // block_rows), -(-C // 128)
    scale = torch.empty((B, nr, nc), dtype=torch.float32, device=x.device) if scale is None else scale
    _lib.check("quantize_blockwise", _lib.lib().quantize_blockwise(_ptr(x), B, R, C, block_rows, codec, _ptr(q),
                                                                    _ptr(scale), _stream(stream)))
    return q, scale


def grouped_mm_blockwise(a, a_scale, b, b_scale, offs, n_groups, M, N, K, out=None, out_dtype=OUT_BF16, stream=None):
    """GROUPED_M over blockwise e4m3fn operands -> out [M, N] (bf16 or f32)."""
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device=a.device)
    _lib.check("grouped_mm_blockwise", _lib.lib().grouped_mm_blockwise(
        _ptr(a), OPD_E4M3FN, _ptr(a_scale), _ptr(b), OPD_E4M3FN, _ptr(b_scale), _ptr(offs), n_groups, M, N, K,
        _ptr(out), out_dtype, _stream(stream)))
    return out


def quantize_blockwise_tokens(x, offs, codec=E4M3FN, ld_q=None, q_t=None, scale=None, stream=None):
    """x bf16 [M, C], offs int32 [E] -> (q_t u8 [C, ld_q], scale f32 [block bound, C])."""
    x = _bits(x).contiguous()
    M, C = x.shape
    E = offs.numel()
    ld_q = (M + 15) // 16 * 16 if ld_q is None else ld_q
    q_t = torch.empty((C, ld_q), dtype=torch.uint8, device=x.device) if q_t is None else q_t
    nb = int(_lib.lib().blockwise_token_blocks_bound(M, E))
    scale = torch.empty((nb, C), dtype=torch.float32, device=x.device) if scale is None else scale
    _lib.check("quantize_blockwise_tokens", _lib.lib().quantize_blockwise_tokens(
        _ptr(x), M, C, _ptr(offs), E, codec, _ptr(q_t), ld_q, _ptr(scale), _stream(stream)))
    return q_t, scale


def grouped_mm_blockwise_k(a_t, a_scale, b_t, b_scale, offs, tokens, out=None, out_dtype=OUT_BF16, stream=None):
    """GROUPED_K over blockwise operands a_t [N, ld], b_t [K, ld] -> out [E, N, K]."""
    N, ld = a_t.shape
    K = b_t.shape[0]
    E = offs.numel()
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32,
                          device=a_t.device)
    _lib.check("grouped_mm_blockwise_k", _lib.lib().grouped_mm_blockwise_k(
        _ptr(a_t), _ptr(a_scale), _ptr(b_t), _ptr(b_scale), _ptr(offs), E, tokens, ld, N, K, _ptr(out), out_dtype,
        _stream(stream)))
    return out


def moe_route_rows_bound(slots: int, n_experts: int, pad: int = 1) -> int:
    return int(_lib.lib().moe_route_rows_bound(slots, n_experts, pad))


def moe_route_workspace_bytes(slots: int, n_experts: int) -> int:
    return int(_lib.lib().moe_route_workspace_bytes(slots, n_experts))


def moe_route(expert_ids, n_experts, pad=1, out=None, workspace=None, stream=None):
    """expert_ids int32 [T, k] -> (counts [E], offs [E], dest [T*k], src [rows bound]), all int32."""
    ids = expert_ids.contiguous()
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise ValueError("moe_route needs int32 expert ids of shape [tokens, topk]")
    T, k = ids.shape
    rows = moe_route_rows_bound(T * k, n_experts, pad)
    ws = int(_lib.lib().moe_route_workspace_bytes(T * k, n_experts))
    if rows < 0 or ws < 0:
        raise ValueError(f"moe_route: invalid sizes tokens={T} topk={k} experts={n_experts} pad={pad}")
    dev = ids.device
    if out is None:
        out = (torch.empty(n_experts, dtype=torch.int32, device=dev), torch.empty(n_experts, dtype=torch.int32, device=dev),
               torch.empty(T * k, dtype=torch.int32, device=dev), torch.empty(rows, dtype=torch.int32, device=dev))
    counts, offs, dest, src = out
    if workspace is None:
        workspace = torch.empty(max(ws, 4), dtype=torch.uint8, device=dev)
    _lib.check("moe_route", _lib.lib().moe_route(_ptr(ids), T, k, n_experts, pad, _ptr(counts), _ptr(offs),
                                                  _ptr(dest), _ptr(src), _ptr(workspace), _stream(stream)))
    return counts, offs, dest, src


def moe_route_noalloc(expert_ids, n_experts, out, pad=1, stream=None):
    """moe_route on the library's fixed scratch: nothing is allocated, so the outputs
    out = (counts [E], offs [E], dest [T*k], src [rows bound]) (int32) must be passed."""
    ids = expert_ids
    if ids.dtype != torch.int32 or ids.dim() != 2 or not ids.is_contiguous():
        raise ValueError("moe_route_noalloc needs contiguous int32 expert ids of shape [tokens, topk]")
    T, k = ids.shape
    counts, offs, dest, src = out
    _lib.check("moe_route_noalloc", _lib.lib().moe_route_noalloc(_ptr(ids), T, k, n_experts, pad, _ptr(counts),
                                                                  _ptr(offs), _ptr(dest), _ptr(src), _stream(stream)))
    return counts, offs, dest, src


def moe_permute(x, src, topk, xg=None, stream=None):
    """x bf16 [T, C], src int32 [R] -> xg bf16 [R, C]: row r = x[src[r] // topk], zeros where src[r] < 0."""
    x = _bits(x).contiguous()
    T, C = x.shape
    R = src.numel()
    xg = torch.empty((R, C), dtype=x.dtype, device=x.device) if xg is None else xg
    _lib.check("moe_permute", _lib.lib().moe_permute(_ptr(x), T, C, topk, _ptr(src), R, _ptr(xg), _stream(stream)))
    return xg


def moe_permute_quantized(q, scale, src, topk, codec=E4M3FN, qg=None, scale_g=None, stream=None):
    """Rowwise codes q u8 [T, C] and scales f32 [T], src int32 [R] -> (qg u8 [R, C], scale_g f32 [R])."""
    q = q.contiguous()
    T, C = q.shape
    R = src.numel()
    qg = torch.empty((R, C), dtype=torch.uint8, device=q.device) if qg is None else qg
    scale_g = torch.empty((R,), dtype=torch.float32, device=q.device) if scale_g is None else scale_g
    _lib.check("moe_permute_quantized", _lib.lib().moe_permute_quantized(
        _ptr(q), _ptr(scale), T, C, topk, _ptr(src), R, codec, _ptr(qg), _ptr(scale_g), _stream(stream)))
    return qg, scale_g


def moe_combine(yg, dest, weights, topk, y=None, stream=None):
    """yg bf16 [R, C], dest int32 [T*k], weights f32 [T, k] or None (every weight 1) -> y bf16 [T, C]."""
    yg = _bits(yg).contiguous()
    R, C = yg.shape
    T = dest.numel() // topk
    if weights is not None:
        weights = weights.contiguous()
        if weights.dtype != torch.float32 or tuple(weights.shape) != (T, topk):
            raise ValueError("moe_combine: weights f32 [T, topk]")
    if dest.numel() != T * topk:
        raise ValueError("moe_combine: dest [T*topk]")
    y = torch.empty((T, C), dtype=yg.dtype, device=yg.device) if y is None else y
    _lib.check("moe_combine", _lib.lib().moe_combine(_ptr(yg), R, _ptr(dest), _ptr(weights), T, topk, C, _ptr(y),
                                                     _stream(stream)))
    return y


def moe_permute_rowwise(x, src, topk, codec=E4M3FN, xg=None, qg=None, scale_g=None, keep_bf16=True, stream=None):
    """x bf16 [T, C], src int32 [R] -> (xg bf16 [R, C] or None, qg u8 [R, C], scale_g f32 [R]): the gathered
    rows and their rowwise codes in one pass (keep_bf16=False skips the bf16 copy)."""
    x = _bits(x).contiguous()
    T, C = x.shape
    R = src.numel()
    if keep_bf16:
        xg = torch.empty((R, C), dtype=x.dtype, device=x.device) if xg is None else xg
    else:
        xg = None
    qg = torch.empty((R, C), dtype=torch.uint8, device=x.device) if qg is None else qg
    scale_g = torch.empty((R,), dtype=torch.float32, device=x.device) if scale_g is None else scale_g
    _lib.check("moe_permute_rowwise", _lib.lib().moe_permute_rowwise(
        _ptr(x), T, C, topk, _ptr(src), R, codec, _ptr(xg), _ptr(qg), _ptr(scale_g), _stream(stream)))
    return xg, qg, scale_g


def moe_combine_backward(dy, yg, dest, src, weights, topk, codec=E4M3FN, codes=True, dyg=None, q=None, scale=None,
                         dweights=None, stream=None, rows_out=True):
    """dy bf16 [T, C], yg bf16 [R, C], dest int32 [T*k], src int32 [R], weights f32 [T, k] ->
    (dyg bf16 [R, C] or None, q u8 [R, C] or None, scale f32 [R] or None, dweights f32 [T*k]).
    rows_out=False: the routed-row gradients are not written (dyg is None)."""
    dy = _bits(dy).contiguous()
    yg = _bits(yg).contiguous()
    T, C = dy.shape
    R = yg.shape[0]
    weights = weights.contiguous()
    if weights.dtype != torch.float32 or tuple(weights.shape) != (T, topk) or dest.numel() != T * topk \
            or src.numel() != R or yg.shape[1] != C:
        raise ValueError("moe_combine_backward: dy [T, C], yg [R, C], weights f32 [T, topk], dest [T*topk], src [R]")
    dev = dy.device
    if rows_out:
        dyg = torch.empty((R, C), dtype=dy.dtype, device=dev) if dyg is None else dyg
    else:
        dyg = None
    if codes:
        q = torch.empty((R, C), dtype=torch.uint8, device=dev) if q is None else q
        scale = torch.empty((R,), dtype=torch.float32, device=dev) if scale is None else scale
    else:
        q = scale = None
    dweights = torch.empty((T * topk,), dtype=torch.float32, device=dev) if dweights is None else dweights
    _lib.check("moe_combine_backward", _lib.lib().moe_combine_backward(
        _ptr(dy), _ptr(yg), R, _ptr(dest), _ptr(src), _ptr(weights), T, topk, C, codec, _ptr(dyg), _ptr(q),
        _ptr(scale), _ptr(dweights), _stream(stream)))
    return dyg, q, scale, dweights


def encode_f32(y, codec=E4M3FN, q=None, stream=None):
    """The device FP8 encoder on fp32 values already inside [-fmax, fmax]."""
    q = torch.empty(y.shape, dtype=torch.uint8, device=y.device) if q is None else q
    _lib.check("fp8moe_encode_f32", _lib.lib().fp8moe_encode_f32(_ptr(y), y.numel(), codec, _ptr(q),
                                                                 _stream(stream)))
    return q


def default_codec(device: int = 0) -> int:
    import ctypes
    out = ctypes.c_int(-1)
    _lib.check("fp8moe_default_codec", _lib.lib().fp8moe_default_codec(device, ctypes.byref(out)))
    return out.value
