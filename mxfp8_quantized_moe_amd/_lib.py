"""ctypes loader for libfp8moe.so (the C ABI in include/fp8moe.h).

The library is loaded from this package directory only; there is no fallback:
if it is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8moe.so")

# status codes and enums (mirror include/fp8moe.h)
OK, ERR_NULL, ERR_SHAPE, ERR_ENUM, ERR_ALIGN, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_DEVICE, ERR_SCRATCH = range(9)
E4M3FN, E4M3FNUZ = 0, 1
MX_FLOOR_OCP, MX_CEIL = 0, 1
MX_LAYOUT_ROWS, MX_LAYOUT_K4 = 0, 1
GROUPED_M, GROUPED_K = 0, 1
OPD_E4M3FN, OPD_E4M3FNUZ, OPD_BF16 = 0, 1, 2
SCALE_F32, SCALE_E8M0, SCALE_NONE, SCALE_E8M0_K4 = 0, 1, 2, 3
OUT_BF16, OUT_F32 = 0, 1

EXPORTS = ["quantize_rowwise", "quantize_colwise", "quantize_mx", "quantize_mx_rows_bound",
           "grouped_mm_scaled", "fp8moe_encode_f32", "fp8moe_status_string", "fp8moe_default_codec",
           "fp8moe_version", "swiglu_quantize_rowwise", "swiglu_backward_quantize_rowwise", "moe_route", "moe_route_workspace_bytes",
           "moe_route_rows_bound", "moe_permute", "moe_combine", "quantize_tensorwise", "moe_permute_quantized",
           "quantize_blockwise", "grouped_mm_blockwise", "quantize_blockwise_tokens",
           "blockwise_token_blocks_bound", "grouped_mm_blockwise_k",
           "quantize_tensorwise_workspace_bytes", "fp8moe_set_colwise_poll_budget", "fp8moe_set_colwise_chunk_rows", "moe_route_noalloc",
           "moe_permute_rowwise", "moe_combine_backward", "quantize_mx_dual", "swiglu_quantize_mx_dual",
           "swiglu_backward_quantize_mx_dual", "moe_permute_quantize_mx_dual", "moe_permute_quantize_colwise"]

_lib = None

_vp, _i64, _i32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int

_SIGS = {
    "quantize_rowwise": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp]),
    "quantize_colwise": (_int, [_vp, _i64, _i64, _i64, _vp, _i32, _int, _vp, _i64, _vp, _vp]),
    "moe_permute_quantize_colwise": (_int, [_vp, _i64, _i64, _i32, _vp, _vp, _i64, _vp, _i32, _int, _vp, _i64, _vp,
                                            _vp]),
    "quantize_mx": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _i32, _int, _int, _vp, _vp, _i64, _vp, _vp]),
    "quantize_mx_rows_bound": (_i64, [_i64, _i32]),
    "grouped_mm_scaled": (_int, [_int, _vp, _int, _vp, _vp, _int, _vp, _int, _vp, _i32, _i64, _i64, _i64,
                                 _vp, _int, _vp]),
    "fp8moe_encode_f32": (_int, [_vp, _i64, _int, _vp, _vp]),
    "fp8moe_status_string": (ctypes.c_char_p, [_int]),
    "fp8moe_default_codec": (_int, [_int, ctypes.POINTER(_int)]),
    "fp8moe_version": (_int, []),
    "fp8moe_set_colwise_poll_budget": (_int, [_int]),
    "fp8moe_set_colwise_chunk_rows": (_int, [_int]),
    "swiglu_quantize_rowwise": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]),
    "swiglu_backward_quantize_rowwise": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp]),
    "quantize_tensorwise": (_int, [_vp, _i64, _i64, _i64, _int, _vp, _vp, _i64, _vp, _i64, _vp, _vp]),
    "quantize_tensorwise_workspace_bytes": (_i64, []),
    "quantize_blockwise_tokens": (_int, [_vp, _i64, _i64, _vp, _i32, _int, _vp, _i64, _vp, _vp]),
    "blockwise_token_blocks_bound": (_i64, [_i64, _i32]),
    "grouped_mm_blockwise_k": (_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _vp, _int, _vp]),
    "quantize_blockwise": (_int, [_vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp]),
    "grouped_mm_blockwise": (_int, [_vp, _int, _vp, _vp, _int, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _int, _vp]),
    "moe_route": (_int, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_workspace_bytes": (_i64, [_i64, _i32]),
    "moe_route_noalloc": (_int, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_rows_bound": (_i64, [_i64, _i32, _i32]),
    "moe_permute": (_int, [_vp, _i64, _i64, _i32, _vp, _i64, _vp, _vp]),
    "moe_permute_quantized": (_int, [_vp, _vp, _i64, _i64, _i32, _vp, _i64, _int, _vp, _vp, _vp]),
    "moe_combine": (_int, [_vp, _i64, _vp, _vp, _i64, _i32, _i64, _vp, _vp]),
    "swiglu_quantize_mx_dual": (_int, [_vp, _i64, _i64, _i64, _vp, _i32, _int, _int, _vp, _vp, _vp, _vp, _vp, _i64,
                                       _vp, _vp]),
    "swiglu_backward_quantize_mx_dual": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _i32, _int, _int, _vp, _vp, _vp,
                                                _vp, _vp, _i64, _vp, _vp]),
    "quantize_mx_dual": (_int, [_vp, _i64, _i64, _i64, _vp, _i32, _int, _int, _vp, _vp, _vp, _vp, _i64, _vp, _vp]),
    "moe_permute_quantize_mx_dual": (_int, [_vp, _i64, _i64, _i32, _vp, _vp, _i64, _vp, _i32, _int, _int, _vp, _vp,
                                            _vp, _vp, _vp, _i64, _vp, _vp]),
    "moe_permute_rowwise": (_int, [_vp, _i64, _i64, _i32, _vp, _i64, _int, _vp, _vp, _vp, _vp]),
    "moe_combine_backward": (_int, [_vp, _vp, _i64, _vp, _vp, _vp, _i64, _i32, _i64, _int, _vp, _vp, _vp, _vp,
                                    _vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises OSError if it is not built or cannot load)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python mxfp8_quantized_moe_amd/build_lib.py")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class Fp8MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().fp8moe_status_string(status).decode()} (status {status})")


def check(fn: str, status: int) -> None:
    if status != OK:
        raise Fp8MoeError(fn, status)
