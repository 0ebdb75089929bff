"""C ABI tests that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call.

Only argument combinations that fail validation are passed here; a call that
passes validation would enqueue GPU work.  Fake pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from mxfp8_quantized_moe_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8moe.h")

P = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)
MIS = 0x10001        # misaligned


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(lib, n)
    nm = os.popen(f"nm -D --defined-only {L.LIB_PATH}").read()
    for n in names:
        assert re.search(rf" T {n}$", nm, flags=re.M), n


def test_status_strings_and_version(lib):
    assert lib.fp8moe_status_string(0) == b"ok"
    for s in range(1, 9):
        assert lib.fp8moe_status_string(s) not in (b"ok", b"unknown status")
    assert lib.fp8moe_status_string(99) == b"unknown status"
    assert lib.fp8moe_version() == 108


def test_rows_bound(lib):
    assert lib.quantize_mx_rows_bound(75, 4) == 224
    assert lib.quantize_mx_rows_bound(16384, 16) == 16896
    assert lib.quantize_mx_rows_bound(0, 1) == 32
    assert lib.quantize_mx_rows_bound(-1, 1) == -1


def test_rowwise_rejections(lib):
    f = lib.quantize_rowwise
    assert f(P, 4, 16, 16, 7, P, P, None) == L.ERR_ENUM
    assert f(P, -1, 16, 16, 0, P, P, None) == L.ERR_SHAPE
    assert f(P, 4, 16, 8, 0, P, P, None) == L.ERR_SHAPE            # ld_x < cols
    assert f(None, 4, 16, 16, 0, P, P, None) == L.ERR_NULL
    assert f(P, 4, 16, 16, 0, None, P, None) == L.ERR_NULL
    assert f(P, 4, 16, 16, 0, P, None, None) == L.ERR_NULL
    assert f(P, 4, 12, 16, 0, P, P, None) == L.ERR_ALIGN            # cols % 8
    assert f(P, 4, 16, 20, 0, P, P, None) == L.ERR_ALIGN            # ld_x % 8
    assert f(MIS, 4, 16, 16, 0, P, P, None) == L.ERR_ALIGN
    assert f(P, 4, 16, 16, 0, MIS, P, None) == L.ERR_ALIGN
    assert f(P, 4, 16, 16, 0, P, P + 2, None) == L.ERR_ALIGN


def test_swiglu_rejections(lib):
    f = lib.swiglu_quantize_rowwise          # (h1, rows, F, ld_h1, codec, a2, q, scale, stream)
    assert f(P, 4, 16, 32, 7, P, P, P, None) == L.ERR_ENUM
    assert f(P, -1, 16, 32, 0, P, P, P, None) == L.ERR_SHAPE
    assert f(P, 4, 16, 24, 0, P, P, P, None) == L.ERR_SHAPE          # ld_h1 < 2F
    assert f(None, 4, 16, 32, 0, P, P, P, None) == L.ERR_NULL
    assert f(P, 4, 16, 32, 0, None, P, P, None) == L.ERR_NULL
    assert f(P, 4, 16, 32, 0, P, None, P, None) == L.ERR_NULL
    assert f(P, 4, 16, 32, 0, P, P, None, None) == L.ERR_NULL
    assert f(P, 4, 12, 32, 0, P, P, P, None) == L.ERR_ALIGN           # F % 8
    assert f(P, 4, 16, 36, 0, P, P, P, None) == L.ERR_ALIGN           # ld_h1 % 8
    assert f(MIS, 4, 16, 32, 0, P, P, P, None) == L.ERR_ALIGN
    assert f(P, 4, 16, 32, 0, MIS, P, P, None) == L.ERR_ALIGN
    assert f(P, 4, 16, 32, 0, P, MIS, P, None) == L.ERR_ALIGN
    assert f(P, 4, 16, 32, 0, P, P, P + 2, None) == L.ERR_ALIGN
    b = lib.swiglu_backward_quantize_rowwise  # (da2, h1, rows, F, ld_h1, codec, dh1, q, scale, stream)
    assert b(P, P, 4, 16, 32, 7, P, P, P, None) == L.ERR_ENUM
    assert b(P, P, 4, 16, 24, 0, P, P, P, None) == L.ERR_SHAPE
    assert b(None, P, 4, 16, 32, 0, P, P, P, None) == L.ERR_NULL
    assert b(P, None, 4, 16, 32, 0, P, P, P, None) == L.ERR_NULL
    assert b(P, P, 4, 16, 32, 0, None, P, P, None) == L.ERR_NULL
    assert b(MIS, P, 4, 16, 32, 0, P, P, P, None) == L.ERR_ALIGN
    assert b(P, P, 4, 12, 32, 0, P, P, P, None) == L.ERR_ALIGN
    # nothing to do: zero rows is accepted without touching any pointer
    assert f(None, 0, 16, 32, 0, None, None, None, None) == L.OK
    assert b(None, None, 0, 16, 32, 0, None, None, None, None) == L.OK


def test_tensorwise_rejections(lib):
    f = lib.quantize_tensorwise   # (x, batch, rows, cols, codec, q, q_t, ld_q, scale, n_scale, workspace, stream)
    assert lib.quantize_tensorwise_workspace_bytes() == 4096
    assert f(P, 1, 4, 16, 7, P, P, 16, P, 4, P, None) == L.ERR_ENUM
    assert f(P, 0, 4, 16, 0, P, P, 16, P, 4, P, None) == L.ERR_SHAPE       # batch 0
    assert f(P, 1, -1, 16, 0, P, P, 16, P, 4, P, None) == L.ERR_SHAPE
    assert f(P, 1, 4, 16, 0, P, P, 16, P, 0, P, None) == L.ERR_SHAPE       # no scale entry
    assert f(P, 1, 20, 16, 0, P, P, 16, P, 4, P, None) == L.ERR_SHAPE      # ld_q < rows
    assert f(None, 1, 4, 16, 0, P, P, 16, P, 4, P, None) == L.ERR_NULL
    assert f(P, 1, 4, 16, 0, P, P, 16, None, 4, P, None) == L.ERR_NULL
    assert f(P, 1, 4, 16, 0, P, P, 16, P, 4, None, None) == L.ERR_NULL
    assert f(P, 1, 4, 12, 0, P, P, 16, P, 4, P, None) == L.ERR_ALIGN       # cols % 8
    assert f(MIS, 1, 4, 16, 0, P, P, 16, P, 4, P, None) == L.ERR_ALIGN
    assert f(P, 1, 4, 16, 0, MIS, P, 16, P, 4, P, None) == L.ERR_ALIGN
    assert f(P, 1, 4, 16, 0, P, MIS, 16, P, 4, P, None) == L.ERR_ALIGN
    assert f(P, 1, 4, 16, 0, P, P, 24, P, 4, P, None) == L.ERR_ALIGN       # ld_q % 16
    assert f(P, 1, 4, 16, 0, P, P, 16, P + 2, 4, P, None) == L.ERR_ALIGN


def test_blockwise_rejections(lib):
    f = lib.quantize_blockwise   # (x, batch, rows, cols, block_rows, codec, q, scale, stream)
    assert f(P, 1, 4, 16, 1, 7, P, P, None) == L.ERR_ENUM
    assert f(P, 1, 4, 16, 64, 0, P, P, None) == L.ERR_ENUM          # tile height 1 or 128 only
    assert f(P, 0, 4, 16, 1, 0, P, P, None) == L.ERR_SHAPE
    assert f(None, 1, 4, 16, 1, 0, P, P, None) == L.ERR_NULL
    assert f(P, 1, 4, 16, 1, 0, P, None, None) == L.ERR_NULL
    assert f(P, 1, 4, 12, 1, 0, P, P, None) == L.ERR_ALIGN
    assert f(MIS, 1, 4, 16, 128, 0, P, P, None) == L.ERR_ALIGN
    g = lib.grouped_mm_blockwise  # (a, a_fmt, sa, b, b_fmt, sb, offs, n_groups, M, N, K, out, out_dtype, stream)
    assert g(P, 0, P, P, 0, P, P, 2, 64, 64, 128, P, 5, None) == L.ERR_ENUM
    assert g(P, 1, P, P, 0, P, P, 2, 64, 64, 128, P, 0, None) == L.ERR_UNSUPPORTED   # fnuz codes
    assert g(P, 0, P, P, 2, P, P, 2, 64, 64, 128, P, 0, None) == L.ERR_UNSUPPORTED   # bf16
    assert g(P, 0, P, P, 0, P, P, 0, 64, 64, 128, P, 0, None) == L.ERR_SHAPE
    assert g(P, 0, P, P, 0, P, P, 2, -1, 64, 128, P, 0, None) == L.ERR_SHAPE
    assert g(P, 0, P, P, 0, P, None, 2, 64, 64, 128, P, 0, None) == L.ERR_NULL
    assert g(P, 0, None, P, 0, P, P, 2, 64, 64, 128, P, 0, None) == L.ERR_NULL
    assert g(P, 0, P, P, 0, P, P, 2, 64, 64, 128, None, 0, None) == L.ERR_NULL
    assert g(P, 0, P, P, 0, P, P, 2, 64, 64, 120, P, 0, None) == L.ERR_ALIGN          # K % 16
    assert g(MIS, 0, P, P, 0, P, P, 2, 64, 64, 128, P, 0, None) == L.ERR_ALIGN
    assert g(P, 0, P, P, 0, P + 2, P, 2, 64, 64, 128, P, 0, None) == L.ERR_ALIGN


def test_blockwise_tokens_rejections(lib):
    f = lib.quantize_blockwise_tokens   # (x, tokens, cols, offs, n_groups, codec, q_t, ld_q, scale, stream)
    assert lib.blockwise_token_blocks_bound(300, 4) == 3 + 4
    assert lib.blockwise_token_blocks_bound(-1, 4) == -1 and lib.blockwise_token_blocks_bound(10, 0) == -1
    assert f(P, 64, 16, P, 2, 7, P, 64, P, None) == L.ERR_ENUM
    assert f(P, 64, 16, P, 0, 0, P, 64, P, None) == L.ERR_SHAPE       # no groups
    assert f(P, 64, 16, P, 2, 0, P, 48, P, None) == L.ERR_SHAPE       # ld_q < tokens
    assert f(P, 64, 16, None, 2, 0, P, 64, P, None) == L.ERR_NULL
    assert f(None, 64, 16, P, 2, 0, P, 64, P, None) == L.ERR_NULL
    assert f(P, 64, 16, P, 2, 0, P, 64, None, None) == L.ERR_NULL
    assert f(P, 64, 12, P, 2, 0, P, 64, P, None) == L.ERR_ALIGN       # cols % 8
    assert f(P, 64, 16, P, 2, 0, P, 72, P, None) == L.ERR_ALIGN       # ld_q % 16
    assert f(P, 64, 16, P, 2, 0, MIS, 64, P, None) == L.ERR_ALIGN
    g = lib.grouped_mm_blockwise_k   # (a_t, sa, b_t, sb, offs, n_groups, tokens, ld, N, K, out, out_dtype, stream)
    assert g(P, P, P, P, P, 2, 64, 64, 32, 32, P, 3, None) == L.ERR_ENUM
    assert g(P, P, P, P, P, 0, 64, 64, 32, 32, P, 0, None) == L.ERR_SHAPE
    assert g(P, P, P, P, P, 2, 64, 48, 32, 32, P, 0, None) == L.ERR_SHAPE   # ld < tokens
    assert g(P, P, P, P, None, 2, 64, 64, 32, 32, P, 0, None) == L.ERR_NULL
    assert g(None, P, P, P, P, 2, 64, 64, 32, 32, P, 0, None) == L.ERR_NULL
    assert g(P, P, P, P, P, 2, 64, 64, 32, 32, None, 0, None) == L.ERR_NULL
    assert g(P, P, P, P, P, 2, 64, 72, 32, 32, P, 0, None) == L.ERR_ALIGN   # ld % 16
    assert g(P, P, MIS, P, P, 2, 64, 64, 32, 32, P, 0, None) == L.ERR_ALIGN


def test_route_rejections(lib):
    r = lib.moe_route        # (ids, tokens, topk, E, pad, counts, offs, dest, src, workspace, stream)
    assert r(P, -1, 2, 8, 1, P, P, P, P, P, None) == L.ERR_SHAPE
    assert r(P, 4, 0, 8, 1, P, P, P, P, P, None) == L.ERR_SHAPE     # topk 0
    assert r(P, 4, 2, 0, 1, P, P, P, P, P, None) == L.ERR_SHAPE     # no experts
    assert r(P, 4, 2, 8, 0, P, P, P, P, P, None) == L.ERR_SHAPE     # pad 0
    assert r(P, 1 << 30, 4, 8, 1, P, P, P, P, P, None) == L.ERR_SHAPE  # slots beyond int32
    assert r(P, 4, 2, 8, 1 << 29, P, P, P, P, P, None) == L.ERR_SHAPE  # rows bound beyond int32
    assert r(P, 4, 2, 1025, 1, P, P, P, P, P, None) == L.ERR_UNSUPPORTED
    assert r(None, 4, 2, 8, 1, P, P, P, P, P, None) == L.ERR_NULL
    assert r(P, 4, 2, 8, 1, None, P, P, P, P, None) == L.ERR_NULL
    assert r(P, 4, 2, 8, 1, P, None, P, P, P, None) == L.ERR_NULL
    assert r(P, 4, 2, 8, 1, P, P, None, P, P, None) == L.ERR_NULL
    assert r(P, 4, 2, 8, 1, P, P, P, None, P, None) == L.ERR_NULL
    assert r(P, 4, 2, 8, 1, P, P, P, P, None, None) == L.ERR_NULL
    assert r(P + 2, 4, 2, 8, 1, P, P, P, P, P, None) == L.ERR_ALIGN
    assert r(P, 4, 2, 8, 1, P, P, P + 2, P, P, None) == L.ERR_ALIGN
    assert r(P, 4, 2, 8, 1, P, P, P, P, P + 1, None) == L.ERR_ALIGN
    assert lib.moe_route_rows_bound(100, 8, 32) == 100 + 8 * 31
    assert lib.moe_route_rows_bound(100, 0, 1) == -1 and lib.moe_route_rows_bound(-1, 8, 1) == -1
    assert lib.moe_route_rows_bound((1 << 31) - 8, 8, 2) == -1
    assert lib.moe_route_workspace_bytes(0, 8) == 0
    assert lib.moe_route_workspace_bytes(1, 8) == lib.moe_route_workspace_bytes(256, 8) > 0
    assert lib.moe_route_workspace_bytes(257, 8) == 2 * lib.moe_route_workspace_bytes(256, 8)
    p = lib.moe_permute      # (x, tokens, cols, topk, src, rows_out, xg, stream)
    assert p(P, -1, 16, 2, P, 8, P, None) == L.ERR_SHAPE
    assert p(P, 4, 16, 0, P, 8, P, None) == L.ERR_SHAPE
    assert p(P, 4, 16, 2, P, -1, P, None) == L.ERR_SHAPE
    assert p(None, 4, 16, 2, P, 8, P, None) == L.ERR_NULL
    assert p(P, 4, 16, 2, None, 8, P, None) == L.ERR_NULL
    assert p(P, 4, 16, 2, P, 8, None, None) == L.ERR_NULL
    assert p(P, 4, 12, 2, P, 8, P, None) == L.ERR_ALIGN             # cols % 8
    assert p(MIS, 4, 16, 2, P, 8, P, None) == L.ERR_ALIGN
    assert p(P, 4, 16, 2, P, 8, MIS, None) == L.ERR_ALIGN
    assert p(None, 0, 16, 2, None, 0, None, None) == L.OK          # nothing to do
    pq = lib.moe_permute_quantized   # (q, scale, tokens, cols, topk, src, rows_out, codec, qg, scale_g, stream)
    assert pq(P, P, 4, 32, 2, P, 8, 7, P, P, None) == L.ERR_ENUM
    assert pq(P, P, -1, 32, 2, P, 8, 0, P, P, None) == L.ERR_SHAPE
    assert pq(P, P, 4, 32, 0, P, 8, 0, P, P, None) == L.ERR_SHAPE
    assert pq(None, P, 4, 32, 2, P, 8, 0, P, P, None) == L.ERR_NULL
    assert pq(P, None, 4, 32, 2, P, 8, 0, P, P, None) == L.ERR_NULL
    assert pq(P, P, 4, 32, 2, P, 8, 0, P, None, None) == L.ERR_NULL
    assert pq(P, P, 4, 24, 2, P, 8, 0, P, P, None) == L.ERR_ALIGN          # cols % 16
    assert pq(MIS, P, 4, 32, 2, P, 8, 0, P, P, None) == L.ERR_ALIGN
    assert pq(P, P + 2, 4, 32, 2, P, 8, 0, P, P, None) == L.ERR_ALIGN
    assert pq(None, None, 0, 32, 2, None, 0, 0, None, None, None) == L.OK
    c = lib.moe_combine      # (yg, rows_in, dest, weights, tokens, topk, cols, y, stream)
    assert c(P, 8, P, P, -1, 2, 16, P, None) == L.ERR_SHAPE
    assert c(P, -1, P, P, 4, 2, 16, P, None) == L.ERR_SHAPE
    assert c(P, 8, P, P, 4, 0, 16, P, None) == L.ERR_SHAPE
    assert c(None, 8, P, P, 4, 2, 16, P, None) == L.ERR_NULL
    assert c(P, 8, None, P, 4, 2, 16, P, None) == L.ERR_NULL
    # weights may be null (every weight 1): that call passes validation, so it is not made here
    assert c(P, 8, P, P, 4, 2, 16, None, None) == L.ERR_NULL
    assert c(P, 8, P, P, 4, 2, 12, P, None) == L.ERR_ALIGN
    assert c(MIS, 8, P, P, 4, 2, 16, P, None) == L.ERR_ALIGN
    assert c(P, 8, P, P + 2, 4, 2, 16, P, None) == L.ERR_ALIGN
    assert c(None, 0, None, None, 0, 2, 16, None, None) == L.OK    # nothing to do
    pr = lib.moe_permute_rowwise   # (x, tokens, cols, topk, src, rows_out, codec, xg, qg, scale_g, stream)
    assert pr(P, 4, 16, 2, P, 8, 7, P, P, P, None) == L.ERR_ENUM
    assert pr(P, -1, 16, 2, P, 8, 0, P, P, P, None) == L.ERR_SHAPE
    assert pr(P, 4, 16, 0, P, 8, 0, P, P, P, None) == L.ERR_SHAPE
    assert pr(P, 4, 16, 2, P, -1, 0, P, P, P, None) == L.ERR_SHAPE
    assert pr(None, 4, 16, 2, P, 8, 0, P, P, P, None) == L.ERR_NULL
    assert pr(P, 4, 16, 2, None, 8, 0, P, P, P, None) == L.ERR_NULL
    assert pr(P, 4, 16, 2, P, 8, 0, P, None, P, None) == L.ERR_NULL
    assert pr(P, 4, 16, 2, P, 8, 0, P, P, None, None) == L.ERR_NULL
    assert pr(P, 4, 16392, 2, P, 8, 0, None, P, P, None) == L.ERR_NULL   # long rows need the bf16 copy
    assert pr(P, 4, 12, 2, P, 8, 0, P, P, P, None) == L.ERR_ALIGN        # cols % 8
    assert pr(MIS, 4, 16, 2, P, 8, 0, P, P, P, None) == L.ERR_ALIGN
    assert pr(P, 4, 16, 2, P, 8, 0, MIS, P, P, None) == L.ERR_ALIGN
    assert pr(P, 4, 16, 2, P, 8, 0, P, MIS, P, None) == L.ERR_ALIGN
    assert pr(P, 4, 16, 2, P, 8, 0, P, P, P + 2, None) == L.ERR_ALIGN
    assert pr(None, 0, 16, 2, None, 0, 0, None, None, None, None) == L.OK   # nothing to do
    cb = lib.moe_combine_backward
    # (dy, yg, rows, dest, src, weights, tokens, topk, cols, codec, dyg, q, scale, dweights, stream)
    assert cb(P, P, 8, P, P, P, 4, 2, 16, 7, P, P, P, P, None) == L.ERR_ENUM
    assert cb(P, P, 8, P, P, P, -1, 2, 16, 0, P, P, P, P, None) == L.ERR_SHAPE
    assert cb(P, P, -1, P, P, P, 4, 2, 16, 0, P, P, P, P, None) == L.ERR_SHAPE
    assert cb(P, P, 8, P, P, P, 4, 0, 16, 0, P, P, P, P, None) == L.ERR_SHAPE
    assert cb(P, P, 8, P, P, P, 4, 2, 16392, 0, P, P, P, P, None) == L.ERR_UNSUPPORTED
    assert cb(P, P, 8, P, P, P, 4, 2, 16, 0, P, None, P, P, None) == L.ERR_NULL   # codes without scales
    assert cb(P, P, 8, P, P, P, 4, 2, 16, 0, P, P, None, P, None) == L.ERR_NULL
    for i in (0, 1, 3, 4, 5, 13):       # (dyg, index 10, may be NULL: the rows are then not written)
        args = [P, P, 8, P, P, P, 4, 2, 16, 0, P, P, P, P, None]
        args[i] = None
        assert cb(*args) == L.ERR_NULL, i
    assert cb(P, P, 8, P, P, P, 4, 2, 12, 0, P, P, P, P, None) == L.ERR_ALIGN    # cols % 8
    for i, bad in ((0, MIS), (1, MIS), (10, MIS), (11, MIS), (3, P + 2), (4, P + 2), (5, P + 2), (12, P + 2),
                   (13, P + 2)):
        args = [P, P, 8, P, P, P, 4, 2, 16, 0, P, P, P, P, None]
        args[i] = bad
        assert cb(*args) == L.ERR_ALIGN, i
    assert cb(None, None, 0, None, None, None, 0, 2, 16, 0, None, None, None, None, None) == L.OK


def test_colwise_rejections(lib):
    f = lib.quantize_colwise
    assert f(P, 1, 64, 16, P, 4, 3, P, 64, P, None) == L.ERR_ENUM
    assert f(P, 0, 64, 16, None, 0, 0, P, 64, P, None) == L.ERR_SHAPE      # batch 0
    assert f(P, 2, 64, 16, P, 4, 0, P, 64, P, None) == L.ERR_SHAPE         # offs needs batch 1
    assert f(P, 1, 64, 16, P, 0, 0, P, 64, P, None) == L.ERR_SHAPE         # no groups
    assert f(P, 1, 64, 16, P, 4, 0, P, 32, P, None) == L.ERR_SHAPE         # ld_q < rows
    assert f(None, 1, 64, 16, P, 4, 0, P, 64, P, None) == L.ERR_NULL
    assert f(P, 1, 64, 12, P, 4, 0, P, 64, P, None) == L.ERR_ALIGN         # cols % 8
    assert f(P, 1, 64, 16, P, 4, 0, P, 72, P, None) == L.ERR_ALIGN         # ld_q % 16
    assert f(P, 1, 64, 16, P, 4, 0, MIS, 64, P, None) == L.ERR_ALIGN


def test_mx_rejections(lib):
    f = lib.quantize_mx
    assert f(P, 1, 64, 64, 1, None, 0, 5, 0, P, P, 0, None, None) == L.ERR_ENUM       # rule
    assert f(P, 1, 64, 64, 2, None, 0, 0, 0, P, P, 0, None, None) == L.ERR_ENUM       # axis
    assert f(P, 1, 64, 64, 1, None, 0, 0, 2, P, P, 0, None, None) == L.ERR_ENUM       # scale layout
    assert f(P, 1, 64, 48, 1, None, 0, 0, 0, P, P, 0, None, None) == L.ERR_ALIGN      # cols % 32
    assert f(P, 1, 64, 48, 1, None, 0, 0, 1, P, P, 0, None, None) == L.ERR_ALIGN      # cols % 32 (K4)
    assert f(P, 1, 64, 64, 1, P, 4, 0, 0, P, P, 0, None, None) == L.ERR_UNSUPPORTED   # offs on axis 1
    assert f(P, 1, 40, 64, 0, None, 0, 0, 0, P, P, 0, None, None) == L.ERR_ALIGN      # rows % 32
    assert f(P, 1, 75, 64, 0, P, 4, 0, 0, P, P, 192, P, None) == L.ERR_SHAPE          # rows_pad < bound
    assert f(P, 1, 75, 64, 0, P, 4, 0, 0, P, P, 230, P, None) == L.ERR_ALIGN          # rows_pad % 32
    assert f(P, 2, 75, 64, 0, P, 4, 0, 0, P, P, 224, P, None) == L.ERR_SHAPE          # batch with offs
    assert f(P, 1, 75, 64, 0, P, 4, 0, 0, None, P, 224, P, None) == L.ERR_NULL
    assert f(P, 1, 75, 64, 0, P, 4, 0, 1, P, None, 224, P, None) == L.ERR_NULL        # K4 scales missing
    # K4 scale tensors are addressed with 32-bit offsets: at most 2^31 - 1 bytes
    assert f(P, 1, 1 << 29, 2048, 1, None, 0, 0, 1, P, P, 0, None, None) == L.ERR_SHAPE


def test_mx_dual_rejections(lib):
    d = lib.quantize_mx_dual
    # (x, batch, rows, cols, offs, n_groups, rule, layout, q, sc, q_t, sc_t, rows_pad, offs_pad, stream)
    assert d(P, 1, 64, 64, None, 0, 5, 0, P, P, P, P, 64, None, None) == L.ERR_ENUM          # rule
    assert d(P, 1, 64, 64, None, 0, 0, 2, P, P, P, P, 64, None, None) == L.ERR_ENUM          # scale layout
    assert d(P, 1, 64, 48, None, 0, 0, 0, P, P, P, P, 64, None, None) == L.ERR_ALIGN         # cols % 32
    assert d(P, 2, 40, 64, None, 0, 0, 0, P, P, P, P, 40, None, None) == L.ERR_ALIGN         # rows % 32 (batched)
    assert d(P, 1, 75, 64, P, 4, 0, 0, P, P, P, P, 192, P, None) == L.ERR_SHAPE              # rows_pad < bound
    assert d(P, 2, 75, 64, P, 4, 0, 0, P, P, P, P, 224, P, None) == L.ERR_SHAPE              # batch with offs
    assert d(P, 1, 64, 64, None, 0, 0, 0, None, P, P, P, 64, None, None) == L.ERR_NULL       # last-dim codes
    assert d(P, 1, 64, 64, None, 0, 0, 0, P, None, P, P, 64, None, None) == L.ERR_NULL       # last-dim scales
    assert d(P, 1, 64, 64, None, 0, 0, 0, P, P, None, P, 64, None, None) == L.ERR_NULL       # row-block codes
    assert d(P, 1, 64, 64, None, 0, 0, 1, P, P, P, None, 64, None, None) == L.ERR_NULL       # row-block scales
    assert d(MIS, 1, 64, 64, None, 0, 0, 0, P, P, P, P, 64, None, None) == L.ERR_ALIGN
    assert d(P, 1, 64, 64, None, 0, 0, 0, MIS, P, P, P, 64, None, None) == L.ERR_ALIGN
    assert d(P, 1, 64, 64, None, 0, 0, 0, P, P, MIS, P, 64, None, None) == L.ERR_ALIGN


def test_moe_permute_mx_dual_rejections(lib):
    f = lib.moe_permute_quantize_mx_dual
    # (x, tokens, cols, topk, src, weights, rows, offs, n_groups, rule, layout, xg, q, sc, q_t, sc_t, rows_pad,
    #  offs_pad, stream)
    ok = [P, 32, 64, 2, P, None, 64, P, 4, 0, 1, None, P, P, P, P, 64 + 128, P, None]
    def call(args, i=None, v=None):
        a = list(args)
        if i is not None:
            a[i] = v
        return f(*a)
    assert call(ok, 9, 5) == L.ERR_ENUM                   # rule
    assert call(ok, 10, 2) == L.ERR_ENUM                  # scale layout
    assert call(ok, 3, 0) == L.ERR_SHAPE                  # topk
    assert call(ok, 1, -1) == L.ERR_SHAPE                 # tokens
    assert call(ok, 1, 1 << 31) == L.ERR_SHAPE            # tokens * topk past int32
    assert call(ok, 16, 64) == L.ERR_SHAPE                # rows_pad below the bound
    assert call(ok, 7, None) == L.ERR_NULL                # offs: the grouped layout is required
    for i in (0, 4, 12, 13, 14, 15):                      # x, src, both codes and both scales
        assert call(ok, i, None) == L.ERR_NULL, i
    assert call(ok, 2, 48) == L.ERR_ALIGN                 # cols % 32
    for i, bad in ((0, MIS), (11, MIS), (12, MIS), (4, P + 2), (5, P + 2)):
        assert call(ok, i, bad) == L.ERR_ALIGN, i


def test_moe_permute_colwise_rejections(lib):
    f = lib.moe_permute_quantize_colwise
    # (x, tokens, cols, topk, src, weights, rows, offs, n_groups, codec, q_t, ld_q, scale, stream)
    ok = [P, 32, 64, 2, P, None, 64, P, 4, 0, P, 64, P, None]
    def call(i=None, v=None):
        a = list(ok)
        if i is not None:
            a[i] = v
        return f(*a)
    assert call(9, 7) == L.ERR_ENUM                       # codec
    assert call(3, 0) == L.ERR_SHAPE                      # topk
    assert call(1, -1) == L.ERR_SHAPE                     # tokens
    assert call(1, 1 << 31) == L.ERR_SHAPE                # tokens * topk past int32
    assert call(11, 48) == L.ERR_SHAPE                    # ld_q < rows
    assert call(7, None) == L.ERR_NULL                    # offs: the grouped layout is required
    for i in (0, 4, 10, 12):                              # x, src, codes, scales
        assert call(i, None) == L.ERR_NULL, i
    assert call(2, 60) == L.ERR_ALIGN                     # cols % 8
    assert call(11, 72) == L.ERR_ALIGN                    # ld_q % 16
    for i, bad in ((0, MIS), (10, MIS), (4, P + 2), (5, P + 2)):
        assert call(i, bad) == L.ERR_ALIGN, i


def test_swiglu_mx_dual_rejections(lib):
    f = lib.swiglu_quantize_mx_dual
    # (h1, rows, F, ld_h1, offs, n_groups, rule, layout, a2, q, sc, q_t, sc_t, rows_pad, offs_pad, stream)
    ok = [P, 64, 64, 128, P, 4, 0, 1, None, P, P, P, P, 64 + 128, P, None]
    def call(fn, args, i=None, v=None):
        a = list(args)
        if i is not None:
            a[i] = v
        return fn(*a)
    assert call(f, ok, 6, 5) == L.ERR_ENUM                 # rule
    assert call(f, ok, 7, 2) == L.ERR_ENUM                 # scale layout
    assert call(f, ok, 3, 100) == L.ERR_SHAPE              # ld_h1 < 2F
    assert call(f, ok, 1, -1) == L.ERR_SHAPE
    assert call(f, ok, 13, 64) == L.ERR_SHAPE              # rows_pad below the bound
    assert call(f, ok, 0, None) == L.ERR_NULL
    assert call(f, ok, 9, None) == L.ERR_NULL
    assert call(f, ok, 11, None) == L.ERR_NULL
    assert call(f, ok, 2, 48) == L.ERR_ALIGN               # F % 32
    assert call(f, ok, 3, 132) == L.ERR_ALIGN              # ld_h1 % 8
    assert call(f, ok, 0, MIS) == L.ERR_ALIGN
    assert call(f, ok, 8, MIS) == L.ERR_ALIGN              # the optional bf16 copy
    b = lib.swiglu_backward_quantize_mx_dual
    okb = [P, P, 64, 128, 256, P, 4, 0, 1, None, P, P, P, P, 64 + 128, P, None]
    assert call(b, okb, 7, 5) == L.ERR_ENUM
    assert call(b, okb, 4, 200) == L.ERR_SHAPE
    assert call(b, okb, 0, None) == L.ERR_NULL             # da2
    assert call(b, okb, 1, None) == L.ERR_NULL             # h1
    assert call(b, okb, 3, 48) == L.ERR_ALIGN
    assert call(b, [P, P, 64, 96, 192, P, 4, 0, 1, None, P, P, P, P, 192, P, None]) == L.ERR_ALIGN   # F % 128
    assert call(b, okb, 0, MIS) == L.ERR_ALIGN


def test_gemm_rejections(lib):
    f = lib.grouped_mm_scaled
    ok = dict(mode=0, a=P, af=0, sa=P, b=P, bf=0, sb=P, sk=0, offs=P, E=4, M=64, N=64, K=64, out=P, od=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["mode"], a["a"], a["af"], a["sa"], a["b"], a["bf"], a["sb"], a["sk"], a["offs"], a["E"],
                 a["M"], a["N"], a["K"], a["out"], a["od"], None)

    assert call(mode=2) == L.ERR_ENUM
    assert call(af=3) == L.ERR_ENUM
    assert call(sk=5) == L.ERR_ENUM
    assert call(od=2) == L.ERR_ENUM
    assert call(M=-1) == L.ERR_SHAPE
    assert call(E=0) == L.ERR_SHAPE
    assert call(offs=None) == L.ERR_NULL                  # several groups need offsets
    assert call(a=None) == L.ERR_NULL
    assert call(sa=None) == L.ERR_NULL
    assert call(af=2) == L.ERR_UNSUPPORTED                # bf16 x fp8
    assert call(af=2, bf=2, sk=2) == L.ERR_UNSUPPORTED    # bf16 only for GROUPED_K
    assert call(sk=2) == L.ERR_UNSUPPORTED                # fp8 without scales
    assert call(sk=1, af=1) == L.ERR_UNSUPPORTED          # e8m0 needs e4m3fn
    assert call(sk=3, bf=1) == L.ERR_UNSUPPORTED          # also in the K4 layout
    assert call(sk=3, K=48) == L.ERR_ALIGN                # K % 32 for e8m0 (K4)
    assert call(sk=3, sa=P + 2) == L.ERR_ALIGN            # K4 scales are read as 4-byte words
    assert call(sk=3, M=1 << 26, N=64, K=1024, E=1, offs=None) == L.ERR_SHAPE   # K4 a_scale of 2^31 B
    assert call(K=40) == L.ERR_ALIGN                      # K % 16 (GROUPED_M)
    assert call(sk=1, K=48) == L.ERR_ALIGN                # K % 32 for e8m0
    assert call(mode=1, M=40) == L.ERR_ALIGN              # M % 16 (GROUPED_K)
    assert call(out=MIS) == L.ERR_ALIGN


def test_encode_rejections(lib):
    assert lib.fp8moe_encode_f32(P, 16, 2, P, None) == L.ERR_ENUM
    assert lib.fp8moe_encode_f32(P, -1, 0, P, None) == L.ERR_SHAPE
    assert lib.fp8moe_encode_f32(None, 16, 0, P, None) == L.ERR_NULL
    assert lib.fp8moe_encode_f32(P + 2, 16, 0, P, None) == L.ERR_ALIGN


def test_python_binding_raises_on_bad_arguments():
    import mxfp8_quantized_moe_amd as fm
    with pytest.raises(fm.Fp8MoeError):
        L.check("quantize_rowwise", L.lib().quantize_rowwise(P, 4, 12, 16, 0, P, P, None))


def test_no_undefined_internal_symbols():
    """Every kernel launch stub and internal function resolves inside the library."""
    und = os.popen(f"nm -D --undefined-only {L.LIB_PATH}").read()
    assert "fp8moe" not in und, [l for l in und.splitlines() if "fp8moe" in l][:5]


def test_colwise_poll_budget_hook(lib):
    """Host-only test hook: returns the previous budget; negative restores the default."""
    f = lib.fp8moe_set_colwise_poll_budget
    first = f(7)
    try:
        assert f(0) == 7
        assert f(-1) == 0
        assert f(-1) == 4096
    finally:
        f(first)


def test_colwise_chunk_rows_hook(lib):
    """Host-only tuning hook: 128, 256 or 512 force a chunk height, anything else selects per call (0)."""
    f = lib.fp8moe_set_colwise_chunk_rows
    first = f(128)
    try:
        assert f(256) == 128
        assert f(512) == 256
        assert f(300) == 512
        assert f(1024) == 0
        assert f(0) == 0
    finally:
        f(first)


def test_route_noalloc_rejections(lib):
    """Host-side checks of the allocation-free routing (no HIP call is reached)."""
    r = lib.moe_route_noalloc   # (ids, tokens, topk, E, pad, counts, offs, dest, src, stream)
    assert r(None, 4, 2, 8, 1, P, P, P, P, None) == L.ERR_NULL
    assert r(P, 4, 2, 0, 1, P, P, P, P, None) == L.ERR_SHAPE
    assert r(P, 4, 2, 2048, 1, P, P, P, P, None) == L.ERR_UNSUPPORTED
    assert r(MIS, 4, 2, 8, 1, P, P, P, P, None) == L.ERR_ALIGN
    # 2^20 slots x 1024 experts: 16 MiB of histograms, beyond the 4 MiB scratch
    assert lib.moe_route_workspace_bytes(1 << 20, 1024) > 4 << 20
    assert r(P, 1 << 18, 4, 1024, 1, P, P, P, P, None) == L.ERR_SCRATCH
