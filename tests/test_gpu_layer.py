"""GPU parity of the timed layer step: every launch of the step bench.py times, on all five workloads,
and for the MoE workloads both the whole MoE layer (route, gather, W1, SwiGLU, W2, combine and the
mirror backward) and the expert GEMMs alone.

The step is built by bench.build_step itself (no copy of its wiring), run twice on the GPU, and each
launch's outputs are checked against the oracle, with the launch's own device inputs (for the MoE
layer's intermediate tensors, the previous launches' outputs):
  * quantization: codes and scales bit-exact on 1/8 of the rows (rowwise, MX last-dim blocks) or of
    the columns (colwise, MX row blocks), strided so every tile and every column strip is hit, plus
    the padded offsets of the grouped MX calls;
  * grouped GEMMs at their real N and K, on the GPU's own (separately checked) operands: GROUPED_M on
    the first, last and random rows of every expert, GROUPED_K on sampled output rows of every expert
    (empty experts exact zeros).
  * the MoE layer's routing bit-exact (and equal to the workload's routed counts); gathers, SwiGLU,
    combines and their backward on sampled rows or tokens, as in their own tests;
  * end to end, on sampled tokens: the layer's output, the tokens' input gradient and the router
    weights' gradient against an fp64 layer with no quantization, within a relative error that
    FP8 rounding explains, which a wrongly wired operand (another expert, another tensor) exceeds.
This covers what no single-kernel test does: the padded row pitch of the grouped colwise outputs,
the K4 e8m0 layout between quantizer and GEMM, the padded offsets the MX weight gradient runs on,
dgrad operands taken from the batched colwise quantizer, and the MoE layer's dataflow.  [P1
Details, Level 2 result (the MoE layer is the measured unit); P4 "Три уровня оптимизации
Triton-ядер", "MoE".]
"""
import concurrent.futures as cf
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import mxfp8_quantized_moe_amd as fm
from oracle import route as o_route, swiglu as o_swiglu
from gpu_helpers import note, host, bf16_bits_to_f64, assert_bytes_equal, assert_f32_bits_equal, assert_within_one_ulp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu

_FWD_BWD = ["gemm fwd W1", "gemm fwd W2", "gemm dgrad W2", "gemm wgrad W2", "gemm dgrad W1", "gemm wgrad W1"]
LAUNCHES = {
    1: ["q_row X", "q_row W", "gemm fwd"],
    2: ["q_row X", "q_row W", "gemm fwd", "q_row dY", "q_col W", "gemm dgrad", "q_col dY", "q_col X", "gemm wgrad",
        "gemm wgrad bf16"],
    3: ["q_row X", "q_row W1", "q_row A2", "q_row W2", "q_row dY", "q_col W2", "q_col dY", "q_col A2", "q_row dH1",
        "q_col W1", "q_col dH1", "q_col X"] + _FWD_BWD,
    5: ["mx X", "mx W1", "mx A2", "mx W2", "mx dY", "mx W2^T", "mx dY^T", "mx A2^T", "mx dH1", "mx W1^T",
        "mx dH1^T", "mx X^T"] + _FWD_BWD,
}
LAUNCHES[4] = LAUNCHES[3]
LAYER = {
    3: ["route", "permute+q X", "q_row W1", "gemm fwd W1", "swiglu+q", "q_row W2", "gemm fwd W2", "combine",
        "combine bwd+q", "q_col W2", "gemm dgrad W2", "q_col dYg (gathered)", "q_col A2", "gemm wgrad W2",
        "swiglu bwd+q", "q_col W1", "gemm dgrad W1", "q_col dH1", "q_col Xg (gathered)", "gemm wgrad W1",
        "combine dX"],
    5: ["route", "permute+mx Xg (both forms)", "mx W1 (both forms)", "gemm fwd W1", "swiglu+mx A2 (both forms)",
        "mx W2 (both forms)", "gemm fwd W2", "combine", "combine bwd (dw)", "permute+mx dYg (both forms)",
        "gemm dgrad W2",
        "gemm wgrad W2", "swiglu bwd+mx dH1 (both forms)", "gemm dgrad W1", "gemm wgrad W1", "combine dX"],
}
LAYER[4] = LAYER[3]
# (workload, variant): the experts-only steps of configs 3-5 and the whole MoE layer
VARIANTS = {**{(c, "experts"): v for c, v in LAUNCHES.items()}, **{(c, "layer"): v for c, v in LAYER.items()}}
SAMPLE = 8          # quantization: every 8th row or column
POOL = 8            # host threads for the oracle (numpy releases the GIL on array work)
_DEV_CACHE = {}     # host copies of the step's device tensors, per fixture


@pytest.fixture(scope="module")
def layer(request):
    cfg, variant = request.param
    note(f"layer step cfg={cfg} {variant}: build")
    step, hst = bench.build_step(cfg, gw=(cfg == 2), n_rotate=1, keep_host=True, experts_only=(variant == "experts"))
    assert sorted(step.specs) == sorted(VARIANTS[(cfg, variant)]), sorted(step.specs)
    for i in range(2):
        note(f"layer step cfg={cfg} {variant}: run {i}")
        step.run()
        torch.cuda.synchronize()
    _DEV_CACHE.clear()
    yield cfg, step, hst
    _DEV_CACHE.clear()
    del step
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ helpers

def _src(hst, name):
    """A named host input, a host array, or a host copy of a device tensor the step computed."""
    if isinstance(name, np.ndarray):
        return name
    if not isinstance(name, str):
        if id(name) not in _DEV_CACHE:
            _DEV_CACHE[id(name)] = host(name)
        return _DEV_CACHE[id(name)]
    return hst["W1"] if name == "W1" else hst[name]


def _pmap(fn, pieces):
    with cf.ThreadPoolExecutor(POOL) as ex:
        return list(ex.map(fn, pieces))


def _split(idx, n=POOL):
    return [p for p in np.array_split(idx, n) if len(p)]


def _strided(n, phase):
    return np.unique(np.concatenate([np.arange(phase % SAMPLE, n, SAMPLE), [n - 1]])) if n else np.zeros(0, int)


def _k4_to_rows(k4, R, NB):
    """e8m0 scales in the K4 layout [ceil(NB/4), R, 4] -> row-major [R, NB]."""
    G = k4.shape[0]
    return np.ascontiguousarray(k4.transpose(1, 0, 2).reshape(R, 4 * G)[:, :NB])


def _check_gemm(got, ref, contract, tight, what):
    fin = ~np.isnan(ref)
    err = np.abs(got[fin] - ref[fin])
    assert not np.any(np.isnan(got[fin])), f"{what}: NaN in output"
    assert not np.any(err > contract[fin]), f"{what}: {(err > contract[fin]).sum()} beyond the contract bound"
    assert not np.any(err > tight[fin]), f"{what}: {(err > tight[fin]).sum()} beyond the diagnostic bound"


def _deq_f32(q, s_rows):
    return oracle.decode(q, 0) / s_rows.astype(np.float64)[..., None]


def _deq_mx(q, x):
    return oracle.decode(q, 0) * np.repeat(oracle.e8m0_decode(x), 32, axis=-1)


def _group_rows(offs, M, k, seed):
    """Per non-empty group: its first and last row and up to k random rows in between."""
    lo, hi = oracle.group_bounds(offs, M)
    rng = np.random.default_rng(seed)
    out = []
    for e in range(len(lo)):
        n = int(hi[e] - lo[e])
        if n == 0:
            continue
        r = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)])) + lo[e]
        out.append((e, r))
    return out


# ------------------------------------------------------------------ quantization checks

def check_q_row(sp, hst, phase):
    R, C = sp["shape"]
    x = _src(hst, sp["src"]).reshape(R, C)
    rows = _strided(R, phase)
    q, s = host(sp["q"]), host(sp["s"])
    res = _pmap(lambda r: oracle.quantize_rowwise(x[r], 0), _split(rows))
    assert_bytes_equal(q[rows], np.concatenate([a for a, _ in res]), "codes")
    assert_f32_bits_equal(s[rows], np.concatenate([b for _, b in res]), "scales")


def check_q_col_grouped(sp, hst, phase):
    x = _src(hst, sp["src"])
    M, C = x.shape
    cols = _strided(C, phase)
    q, s = host(sp["q"]), host(sp["s"])
    res = _pmap(lambda c: oracle.quantize_colwise_grouped(np.ascontiguousarray(x[:, c]), sp["offs"], 0),
                _split(cols))
    assert_bytes_equal(q[cols, :M], np.concatenate([a for a, _ in res]), "codes (transposed)")
    assert_f32_bits_equal(s[:, cols], np.concatenate([b for _, b in res], axis=1), "scales")


def _gathered(sp, hst):
    """The grouped rows a gathered launch forms from token rows: the oracle's gather, or with router
    weights the routed-row gradients of its combine backward, on the step's own routing."""
    x, rsrc, dest, k = hst[sp["x"]], _src(hst, sp["rsrc"]), _src(hst, sp["dest"]), sp["topk"]
    T, C = x.shape
    if sp["w"] is None:
        return o_route.permute(x, rsrc, k)
    return o_route.combine_backward(x, np.zeros((rsrc.size, C), np.uint16), rsrc, dest, hst[sp["w"]], T, k)[0]


def check_permute_q_col(sp, hst, phase):
    """The gather fused with the grouped colwise quantizer, checked as check_q_col_grouped checks a tensor
    in memory."""
    check_q_col_grouped(dict(src=_gathered(sp, hst), offs=sp["offs"], q=sp["q"], s=sp["s"]), hst, phase)


def check_q_col_batched(sp, hst, phase):
    B, R, C = sp["shape"]
    x = _src(hst, sp["src"]).reshape(B, R, C)
    cols = _strided(C, phase)
    q, s = host(sp["q"]), host(sp["s"])
    res = _pmap(lambda c: oracle.quantize_colwise_batched(np.ascontiguousarray(x[:, :, c]), 0), _split(cols))
    assert_bytes_equal(q[:, cols, :], np.concatenate([a for a, _ in res], axis=1), "codes (transposed)")
    assert_f32_bits_equal(s[:, cols], np.concatenate([b for _, b in res], axis=1), "scales")


def check_mx_last(sp, hst, phase):
    R, C = sp["shape"]
    x = _src(hst, sp["src"]).reshape(R, C)
    rows = _strided(R, phase)
    q = host(sp["q"])
    sc = _k4_to_rows(host(sp["s"]), R, C // 32)
    res = _pmap(lambda r: oracle.quantize_mx_lastdim(x[r], sp["rule"]), _split(rows))
    assert_bytes_equal(q[rows], np.concatenate([a for a, _ in res]), "codes")
    assert_bytes_equal(sc[rows], np.concatenate([b for _, b in res]), "e8m0")
    k4 = host(sp["s"])                          # bytes past a row's last block are zero
    if (C // 32) % 4:
        assert not k4[-1, :, (C // 32) % 4:].any()


def check_mx_rows_b(sp, hst, phase):
    B, R, C = sp["shape"]
    x = _src(hst, sp["src"]).reshape(B, R, C)
    cols = _strided(C, phase)
    q = host(sp["q"])
    sc = _k4_to_rows(host(sp["s"]), B * C, R // 32).reshape(B, C, R // 32)
    res = _pmap(lambda c: oracle.quantize_mx_rows_batched(np.ascontiguousarray(x[:, :, c]), sp["rule"]),
                _split(cols))
    assert_bytes_equal(q[:, cols, :], np.concatenate([a for a, _ in res], axis=1), "codes (transposed)")
    assert_bytes_equal(sc[:, cols, :], np.concatenate([b for _, b in res], axis=1), "e8m0")


def check_mx_rows_g(sp, hst, phase):
    x = _src(hst, sp["src"])
    M, C = x.shape
    Mp = sp["rows_pad"]
    cols = _strided(C, phase)
    q = host(sp["q"])
    sc = _k4_to_rows(host(sp["s"]), C, Mp // 32)
    res = _pmap(lambda c: oracle.quantize_mx_rows_grouped(np.ascontiguousarray(x[:, c]), sp["offs"], sp["rule"], Mp),
                _split(cols))
    assert_bytes_equal(q[cols], np.concatenate([a for a, _, _ in res]), "codes (transposed, padded)")
    assert_bytes_equal(sc[cols], np.concatenate([b for _, b, _ in res]), "e8m0")
    assert_bytes_equal(host(sp["offs_pad"]), res[0][2], "padded offsets")


def check_mx_dual(sp, hst, phase):
    """Both MX forms from one read: the last-dim half as check_mx_last, the row-block half as
    check_mx_rows_b (batched) or check_mx_rows_g (grouped)."""
    last = dict(src=sp["src"], rule=sp["rule"], q=sp["q"], s=sp["s"])
    if "offs" in sp:
        last["shape"] = sp["shape"]
        check_mx_last(last, hst, phase)
        check_mx_rows_g(dict(src=sp["src"], offs=sp["offs"], rows_pad=sp["rows_pad"], rule=sp["rule"], q=sp["qt"],
                             s=sp["st"], offs_pad=sp["offs_pad"]), hst, phase)
    else:
        B, R, C = sp["shape"]
        last["shape"] = (B * R, C)
        check_mx_last(last, hst, phase)
        check_mx_rows_b(dict(src=sp["src"], shape=sp["shape"], rule=sp["rule"], q=sp["qt"], s=sp["st"]), hst, phase)


def check_permute_mx_dual(sp, hst, phase):
    """The gather into the grouped layout fused with both MX forms: the gathered rows (times the router
    weights for the routed-row gradients) are formed here by the oracle's permute (or combine backward)
    from the step's own routing, then checked as check_mx_dual checks a tensor in memory."""
    g = _gathered(sp, hst)
    check_mx_dual(dict(src=g, shape=sp["shape"], offs=sp["offs"], rows_pad=sp["rows_pad"], rule=sp["rule"],
                       q=sp["q"], s=sp["s"], qt=sp["qt"], st=sp["st"], offs_pad=sp["offs_pad"]), hst, phase)


def check_swiglu_mx(sp, hst, phase):
    """SwiGLU (or its backward) fused with both MX forms: the launch's outputs equal those of the same entry
    point asked to also write the bf16 tensor it quantizes, and that tensor is checked against the oracle
    (within one bf16 ulp on sampled rows, then both MX forms bit-exact against the oracle's quantizers of it)."""
    h1 = sp["h1"]
    offs_d = torch.from_numpy(np.asarray(sp["offs"], np.int32)).to(h1.device)
    F = sp["F"]
    R = h1.shape[0]
    C = F if sp["da2"] is None else 2 * F
    copy = torch.empty(R, C, dtype=torch.bfloat16, device=h1.device)
    if sp["da2"] is None:
        r = fm.swiglu_quantize_mx_dual(h1, offs_d, rule=sp["rule"], rows_pad=sp["rows_pad"], a2=copy)
    else:
        r = fm.swiglu_backward_quantize_mx_dual(sp["da2"], h1, offs_d, rule=sp["rule"], rows_pad=sp["rows_pad"],
                                                dh1=copy)
    for got, want, what in zip((sp["q"], sp["s"], sp["qt"], sp["st"], sp["offs_pad"]), r[1:],
                               ("last-dim codes", "last-dim e8m0", "row-block codes", "row-block e8m0",
                                "padded offsets")):
        assert torch.equal(got, want), f"{what} differ from the run that writes the bf16 tensor"
    rows = _strided(R, phase)[::4]
    h1h = _src(hst, h1)[rows]
    t = host(copy)
    ref = o_swiglu.swiglu_fwd(h1h, F) if sp["da2"] is None else o_swiglu.swiglu_bwd(_src(hst, sp["da2"])[rows], h1h, F)
    assert_within_one_ulp(t[rows], ref, "bf16 tensor")
    _DEV_CACHE[id(copy)] = t
    check_mx_dual(dict(src=copy, shape=(R, C), offs=sp["offs"], rows_pad=sp["rows_pad"], rule=sp["rule"],
                       q=sp["q"], s=sp["s"], qt=sp["qt"], st=sp["st"], offs_pad=sp["offs_pad"]), hst, phase)
    del _DEV_CACHE[id(copy)]


# ------------------------------------------------------------------ GEMM checks

def _mx(sp):
    return sp["sk"] in (fm.SCALE_E8M0, fm.SCALE_E8M0_K4)


def check_g_m(sp, hst, phase):
    M, N, K = sp["M"], sp["N"], sp["K"]
    offs = sp["offs"]
    E = len(offs)
    got = bf16_bits_to_f64(host(sp["out"]))
    qa, qb = host(sp["qa"]), host(sp["qb"]).reshape(E, N, K)
    if _mx(sp):
        sa = _k4_to_rows(host(sp["sa"]), M, K // 32)
        sb = _k4_to_rows(host(sp["sb"]), E * N, K // 32).reshape(E, N, K // 32)
    else:
        sa, sb = host(sp["sa"]), host(sp["sb"]).reshape(E, N)
    for e, rows in _group_rows(offs, M, 4, 100 + phase):
        one = np.array([len(rows)], np.int32)
        if _mx(sp):
            ref = oracle.mm_grouped_m_mx(qa[rows], sa[rows], qb[e:e + 1], sb[e:e + 1], one)
            A, B = _deq_mx(qa[rows], sa[rows]), _deq_mx(qb[e:e + 1], sb[e:e + 1])
        else:
            ref = oracle.mm_grouped_m(qa[rows], sa[rows], qb[e:e + 1], sb[e:e + 1], one, 0, 0)
            A, B = _deq_f32(qa[rows], sa[rows]), _deq_f32(qb[e:e + 1], sb[e:e + 1])
        contract, tight = oracle.error_bounds_m(A, B, one, oracle.ACC_FP8_MFMA)
        _check_gemm(got[rows], ref, contract, tight, f"expert {e}")


def check_g_k(sp, hst, phase):
    Mc, N, K = sp["M"], sp["N"], sp["K"]
    offs = sp["offs"] if isinstance(sp["offs"], np.ndarray) else host(sp["offs"])
    E = len(offs)
    got = bf16_bits_to_f64(host(sp["out"]))
    n_rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(200 + phase).choice(N, 14, replace=False)]))
    qa, qb = host(sp["qa"])[n_rows, :Mc], host(sp["qb"])[:, :Mc]
    if _mx(sp):
        sa = _k4_to_rows(host(sp["sa"]), N, Mc // 32)[n_rows]
        sb = _k4_to_rows(host(sp["sb"]), K, Mc // 32)
        ref = oracle.mm_grouped_k_mx(qa, sa, qb, sb, offs)
        A, B = _deq_mx(qa, sa), _deq_mx(qb, sb)
        contract, tight = oracle.error_bounds_k(A, B, offs, oracle.ACC_FP8_MFMA)
    else:
        sa, sb = host(sp["sa"])[:, n_rows], host(sp["sb"])
        ref = oracle.mm_grouped_k(qa, sa, qb, sb, offs, 0, 0)
        lo, hi = oracle.group_bounds(offs, Mc)
        contract = np.zeros_like(ref)
        tight = np.zeros_like(ref)
        Aq, Bq = oracle.decode(qa, 0), oracle.decode(qb, 0)
        for e in range(E):          # each group's columns carry that group's scales
            if hi[e] == lo[e]:
                continue
            A = Aq[:, lo[e]:hi[e]] / sa[e].astype(np.float64)[:, None]
            B = Bq[:, lo[e]:hi[e]] / sb[e].astype(np.float64)[:, None]
            one = np.array([hi[e] - lo[e]], np.int32)
            c, t = oracle.error_bounds_k(A, B, one, oracle.ACC_FP8_MFMA)
            contract[e], tight[e] = c[0], t[0]
    lo, hi = oracle.group_bounds(offs, Mc)
    for e in range(E):
        if hi[e] == lo[e]:
            assert not got[e].any(), f"empty expert {e}: not exact zeros"
    _check_gemm(got[:, n_rows], ref, contract, tight, "weight gradient")


def check_g_k_bf16(sp, hst, phase):
    a, b = hst[sp["a"]], hst[sp["b"]]
    offs = sp["offs"]
    N = a.shape[1]
    got = bf16_bits_to_f64(host(sp["out"]))
    n_rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(300 + phase).choice(N, 14, replace=False)]))
    ar = np.ascontiguousarray(a[:, n_rows])
    ref = oracle.mm_grouped_k_bf16(ar, b, offs)
    contract, tight = oracle.error_bounds_k(bf16_bits_to_f64(np.ascontiguousarray(ar.T)),
                                            bf16_bits_to_f64(np.ascontiguousarray(b.T)), offs)
    _check_gemm(got[:, n_rows], ref, contract, tight, "bf16 weight gradient")


# ------------------------------------------------------------------ MoE layer checks

def check_route(sp, hst, phase):
    ref = o_route.route(hst[sp["ids"]], sp["E"], sp["pad"])
    for nm, g, r in zip(("counts", "offs", "dest", "src"), sp["out"], ref):
        assert_bytes_equal(_src(hst, g), r, f"route {nm}")


def _rows_sample(n, phase):
    return _strided(n, phase)


def check_permute(sp, hst, phase):
    x, rsrc = _src(hst, sp["src"]), _src(hst, sp["rsrc"])
    rows = _rows_sample(rsrc.size, phase)
    assert_bytes_equal(_src(hst, sp["out"])[rows], o_route.permute(x, rsrc[rows], sp["topk"]), "gathered rows")


def check_permute_rowwise(sp, hst, phase):
    x, rsrc = _src(hst, sp["src"]), _src(hst, sp["rsrc"])
    rows = _rows_sample(rsrc.size, phase)
    xg = o_route.permute(x, rsrc[rows], sp["topk"])
    if sp["xg"] is not None:                            # the bf16 copy is optional
        assert_bytes_equal(_src(hst, sp["xg"])[rows], xg, "gathered rows")
    q, s = oracle.quantize_rowwise(xg, 0)
    assert_bytes_equal(_src(hst, sp["q"])[rows], q, "codes")
    assert_f32_bits_equal(_src(hst, sp["s"])[rows], s, "scales")


def check_swiglu(sp, hst, phase):
    h1 = _src(hst, sp["h1"])
    rows = _rows_sample(h1.shape[0], phase)
    a2 = _src(hst, sp["a2"])[rows]
    assert_within_one_ulp(a2, o_swiglu.swiglu_fwd(h1[rows], sp["F"]), "a2")
    if sp["q"] is not None:
        q, s = oracle.quantize_rowwise(a2, 0)
        assert_bytes_equal(_src(hst, sp["q"])[rows], q, "a2 codes")
        assert_f32_bits_equal(_src(hst, sp["s"])[rows], s, "a2 scales")


def check_swiglu_bwd(sp, hst, phase):
    h1, da2 = _src(hst, sp["h1"]), _src(hst, sp["da2"])
    rows = _rows_sample(h1.shape[0], phase)
    dh1 = _src(hst, sp["dh1"])[rows]
    assert_within_one_ulp(dh1, o_swiglu.swiglu_bwd(da2[rows], h1[rows], sp["F"]), "dh1")
    if sp["q"] is not None:
        q, s = oracle.quantize_rowwise(dh1, 0)
        assert_bytes_equal(_src(hst, sp["q"])[rows], q, "dh1 codes")
        assert_f32_bits_equal(_src(hst, sp["s"])[rows], s, "dh1 scales")


def _token_sample(T, phase):
    return np.unique(np.concatenate([[0, T - 1], np.random.default_rng(400 + phase).choice(T, 255, replace=False)]))


def _sub_routing(dest, toks, k):
    """The grouped rows the sampled tokens use, renumbered: (rows to take, dest of the sub-problem)."""
    d = dest.reshape(-1, k)[toks].ravel()
    return np.clip(d, 0, None), np.where(d >= 0, np.arange(d.size), -1).astype(np.int32)


def check_combine(sp, hst, phase):
    yg, dest, k = _src(hst, sp["yg"]), _src(hst, sp["dest"]), sp["topk"]
    T = dest.size // k
    toks = _token_sample(T, phase)
    take, d_sub = _sub_routing(dest, toks, k)
    wts = None if sp["w"] is None else hst[sp["w"]][toks]
    assert_bytes_equal(_src(hst, sp["out"])[toks], o_route.combine(yg[take], d_sub, wts, len(toks), k), "combined")


def check_combine_bwd(sp, hst, phase):
    yg, dest, rsrc, k = _src(hst, sp["yg"]), _src(hst, sp["dest"]), _src(hst, sp["src"]), sp["topk"]
    dy, wts = hst[sp["dy"]], hst[sp["w"]]
    T = dest.size // k
    toks = _token_sample(T, phase)
    take, d_sub = _sub_routing(dest, toks, k)
    s_sub = np.arange(d_sub.size, dtype=np.int32)
    dyg_ref, dw_ref = o_route.combine_backward(dy[toks], yg[take], s_sub, d_sub, wts[toks], len(toks), k)
    dyg = _src(hst, sp["dyg"]) if sp["dyg"] is not None else None     # None: router-weight gradients only
    if dyg is not None:
        assert_bytes_equal(dyg[take], dyg_ref, "routed-row gradients")
    if sp["q"] is not None:
        q, s = oracle.quantize_rowwise(dyg_ref, 0)
        assert_bytes_equal(_src(hst, sp["q"])[take], q, "codes")
        assert_f32_bits_equal(_src(hst, sp["s"])[take], s, "scales")
    slots = (toks[:, None] * k + np.arange(k)[None, :]).ravel()
    dw = _src(hst, sp["dw"])[slots].astype(np.float64)
    mag = np.einsum("sc,sc->s", np.abs(bf16_bits_to_f64(dy[toks]).repeat(k, axis=0)),
                    np.abs(bf16_bits_to_f64(yg[take])))
    assert np.all(np.abs(dw - dw_ref) <= dy.shape[1] * 2.0 ** -24 * mag), "router-weight gradients"
    if dyg is not None:
        pad = rsrc < 0                                  # rows holding no slot are zeros
        assert not dyg[pad].any()


CHECKS = {"q_row": check_q_row, "q_col_grouped": check_q_col_grouped, "q_col_batched": check_q_col_batched,
          "mx_last": check_mx_last, "mx_rows_b": check_mx_rows_b, "mx_rows_g": check_mx_rows_g,
          "g_m": check_g_m, "g_k": check_g_k, "g_k_bf16": check_g_k_bf16,
          "mx_dual": check_mx_dual, "permute_mx_dual": check_permute_mx_dual, "permute_q_col": check_permute_q_col, "swiglu_mx": check_swiglu_mx, "route": check_route, "permute": check_permute, "permute_rowwise": check_permute_rowwise,
          "swiglu": check_swiglu, "swiglu_bwd": check_swiglu_bwd, "combine": check_combine,
          "combine_bwd": check_combine_bwd}


_CASES = [(v, n) for v in sorted(VARIANTS) for n in VARIANTS[v]]


@pytest.mark.parametrize("layer,launch", _CASES, indirect=["layer"], scope="module",
                         ids=[f"cfg{c}-{v}-{n.replace(' ', '_')}" for (c, v), n in _CASES])
def test_layer_launch(layer, launch):
    cfg, step, hst = layer
    sp = step.specs[launch]
    note(f"layer step cfg={cfg}: check {launch} ({sp['op']})")
    CHECKS[sp["op"]](sp, hst, phase=cfg + len(launch))


def _swiglu64(h, F):
    g, u = h[:, :F], h[:, F:]
    return g / (1.0 + np.exp(-g)) * u


@pytest.mark.parametrize("layer", [(c, "layer") for c in sorted(LAYER)], indirect=True, scope="module",
                         ids=[f"cfg{c}-layer" for c in sorted(LAYER)])
def test_layer_end_to_end(layer):
    """The MoE layer's output y, the tokens' input gradient dx and the router weights' gradient dw on
    8 sampled tokens, against an fp64 layer with no quantization computed here from the host inputs:
    y[t] = sum_j w[t,j] W2[e_j] swiglu(W1[e_j] x[t]), and its gradients for the loss <dy, y>.  FP8
    keeps 3 significand bits: a quantized operand's elements carry a relative rounding error of at
    most 2^-4 (about 0.036 root mean square), and a pass chains four quantized operands (x, W1, a2,
    W2 forward), so the layer's relative error is about 2 x 0.036, 0.07; measured worst cases over
    the sampled tokens are 0.07-0.11.  Bound 0.25.  A router-weight gradient is one dot product
    <dy, y_e> whose exact value may sit near zero, so its error is taken against the size such a
    product has, |dy| |y_e| / sqrt(H) (measured worst 0.13-0.17), bound 0.4.  Another expert's
    weights, an unweighted combine or a transposed operand give errors of order 1 (another
    expert: about sqrt(2))."""
    cfg, step, hst = layer
    k = hst["IDS"].shape[1]
    X, DY, RW, IDS = hst["X"], hst["DY"], hst["RW"], hst["IDS"]
    W1, W2 = hst["W1"], hst["W2"]
    F2, H = W1.shape[1], W1.shape[2]
    F = F2 // 2
    out = step.outputs
    y, dx, dw = host(out["y"]), host(out["dx"]), host(out["dw"])
    toks = np.random.default_rng(cfg).choice(X.shape[0], 8, replace=False)
    errs = {"y": [], "dx": [], "dw": []}
    for t in toks:
        x = bf16_bits_to_f64(X[t])
        dyt = bf16_bits_to_f64(DY[t])
        y_ref = np.zeros(H)
        dx_ref = np.zeros(H)
        dw_ref = np.zeros(k)
        dw_scale = np.zeros(k)
        for j in range(k):
            e = int(IDS[t, j])
            w1, w2 = bf16_bits_to_f64(W1[e]), bf16_bits_to_f64(W2[e])
            h1 = w1 @ x                                   # [2F]
            g, u = h1[:F], h1[F:]
            sg = 1.0 / (1.0 + np.exp(-g))
            a2 = g * sg * u
            ye = w2 @ a2                                  # [H]
            y_ref += float(RW[t, j]) * ye
            dw_ref[j] = dyt @ ye
            dw_scale[j] = np.linalg.norm(dyt) * np.linalg.norm(ye) / np.sqrt(H)
            da2 = (float(RW[t, j]) * dyt) @ w2            # [F]
            dh1 = np.concatenate([da2 * u * sg * (1.0 + g * (1.0 - sg)), da2 * g * sg])
            dx_ref += dh1 @ w1
        rel = lambda got, ref: float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
        errs["y"].append(rel(bf16_bits_to_f64(y[t]), y_ref))
        errs["dx"].append(rel(bf16_bits_to_f64(dx[t]), dx_ref))
        errs["dw"].append(float(np.max(np.abs(dw[t * k:(t + 1) * k].astype(np.float64) - dw_ref) / dw_scale)))
    note(f"end to end cfg={cfg}: worst relative error " + ", ".join(f"{n} {max(v):.3e}" for n, v in errs.items()))
    for n, bound in (("y", 0.25), ("dx", 0.25), ("dw", 0.4)):
        assert max(errs[n]) < bound, f"{n}: relative error {max(errs[n]):.3e} on a sampled token"
