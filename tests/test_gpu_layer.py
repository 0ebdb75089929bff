"""GPU parity of the timed layer step: every launch of the step bench.py times, on all five workloads.

The step is built by bench.build_step itself (no copy of its wiring), run twice on the GPU, and each
launch's outputs are checked against the oracle:
  * quantization: codes and scales bit-exact on 1/8 of the rows (rowwise, MX last-dim blocks) or of
    the columns (colwise, MX row blocks), strided so every tile and every column strip is hit, plus
    the padded offsets of the grouped MX calls;
  * grouped GEMMs at their real N and K, on the GPU's own (separately checked) operands: GROUPED_M on
    the first, last and random rows of every expert, GROUPED_K on sampled output rows of every expert
    (empty experts exact zeros).
This covers what no single-kernel test does: the padded row pitch of the grouped colwise outputs,
the K4 e8m0 layout between quantizer and GEMM, the padded offsets the MX weight gradient runs on,
and dgrad operands taken from the batched colwise quantizer.  [P1 Details, Level 2 result (the
MoE layer is the measured unit); P4 "Три уровня оптимизации Triton-ядер".]
"""
import concurrent.futures as cf
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import mxfp8_quantized_moe_amd as fm
from gpu_helpers import note, host, bf16_bits_to_f64, assert_bytes_equal, assert_f32_bits_equal

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
SAMPLE = 8          # quantization: every 8th row or column
POOL = 8            # host threads for the oracle (numpy releases the GIL on array work)


@pytest.fixture(scope="module")
def layer(request):
    cfg = request.param
    note(f"layer step cfg={cfg}: build")
    step, hst = bench.build_step(cfg, gw=(cfg == 2), n_rotate=1, keep_host=True)
    assert sorted(step.specs) == sorted(LAUNCHES[cfg]), sorted(step.specs)
    for i in range(2):
        note(f"layer step cfg={cfg}: run {i}")
        step.run()
        torch.cuda.synchronize()
    yield cfg, step, hst
    del step
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ helpers

def _src(hst, name):
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


CHECKS = {"q_row": check_q_row, "q_col_grouped": check_q_col_grouped, "q_col_batched": check_q_col_batched,
          "mx_last": check_mx_last, "mx_rows_b": check_mx_rows_b, "mx_rows_g": check_mx_rows_g,
          "g_m": check_g_m, "g_k": check_g_k, "g_k_bf16": check_g_k_bf16}


@pytest.mark.parametrize("layer,launch", [(c, n) for c in sorted(LAUNCHES) for n in LAUNCHES[c]],
                         indirect=["layer"], scope="module", ids=[f"cfg{c}-{n.replace(' ', '_')}" for c in sorted(LAUNCHES)
                                                  for n in LAUNCHES[c]])
def test_layer_launch(layer, launch):
    cfg, step, hst = layer
    sp = step.specs[launch]
    note(f"layer step cfg={cfg}: check {launch} ({sp['op']})")
    CHECKS[sp["op"]](sp, hst, phase=cfg + len(launch))
