"""Pins for the oracle's grouped GEMMs (CPU only).

Independent checks: pure-Python triple loops over decoded codes (exact
rational arithmetic through ``fractions``) on tiny inputs, integer-valued
operands whose products are exact integers, the E = 1 case against a plain
dense product, and planted mistakes (transposed operand, dropped scale) that
the acceptance bound must reject.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import E4M3FN, E4M3FNUZ
from mxfp8_quantized_moe_amd.synth import normal_bf16


def dec_frac(code: int, codec: int) -> Fraction:
    """Exact value of an FP8 code from its fields (independent of the oracle table)."""
    bias = 7 if codec == E4M3FN else 8
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(2) ** (1 - bias)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - bias)


def rand_codes(rng, shape, codec):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    bad = (q & 0x7F) == 0x7F if codec == E4M3FN else q == 0x80
    q[bad] = 0x3C
    return q


def test_grouped_m_brute_force_exact():
    rng = np.random.default_rng(1)
    M, N, K, E = 13, 5, 24, 4
    qa = rand_codes(rng, (M, K), E4M3FN)
    qb = rand_codes(rng, (E, N, K), E4M3FNUZ)
    sa = rng.uniform(0.5, 4, M).astype(np.float32)
    sb = rng.uniform(0.5, 4, (E, N)).astype(np.float32)
    offs = np.array([4, 4, 9, 11], np.int32)                 # 4, 0, 5, 2 rows; rows 11, 12 unrouted
    out = oracle.mm_grouped_m(qa, sa, qb, sb, offs, E4M3FN, E4M3FNUZ)
    grp = [0] * 4 + [2] * 5 + [3] * 2
    for m in range(M):
        for n in range(N):
            if m >= 11:
                assert np.isnan(out[m, n])
                continue
            e = grp[m]
            acc = sum(dec_frac(int(qa[m, k]), E4M3FN) * dec_frac(int(qb[e, n, k]), E4M3FNUZ) for k in range(K))
            ref = acc / (Fraction(float(sa[m])) * Fraction(float(sb[e, n])))
            assert out[m, n] == float(ref)      # dot exact, one fp64 rounding in the division


def test_grouped_k_brute_force_exact():
    rng = np.random.default_rng(2)
    N, K, M = 4, 3, 17
    offs = np.array([6, 6, 17], np.int32)
    qa = rand_codes(rng, (N, M), E4M3FN)
    qb = rand_codes(rng, (K, M), E4M3FN)
    sa = rng.uniform(0.5, 4, (3, N)).astype(np.float32)
    sb = rng.uniform(0.5, 4, (3, K)).astype(np.float32)
    out = oracle.mm_grouped_k(qa, sa, qb, sb, offs, E4M3FN, E4M3FN)
    bounds = [(0, 6), (6, 6), (6, 17)]
    for e, (lo, hi) in enumerate(bounds):
        for n in range(N):
            for k in range(K):
                acc = sum(dec_frac(int(qa[n, m]), 0) * dec_frac(int(qb[k, m]), 0) for m in range(lo, hi))
                ref = acc / (Fraction(float(sa[e, n])) * Fraction(float(sb[e, k])))
                assert out[e, n, k] == float(ref)
    assert not out[1].any()                                   # empty group -> exact zeros


def test_integer_valued_operands_give_integer_products():
    # e4m3fn codes of small integers: 1 -> 0x38, 2 -> 0x40, 3 -> 0x44, -1 -> 0xB8, 0 -> 0
    vals = {0x38: 1, 0x40: 2, 0x44: 3, 0xB8: -1, 0x00: 0}
    rng = np.random.default_rng(3)
    keys = np.array(list(vals))
    qa = keys[rng.integers(0, 5, (8, 40))].astype(np.uint8)
    qb = keys[rng.integers(0, 5, (2, 6, 40))].astype(np.uint8)
    ones_a = np.ones(8, np.float32)
    ones_b = np.ones((2, 6), np.float32)
    out = oracle.mm_grouped_m(qa, ones_a, qb, ones_b, np.array([3, 8], np.int32), E4M3FN, E4M3FN)
    ia = np.vectorize(vals.get)(qa).astype(object)
    ib = np.vectorize(vals.get)(qb).astype(object)
    for m in range(8):
        e = 0 if m < 3 else 1
        for n in range(6):
            assert out[m, n] == sum(ia[m, k] * ib[e, n, k] for k in range(40))


def test_single_group_is_dense_scaled_gemm():
    rng = np.random.default_rng(4)
    qa = rand_codes(rng, (32, 64), E4M3FN)
    qb = rand_codes(rng, (1, 16, 64), E4M3FN)
    sa = rng.uniform(1, 2, 32).astype(np.float32)
    sb = rng.uniform(1, 2, (1, 16)).astype(np.float32)
    out = oracle.mm_grouped_m(qa, sa, qb, sb, np.array([32], np.int32), E4M3FN, E4M3FN)
    tab = np.array([float(dec_frac(c, 0)) if (c & 0x7F) != 0x7F else 0.0 for c in range(256)])
    dense = np.einsum("mk,nk->mn", tab[qa], tab[qb[0]]) / np.outer(sa.astype(np.float64), sb[0].astype(np.float64))
    assert np.array_equal(out, dense)


@pytest.mark.parametrize("mode", ["m", "k"])
def test_mx_gemm_brute_force(mode):
    rng = np.random.default_rng(5)
    if mode == "m":
        M, N, K = 6, 3, 64
        qa = rand_codes(rng, (M, K), 0)
        qb = rand_codes(rng, (2, N, K), 0)
        xa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
        xb = rng.integers(110, 140, (2, N, K // 32)).astype(np.uint8)
        offs = np.array([2, 6], np.int32)
        out = oracle.mm_grouped_m_mx(qa, xa, qb, xb, offs)
        for m in range(M):
            e = 0 if m < 2 else 1
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    acc += (dec_frac(int(qa[m, k]), 0) * Fraction(2) ** (int(xa[m, k // 32]) - 127)
                            * dec_frac(int(qb[e, n, k]), 0) * Fraction(2) ** (int(xb[e, n, k // 32]) - 127))
                assert abs(out[m, n] - float(acc)) <= 2.0 ** -50 * abs(float(acc)) + 1e-300
    else:
        N, K, Mp = 3, 2, 96
        qa = rand_codes(rng, (N, Mp), 0)
        qb = rand_codes(rng, (K, Mp), 0)
        xa = rng.integers(110, 140, (N, Mp // 32)).astype(np.uint8)
        xb = rng.integers(110, 140, (K, Mp // 32)).astype(np.uint8)
        offs = np.array([32, 32, 96], np.int32)
        out = oracle.mm_grouped_k_mx(qa, xa, qb, xb, offs)
        for e, (lo, hi) in enumerate([(0, 32), (32, 32), (32, 96)]):
            for n in range(N):
                for k in range(K):
                    acc = Fraction(0)
                    for m in range(lo, hi):
                        acc += (dec_frac(int(qa[n, m]), 0) * Fraction(2) ** (int(xa[n, m // 32]) - 127)
                                * dec_frac(int(qb[k, m]), 0) * Fraction(2) ** (int(xb[k, m // 32]) - 127))
                    assert abs(out[e, n, k] - float(acc)) <= 2.0 ** -50 * abs(float(acc)) + 1e-300
        assert not out[1].any()


def test_bf16_grouped_k_brute_force():
    a = normal_bf16(6, (10, 3), 1.0)
    b = normal_bf16(7, (10, 4), 1.0)
    offs = np.array([0, 7, 10], np.int32)
    out = oracle.mm_grouped_k_bf16(a, b, offs)
    av = oracle.bf16_to_f32(a).astype(np.float64)
    bv = oracle.bf16_to_f32(b).astype(np.float64)
    assert not out[0].any()
    for e, (lo, hi) in [(1, (0, 7)), (2, (7, 10))]:
        for n in range(3):
            for k in range(4):
                ref = sum(Fraction(float(av[m, n])) * Fraction(float(bv[m, k])) for m in range(lo, hi))
                assert out[e, n, k] == float(ref)


def test_bounds_reject_planted_mistakes():
    """A transposed operand or a dropped scale must exceed the contract bound."""
    x = normal_bf16(8, (64, 128), 1.0)
    w = normal_bf16(9, (1, 48, 128), 0.02)
    qa, sa = oracle.quantize_rowwise(x, E4M3FN)
    qb, sb = oracle.quantize_rowwise(w[0], E4M3FN)
    qb, sb = qb[None], sb[None]
    offs = np.array([64], np.int32)
    ref = oracle.mm_grouped_m(qa, sa, qb, sb, offs, E4M3FN, E4M3FN)
    A = oracle.decode(qa, 0) / sa[:, None]
    B = oracle.decode(qb, 0) / sb[..., None]
    contract, tight = oracle.error_bounds_m(A, B, offs)
    assert np.all(np.abs(ref - A @ B[0].T) <= tight)          # the reference meets its own bound
    dropped = ref * float(sb[0, 0])                            # forgot one weight scale
    assert np.any(np.abs(dropped - ref) > contract)
    rng = np.random.default_rng(0)
    perm = rng.permutation(128)
    wrong_k = oracle.mm_grouped_m(qa[:, perm], sa, qb, sb, offs, E4M3FN, E4M3FN)   # mis-indexed K
    assert np.any(np.abs(wrong_k - ref) > contract)


def _bounds_k_by_hand(A, B, lo, hi, acc):
    """Pure-Python loops: the GROUPED_K contract bound 1e-2 * |a_row| * |b_col| and the diagnostic
    2^-8 |ref| + rel * sum|a*b|, norms and sums over the group's tokens [lo, hi) only."""
    N, K = A.shape[0], B.shape[0]
    contract = [[0.0] * K for _ in range(N)]
    tight = [[0.0] * K for _ in range(N)]
    rel = max(hi - lo, 1) * 2.0 ** -23 if acc == oracle.ACC_FP32 else 2.0 ** -10
    for n in range(N):
        na = sum(float(A[n, m]) ** 2 for m in range(lo, hi)) ** 0.5
        for k in range(K):
            nb = sum(float(B[k, m]) ** 2 for m in range(lo, hi)) ** 0.5
            ref = sum(Fraction(float(A[n, m])) * Fraction(float(B[k, m])) for m in range(lo, hi))
            absdot = sum(abs(Fraction(float(A[n, m])) * Fraction(float(B[k, m]))) for m in range(lo, hi))
            contract[n][k] = 1e-2 * na * nb
            tight[n][k] = 2.0 ** -8 * abs(float(ref)) + rel * float(absdot)
    return np.array(contract), np.array(tight)


@pytest.mark.parametrize("acc", [oracle.ACC_FP32, oracle.ACC_FP8_MFMA])
def test_error_bounds_k_brute_force_two_groups(acc):
    """Per group, norms and |a*b| sums run over that group's tokens only; an empty group (and a
    decreasing offset) gets zero bounds, so only exact zeros pass there."""
    rng = np.random.default_rng(21)
    N, K, M = 3, 4, 11
    A = rng.standard_normal((N, M)) * np.array([10.0] * 4 + [0.01] * 7)   # group 0 tokens much larger
    B = rng.standard_normal((K, M))
    offs = np.array([4, 4, 11, 9], np.int32)                           # groups [0,4), [], [4,11), []
    contract, tight = oracle.error_bounds_k(A, B, offs, acc)
    assert contract.shape == tight.shape == (4, N, K)
    for e, (lo, hi) in enumerate([(0, 4), (4, 4), (4, 11), (11, 11)]):
        c, t = _bounds_k_by_hand(A, B, lo, hi, acc)
        np.testing.assert_allclose(contract[e], c, rtol=1e-12, atol=0)
        np.testing.assert_allclose(tight[e], t, rtol=1e-12, atol=0)
    assert not contract[1].any() and not contract[3].any()


def test_error_bounds_k_catches_slicing_mistakes():
    """Planted mistakes about the group's token range.  (1) A bound that takes its norms over all M
    tokens instead of the group's disagrees with the loops above.  (2) A weight gradient of group 1
    that drops the group's last token (an off-by-one slicing mistake in a kernel) is outside the
    real bound, but inside the loosened bound of mistake (1); so is (3) one that contracts group 1
    over every token."""
    rng = np.random.default_rng(22)
    N, K, M = 5, 6, 40
    scale = np.where(np.arange(M) < 24, 1.0, 1e-3)                    # group 0 dominates the norms
    A = rng.standard_normal((N, M)) * scale
    B = rng.standard_normal((K, M)) * scale
    offs = np.array([24, 40], np.int32)

    def bounds_over_all_tokens(A_t, B_t, offs_, acc=oracle.ACC_FP32):   # the planted mistake (1)
        c, t = oracle.error_bounds_k(A_t, B_t, np.array([A_t.shape[1]], np.int32), acc)
        return np.repeat(c, len(offs_), 0), np.repeat(t, len(offs_), 0)

    c_bad, _ = bounds_over_all_tokens(A, B, offs)
    c_hand, _ = _bounds_k_by_hand(A, B, 24, 40, oracle.ACC_FP32)
    assert not np.allclose(c_bad[1], c_hand, rtol=1e-6)                 # the loops catch it
    contract, _ = oracle.error_bounds_k(A, B, offs)
    np.testing.assert_allclose(contract[1], c_hand, rtol=1e-12)
    ref1 = A[:, 24:] @ B[:, 24:].T
    short1 = A[:, 24:39] @ B[:, 24:39].T                                # mistake (2): last token dropped
    assert np.any(np.abs(short1 - ref1) > contract[1])
    assert np.all(np.abs(short1 - ref1) <= c_bad[1])                   # the mutant bound would pass it
    wrong1 = A @ B.T                                                    # mistake (3): every token
    assert np.any(np.abs(wrong1 - ref1) > contract[1])
