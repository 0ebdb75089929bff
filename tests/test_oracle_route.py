"""Pins of the routing oracle (oracle/route.py): pure-Python loops, the
structural invariants of a stable grouping, special routings, and a round
trip through permute and combine."""
import numpy as np
import pytest

import oracle
from oracle import route as rt
from oracle.swiglu import round_bf16


def loops_route(ids, E, pad):
    """Straight loops: experts in order, slots in order within each."""
    flat = [int(v) for v in np.asarray(ids).ravel()]
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    dest = [-1] * len(flat)
    src = [-1] * (len(flat) + E * (pad - 1))
    row, offs = 0, []
    for e in range(E):
        for i, v in enumerate(flat):
            if v == e:
                dest[i] = row
                src[row] = i
                row += 1
        row += (-counts[e]) % pad
        offs.append(row)
    return counts, offs, dest, src


CASES = [
    (np.array([[2, 0, 1], [1, 2, 4], [0, 0, 3], [4, 1, 2], [2, 3, 0], [1, 1, 4], [3, 2, 0]]), 5, 1),
    (np.array([[2, 0, 1], [1, 2, 4], [0, 0, 3], [4, 1, 2], [2, 3, 0], [1, 1, 4], [3, 2, 0]]), 5, 4),
    (np.zeros((9, 2), dtype=int), 3, 1),                  # every slot to expert 0; experts 1, 2 empty
    (np.zeros((9, 2), dtype=int), 3, 8),
    (np.arange(12).reshape(12, 1) % 4, 4, 1),             # topk 1, round robin
    (np.array([[0, 7], [-1, 2], [2, 2], [5, 1]]), 6, 2),  # ids 7 and -1 drop their slots
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_route_matches_loops(case):
    ids, E, pad = CASES[case]
    counts, offs, dest, src = rt.route(ids, E, pad)
    lc, lo, ld, ls = loops_route(ids, E, pad)
    assert counts.tolist() == lc and offs.tolist() == lo and dest.tolist() == ld and src.tolist() == ls


def test_route_invariants_random():
    rng = np.random.default_rng(0)
    for trial in range(20):
        T, k, E, pad = int(rng.integers(1, 300)), int(rng.integers(1, 7)), int(rng.integers(1, 70)), \
            int(rng.choice([1, 16, 32]))
        ids = rng.integers(0, E, size=(T, k))
        counts, offs, dest, src = rt.route(ids, E, pad)
        assert counts.sum() == T * k
        assert np.all(np.diff(np.concatenate([[0], offs])) == (counts + pad - 1) // pad * pad)
        assert np.all(src[dest] == np.arange(T * k))                       # inverse permutation
        start = offs - (counts + pad - 1) // pad * pad
        flat = ids.ravel()
        assert np.all(dest >= start[flat]) and np.all(dest < start[flat] + counts[flat])
        for e in range(E):                                                 # stable within a group
            d = dest[flat == e]
            assert np.all(np.diff(d) == 1)
        assert (src >= 0).sum() == T * k and src.size == rt.rows_bound(T * k, E, pad)


def test_permute_matches_loops():
    rng = np.random.default_rng(1)
    T, k, C, E, pad = 11, 3, 16, 4, 4
    ids = rng.integers(0, E, size=(T, k))
    x = rng.integers(0, 1 << 16, size=(T, C), dtype=np.uint16)
    _, _, _, src = rt.route(ids, E, pad)
    xg = rt.permute(x, src, k)
    for r in range(src.size):
        want = x[src[r] // k] if src[r] >= 0 else np.zeros(C, np.uint16)
        assert np.array_equal(xg[r], want)


def test_combine_matches_loops_in_fp32_order():
    rng = np.random.default_rng(2)
    T, k, C, E = 9, 4, 8, 5
    ids = rng.integers(0, E, size=(T, k))
    ids[3, 1] = -1                                                          # a dropped slot
    _, _, dest, src = rt.route(ids, E, 1)
    yg = round_bf16(rng.standard_normal((src.size, C)))
    w = rng.random((T, k)).astype(np.float32)
    y = rt.combine(yg, dest, w, T, k)
    ygf = oracle.bf16_to_f32(yg)
    for t in range(T):
        for c in range(C):
            acc = np.float32(0.0)
            for j in range(k):
                d = dest[t * k + j]
                if d >= 0:
                    acc = np.float32(acc + np.float32(w[t, j] * ygf[d, c]))
            assert y[t, c] == round_bf16(np.array([float(acc)]))[0]


def test_permute_then_combine_round_trip():
    """Identity experts and weights summing to 1 per token give the tokens back (within the
    fp32 sum's rounding, far inside one bf16 step)."""
    rng = np.random.default_rng(3)
    T, k, C, E = 50, 3, 32, 7
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    x = round_bf16(rng.standard_normal((T, C)))
    counts, offs, dest, src = rt.route(ids, E, 32)
    xg = rt.permute(x, src, k)
    w = np.full((T, k), 1.0 / 4.0, np.float32)
    w[:, 0] = 0.5                                                           # 0.5 + 0.25 + 0.25, exact
    y = rt.combine(xg, dest, w, T, k)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("codec", [oracle.E4M3FN, oracle.E4M3FNUZ])
def test_permute_quantized_equals_quantize_after_permute(codec):
    """Gathering rowwise codes and scales gives the bits of quantizing the gathered bf16 rows, padding
    rows (zeros) included."""
    rng = np.random.default_rng(4)
    T, k, C, E = 60, 3, 48, 5
    ids = rng.integers(0, E, size=(T, k))
    ids[7, 2] = -1
    x = round_bf16(rng.standard_normal((T, C)) * 3)
    x[11] = 0.0                                                             # an all-zero token
    _, _, _, src = rt.route(ids, E, 16)
    q, s = oracle.quantize_rowwise(x, codec)
    qg, sg = rt.permute_quantized(q, s, src, k, codec)
    qr, sr = oracle.quantize_rowwise(rt.permute(x, src, k), codec)
    assert np.array_equal(qg, qr)
    assert np.array_equal(sg.view(np.uint32), sr.view(np.uint32))
