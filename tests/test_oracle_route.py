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


def test_combine_without_weights_sums_the_copies():
    """No weights means weight 1 for every slot: the sum of a token's routed copies.  With 4 copies of
    a bf16 row the sum is 4x the row, exact in fp32 and in bf16."""
    rng = np.random.default_rng(5)
    T, k, C, E = 20, 4, 16, 6
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    x = round_bf16(rng.standard_normal((T, C)))
    _, _, dest, src = rt.route(ids, E, 1)
    y = rt.combine(rt.permute(x, src, k), dest, None, T, k)
    assert np.array_equal(oracle.bf16_to_f32(y), 4.0 * oracle.bf16_to_f32(x))


def test_combine_backward_worked_example():
    """Two tokens, two choices each, values chosen so every product and sum is exact.
    Token 0 -> experts (1, 0) with weights (0.5, 0.25); token 1 -> (1, 1) with (1.0, 2.0).
    Grouping (stable, pad 1): expert 0 holds slot 1 (row 0); expert 1 holds slots 0, 2, 3 (rows 1, 2, 3)."""
    ids = np.array([[1, 0], [1, 1]])
    _, _, dest, src = rt.route(ids, 2, 1)
    assert dest.tolist() == [1, 0, 2, 3] and src.tolist() == [1, 0, 2, 3]
    dy = round_bf16(np.array([[1.0, -2.0], [4.0, 0.5]]))
    yg = round_bf16(np.array([[3.0, 1.0],      # row 0: token 0's expert-0 output
                              [2.0, 2.0],      # row 1: token 0's expert-1 output
                              [-1.0, 8.0],     # row 2: token 1, first choice
                              [0.5, 0.25]]))   # row 3: token 1, second choice
    w = np.array([[0.5, 0.25], [1.0, 2.0]], np.float32)
    dyg, dw = rt.combine_backward(dy, yg, src, dest, w, 2, 2)
    assert oracle.bf16_to_f32(dyg).tolist() == [[0.25, -0.5], [0.5, -1.0], [4.0, 0.5], [8.0, 1.0]]
    # dw[s] = <dy[token], yg[dest[s]]>: slot 0 -> row 1, 1 -> row 0, 2 -> row 2, 3 -> row 3
    assert dw.tolist() == [1.0 * 2 - 2.0 * 2, 1.0 * 3 - 2.0 * 1, 4.0 * -1 + 0.5 * 8, 4.0 * 0.5 + 0.5 * 0.25]


def test_combine_backward_is_the_gradient_of_combine():
    """torch autograd (fp64) differentiates the weighted sum of the routed rows: the rows' gradient,
    rounded as the reading states (fp32 product, then bf16), is dyg bit for bit, and the weights'
    gradient is dw.  Padding rows and a dropped slot get zeros."""
    import torch
    rng = np.random.default_rng(6)
    T, k, C, E, pad = 40, 3, 24, 5, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    ids[5, 1] = -1                                                          # dropped slot
    _, offs, dest, src = rt.route(ids, E, pad)
    rows = src.size
    dy = round_bf16(rng.standard_normal((T, C)))
    yg = round_bf16(rng.standard_normal((rows, C)))
    w = (rng.random((T, k)) + 0.1).astype(np.float32)
    dyg, dw = rt.combine_backward(dy, yg, src, dest, w, T, k)

    ygt = torch.tensor(oracle.bf16_to_f32(yg), dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    d = torch.tensor(dest.astype(np.int64)).reshape(T, k)
    ok = (d >= 0).to(torch.float64)
    y = (wt[:, :, None] * ygt[d.clamp(min=0)] * ok[:, :, None]).sum(1)
    (y * torch.tensor(oracle.bf16_to_f32(dy), dtype=torch.float64)).sum().backward()
    want_rows = round_bf16(ygt.grad.numpy().astype(np.float32).astype(np.float64))
    assert np.array_equal(dyg, want_rows)
    assert np.allclose(dw, wt.grad.numpy().ravel(), rtol=1e-13, atol=0.0)
    assert dw[5 * k + 1] == 0.0
    assert np.all(dyg[src < 0] == 0)


def test_combine_backward_catches_index_mistakes():
    """Two plausible slips, planted in copies of the oracle's arithmetic (each a one-token slip: the
    slot's token taken as src // 1, or the weight of the token's first choice for every choice), fail
    the autograd comparison above on the same inputs."""
    import torch
    rng = np.random.default_rng(7)
    T, k, C, E = 12, 2, 8, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    _, _, dest, src = rt.route(ids, E, 1)
    dy = round_bf16(rng.standard_normal((T, C)))
    w = (rng.random((T, k)) + 0.1).astype(np.float32)
    dyf = oracle.bf16_to_f32(dy)
    wt = torch.tensor(w, dtype=torch.float64)
    ygt = torch.zeros((src.size, C), dtype=torch.float64, requires_grad=True)
    d = torch.tensor(dest.astype(np.int64)).reshape(T, k)
    ((wt[:, :, None] * ygt[d]).sum(1) * torch.tensor(dyf, dtype=torch.float64)).sum().backward()
    want = round_bf16(ygt.grad.numpy().astype(np.float32).astype(np.float64))
    s = src.astype(np.int64)
    wrong_token = round_bf16((w.ravel()[s][:, None] * dyf[np.minimum(s, T - 1)]).astype(np.float64))
    wrong_weight = round_bf16((w.ravel()[(s // k) * k][:, None] * dyf[s // k]).astype(np.float64))
    right = round_bf16((w.ravel()[s][:, None] * dyf[s // k]).astype(np.float64))
    assert np.array_equal(right, want)
    assert not np.array_equal(wrong_token, want) and not np.array_equal(wrong_weight, want)
