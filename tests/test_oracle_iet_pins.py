"""Pins of the IET propagation / sparsification oracle (``oracle.iet_propagate``).

Source: "From Local Windows to Adaptive Candidates via Individualized
Exploratory" (propagation and sparsification paragraphs; the architecture
paragraph gives k1 = [22, 20, 14, 12], k2 = [12, 10, 7, 6]). The equation of the
merge is lost in the page text; the reading is T_k1(i) united with T_k2(u) over
u in T_k2(i), de-duplicated, where T_k(i) is row i's k highest-scoring
candidates (ties to the lower token index) and the score sums the heads' maps.
"""

import numpy as np

import oracle


def test_hand_worked_example():
    """Six tokens, three candidates each, scores on a 1/8 grid, k1 = 2, k2 = 1.
    Worked by hand: T2 = [1, 0, 1, 5, 1, 4] (rows 2 and 4 break a tie to the
    lower index), T1 = [{1,2}, {0,4}, {1,0}, {5,0}, {1,3}, {4,2}], and each row
    adds T2 of its T2 neighbour."""
    I = np.array([[1, 2, 3], [0, 2, 4], [5, 0, 1], [4, 5, 0], [3, 1, 2], [2, 3, 4]], dtype=np.int32)
    S = np.array([[4, 3, 2], [5, 1, 3], [2, 2, 5], [1, 6, 2], [3, 3, 2], [2, 2, 3]], dtype=np.float32) / 8
    out, cnt = oracle.iet_propagate(I, S[None], 2, 1)
    expect = [[0, 1, 2], [0, 1, 4], [0, 1, -1], [0, 4, 5], [0, 1, 3], [1, 2, 4]]
    np.testing.assert_array_equal(out, np.array(expect, dtype=np.int32))
    np.testing.assert_array_equal(cnt, [3, 3, 2, 3, 3, 3])


def test_scores_sum_over_heads():
    """Two maps that rank row 0 differently on their own: the sum decides.
    Row 0: map 0 = (0.5, 0.25, 0), map 1 = (0, 0.5, 0.375) -> sums (0.5, 0.75,
    0.375): candidate 2 (token 2) is first, so with k1 = k2 = 1 row 0 keeps
    token 2 and adds T1 of token 2 (its own first candidate)."""
    I = np.array([[1, 2, 3], [0, 2, 3], [3, 0, 1], [0, 1, 2]], dtype=np.int32)
    m0 = np.array([[0.5, 0.25, 0], [1, 0, 0], [1, 0, 0], [1, 0, 0]], dtype=np.float32)
    m1 = np.array([[0, 0.5, 0.375], [0, 0, 0], [0, 0, 0], [0, 0, 0]], dtype=np.float32)
    out, cnt = oracle.iet_propagate(I, np.stack([m0, m1]), 1, 1)
    # T1 = T2: row0 -> 2, row1 -> 0, row2 -> 3, row3 -> 0; row0: {2} U T2(2) = {2, 3}
    np.testing.assert_array_equal(out[:, :2], [[2, 3], [0, 2], [0, 3], [0, 2]])
    np.testing.assert_array_equal(cnt, [2, 2, 2, 2])


def test_ring_closed_forms():
    """Ring graph I(i) = (i-1, i, i+1) mod N with equal scores: with k1 = k2 = 3
    every candidate is kept and the result is the two-hop ring i-2 .. i+2; with
    the self weight largest and k2 = 1, nothing is added to T_k1(i)."""
    N = 11
    i = np.arange(N)
    I = np.stack([(i - 1) % N, i, (i + 1) % N], axis=1).astype(np.int32)
    out, cnt = oracle.iet_propagate(I, np.ones((1, N, 3), np.float32), 3, 3)
    for r in range(N):
        assert out[r, :5].tolist() == sorted(((r + t) % N) for t in range(-2, 3))
    assert (cnt == 5).all() and (out[:, 5:] == -1).all()
    A = np.tile(np.array([0.25, 0.5, 0.25], np.float32), (1, N, 1))
    out, cnt = oracle.iet_propagate(I, A, 3, 1)
    for r in range(N):
        assert out[r, :3].tolist() == sorted(((r + t) % N) for t in (-1, 0, 1))
    assert (cnt == 3).all()


def test_invariants_random():
    """Random index matrix: rows ascending and unique, within the two-hop closure
    of I, containing the top-k1 candidates, sizes <= k1 + k2^2; equal scores keep
    the lowest token indices."""
    g = np.random.Generator(np.random.PCG64(5))
    N, k, k1, k2 = 300, 16, 9, 4
    I = np.stack([g.permutation(N)[:k] for _ in range(N)]).astype(np.int32)
    A = g.random((3, N, k)).astype(np.float32)
    out, cnt = oracle.iet_propagate(I, A, k1, k2)
    S = oracle.iet_select_scores(A)
    for r in range(N):
        row = out[r, :cnt[r]]
        assert (np.diff(row) > 0).all() and (out[r, cnt[r]:] == -1).all()
        closure = set(I[r].tolist())
        for u in I[r]:
            closure.update(I[u].tolist())
        assert set(row.tolist()) <= closure
        top = I[r][np.lexsort((I[r], -S[r]))[:k1]]
        assert set(top.tolist()) <= set(row.tolist())
    assert (cnt <= k1 + k2 * k2).all()
    out_eq, _ = oracle.iet_propagate(I, np.ones((1, N, k), np.float32), k1, 1)
    for r in range(N):
        assert set(np.sort(I[r])[:k1].tolist()) <= set(out_eq[r].tolist())
