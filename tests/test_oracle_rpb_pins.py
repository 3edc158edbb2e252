"""Pins of the oracle's relative position bias (the score step with a bias
table): PFT is described as a relative-position-bias based network, and IET
applies relative positional encoding in its first block ("From Local Windows to
Adaptive Candidates via Individualized Exploratory", architecture paragraph).
Reading: a per-head table b of (2w - 1)^2 entries, added to the scaled score of
slots (i, j) at the window-local offset (row_i - row_j, col_i - col_j), before
the softmax.
"""

import numpy as np
import pytest

import oracle
from tests.brute import masked_dense_layer, window_rows


def rnd(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def dense_bias(table, win):
    """[N, N] bias of one head from its table, by explicit coordinates."""
    N = win * win
    out = np.empty((N, N))
    for i in range(N):
        yi, xi = divmod(i, win)
        for j in range(N):
            yj, xj = divmod(j, win)
            out[i, j] = table[(yi - yj + win - 1) * (2 * win - 1) + (xi - xj + win - 1)]
    return out


@pytest.mark.parametrize("win,K_prev,K_l", [(4, 16, 5), (4, 9, 3), (8, 40, 12)])
def test_bias_matches_masked_dense(win, K_prev, K_l):
    """Brute force with an explicit dense bias matrix, every window-head."""
    B, heads, H, W, d = 1, 2, 2 * win, 2 * win, 8
    N = win * win
    Q, K, V = (rnd((B, heads, H, W, d), 10 + t) for t in range(3))
    table = rnd((heads, (2 * win - 1) ** 2), 20) * 2
    g = np.random.Generator(np.random.PCG64(21))
    nwin = 4
    C = np.stack([g.permutation(N)[:K_prev] for _ in range(B * heads * nwin * N)]).astype(np.int32)
    C = C.reshape(B, heads, nwin, N, K_prev)
    a = g.random((B, heads, nwin, N, K_prev)) + 0.05
    r = oracle.layer(Q, K, V, win=win, shift=0, K_l=K_l, I_prev=C, A_prev=a, bias=table)
    for h in range(heads):
        Bm = dense_bias(table[h], win)
        for wid in range(nwin):
            wy, wx = divmod(wid, 2)
            q, k, v = (window_rows(x, 0, h, wy, wx, win) for x in (Q, K, V))
            keep, A, O = masked_dense_layer(q, k, v, C[0, h, wid], a[0, h, wid], K_l, bias=Bm)
            n = h * nwin + wid
            for i in range(N):
                kept = np.nonzero(keep[i])[0]
                assert sorted(r["I"][n, i].tolist()) == kept.tolist()
                np.testing.assert_allclose(r["A"][n, i], A[i, r["I"][n, i]], rtol=1e-11)
            Or = r["O"][0, h, wy * win:(wy + 1) * win, wx * win:(wx + 1) * win].reshape(N, d)
            np.testing.assert_allclose(Or, O, rtol=1e-10, atol=1e-12)


def test_zero_and_constant_bias():
    """A zero table changes nothing; a constant table shifts every score of a
    row equally, which the softmax and both normalisations absorb."""
    win, d = 8, 8
    Q, K, V = (rnd((1, 2, 16, 16, d), 30 + t) for t in range(3))
    base = oracle.layer(Q, K, V, win=win, shift=3, K_l=20)
    zero = oracle.layer(Q, K, V, win=win, shift=3, K_l=20, bias=np.zeros((2, 225)))
    assert np.array_equal(base["I"], zero["I"]) and np.array_equal(base["A"], zero["A"])
    const = oracle.layer(Q, K, V, win=win, shift=3, K_l=20, bias=np.full((2, 225), 3.25))
    assert np.array_equal(base["I"], const["I"])
    np.testing.assert_allclose(const["A"], base["A"], rtol=1e-12)


def test_bias_under_shift_is_window_local():
    """The bias uses window-local slot coordinates, so a shifted layer equals the
    unshifted layer on rolled inputs with the same table (O rolled back)."""
    win, d, s = 4, 4, 2
    Q, K, V = (rnd((1, 1, 8, 8, d), 40 + t) for t in range(3))
    table = rnd((1, 49), 41)
    r = oracle.layer(Q, K, V, win=win, shift=s, K_l=6, bias=table)
    rolled = [np.roll(x, (-s, -s), axis=(2, 3)) for x in (Q, K, V)]
    r0 = oracle.layer(*rolled, win=win, shift=0, K_l=6, bias=table)
    assert np.array_equal(r["I"], r0["I"])
    np.testing.assert_allclose(r["A"], r0["A"], rtol=1e-12)
    np.testing.assert_allclose(np.roll(r0["O"], (s, s), axis=(2, 3)), r["O"], rtol=1e-12, atol=1e-14)


def test_dominant_diagonal_bias():
    """A large bias at offset (0, 0) concentrates every row on itself: O_i = v_i."""
    win, d = 4, 4
    Q, K, V = (rnd((1, 1, 8, 8, d), 50 + t) for t in range(3))
    table = np.zeros((1, 49))
    table[0, 3 * 7 + 3] = 60.0
    r = oracle.layer(Q, K, V, win=win, shift=0, K_l=16, bias=table)
    np.testing.assert_allclose(r["O"], V, rtol=1e-12, atol=1e-20)


def test_bias_gradient_finite_differences():
    """dbias of the backward oracle against central differences of the forward
    oracle (kept set forced), every table entry."""
    win, d, K_prev, K_l = 4, 4, 11, 5
    g = np.random.Generator(np.random.PCG64(60))
    Q, K, V = (g.standard_normal((1, 2, 8, 8, d)) for _ in range(3))
    N = 16
    I_prev = np.stack([g.permutation(N)[:K_prev] for _ in range(2 * 4 * N)]).astype(np.int32).reshape(1, 2, 4, N,
                                                                                                          K_prev)
    A_prev = g.random((1, 2, 4, N, K_prev)) * 0.9 + 0.1
    table = g.standard_normal((2, 49))
    r = oracle.layer(Q, K, V, win=win, shift=1, K_l=K_l, I_prev=I_prev, A_prev=A_prev, bias=table)
    dO = g.standard_normal(Q.shape)
    dA = g.standard_normal(r["I"].shape)
    b = oracle.layer_backward(Q, K, V, win=win, shift=1, keep=r["I"], dO=dO, dA=dA, I_prev=I_prev, A_prev=A_prev,
                              bias=table)

    def loss(t):
        f = oracle.layer(Q, K, V, win=win, shift=1, K_l=K_l, I_prev=I_prev, A_prev=A_prev, bias=t,
                         forced_keep=r["I"])
        return float(np.sum(dO * f["O"]) + np.sum(dA * f["A"]))
    h = 1e-5
    fd = np.empty(table.shape)
    for idx in np.ndindex(table.shape):
        t = table.copy()
        t[idx] += h
        lp = loss(t)
        t[idx] -= 2 * h
        fd[idx] = (lp - loss(t)) / (2 * h)
    assert np.abs(fd - b["dbias"]).max() < 1e-7 * (1 + np.abs(b["dbias"]).max())
