"""Pins of the fp64 backward oracle (``oracle.layer_backward``).

The backward pass of a PFA layer treats the kept sets as constants (top-K is
piecewise constant) and differentiates through the renormalisation, the
Hadamard product with A^{l-1}, the softmax and the two sparse products
("Progressive Focused Transformer for Single Image Super-Resolution" paper
notes, sections "Progressive attention across layers" and "Sparse matrix
multiplication"; the pages train the network end to end but print no gradient,
so everything here is pinned by mathematics, not by printed values).

* central finite differences of the forward oracle (kept set forced), over
  every entry of Q, K, V and A^{l-1}: catches any dropped term, wrong sign,
  index or transposed operand in the backward;
* the all-candidates special case equals torch autograd of plain softmax
  attention in float64 (a library routine);
* invariants that follow from the forward's symmetries (row scaling of
  A^{l-1}, a constant added to every key, the scale trade between Q and K,
  rows of A^l summing to one).
"""

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def case(B, heads, H, W, d, win, K_prev, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    Q, K, V = (g.standard_normal((B, heads, H, W, d)) for _ in range(3))
    N = win * win if win else H * W
    nwin = (H // win) * (W // win) if win else 1
    rows = B * heads * nwin * N
    I_prev = np.stack([g.permutation(N)[:K_prev] for _ in range(rows)]).astype(np.int32)
    I_prev = I_prev.reshape(B, heads, nwin, N, K_prev)
    A_prev = (g.random((B, heads, nwin, N, K_prev)) * 0.9 + 0.1)
    return Q, K, V, I_prev, A_prev


def loss_fn(Q, K, V, A_prev, I_prev, *, win, shift, keep, dO, dA):
    r = oracle.layer(Q, K, V, win=win, shift=shift, K_l=keep.shape[-1], I_prev=I_prev, A_prev=A_prev,
                     forced_keep=keep)
    return float(np.sum(dO * r["O"]) + (np.sum(dA * r["A"]) if dA is not None else 0.0))


def test_finite_differences_zero_previous_weights():
    """Kept slots whose previous weight is exactly 0 (kept when K_l exceeds a
    row's positive weights; their A^l is 0) still have a nonzero derivative with
    respect to that weight: exp(s) / sum_kept A^{l-1} exp(s) times g. Pinned by
    central differences of the forward oracle over every entry of A^{l-1}."""
    win, shift, d, K_prev, K_l = 4, 2, 4, 11, 8
    Q, K, V, I_prev, A_prev = case(1, 1, 8, 8, d, win, K_prev, 91)
    g = np.random.Generator(np.random.PCG64(92))
    zero = g.random(A_prev.shape) < 0.6
    zero[..., 0] = False
    A_prev[zero] = 0.0
    r = oracle.layer(Q, K, V, win=win, shift=shift, K_l=K_l, I_prev=I_prev, A_prev=A_prev)
    keep = r["I"]
    dO = rnd(Q.shape, 93)
    dA = rnd(keep.shape, 94)
    b = oracle.layer_backward(Q, K, V, win=win, shift=shift, keep=keep, dO=dO, dA=dA, I_prev=I_prev, A_prev=A_prev)
    grad = b["dA_prev"].reshape(A_prev.shape)
    # kept slots with a zero weight exist and get nonzero gradients
    flat_I = I_prev.reshape(-1, K_prev)
    kept_mask = np.stack([np.isin(flat_I[n], keep.reshape(-1, K_l)[n]) for n in range(flat_I.shape[0])])
    kz = kept_mask & zero.reshape(-1, K_prev)
    assert kz.sum() > 20
    assert (np.abs(grad.reshape(-1, K_prev)[kz]) > 1e-6).mean() > 0.9
    args = dict(win=win, shift=shift, keep=keep, dO=dO, dA=dA)
    h = 1e-6
    fd = np.empty(A_prev.shape)
    for idx in np.ndindex(A_prev.shape):
        x0 = A_prev[idx]
        A_prev[idx] = x0 + h
        lp = loss_fn(Q, K, V, A_prev, I_prev, **args)
        A_prev[idx] = x0 - h
        lm = loss_fn(Q, K, V, A_prev, I_prev, **args)
        A_prev[idx] = x0
        fd[idx] = (lp - lm) / (2 * h)
    err = np.abs(fd - grad).max()
    assert err < 1e-6 * (1 + np.abs(grad).max()), err


@pytest.mark.parametrize("win,shift,with_dA", [(4, 2, True), (4, 0, False), (0, 0, True)])
def test_finite_differences(win, shift, with_dA):
    """Every gradient entry against a central difference of the forward oracle
    with the kept set held fixed."""
    H = W = 8 if win else 4
    d, K_prev, K_l = 4, 11, 5
    Q, K, V, I_prev, A_prev = case(1, 2, H, W, d, win, K_prev, 11 + win + shift)
    r = oracle.layer(Q, K, V, win=win, shift=shift, K_l=K_l, I_prev=I_prev, A_prev=A_prev)
    keep = r["I"]
    dO = rnd(Q.shape, 5)
    dA = rnd(keep.shape, 6) if with_dA else None
    b = oracle.layer_backward(Q, K, V, win=win, shift=shift, keep=keep, dO=dO, dA=dA, I_prev=I_prev,
                              A_prev=A_prev)
    args = dict(win=win, shift=shift, keep=keep, dO=dO, dA=dA)
    h = 1e-5
    params = {"dQ": Q, "dK": K, "dV": V, "dA_prev": A_prev}
    for name, X in params.items():
        grad = b[name].reshape(X.shape)
        fd = np.empty(X.shape)
        for idx in np.ndindex(X.shape):
            x0 = X[idx]
            X[idx] = x0 + h
            lp = loss_fn(Q, K, V, A_prev, I_prev, **args)
            X[idx] = x0 - h
            lm = loss_fn(Q, K, V, A_prev, I_prev, **args)
            X[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - grad).max()
        assert err < 1e-7 * (1 + np.abs(grad).max()), (name, err)
    # dropped candidates of A^{l-1} get exactly no gradient from the fixed set
    flat_I = I_prev.reshape(-1, K_prev)
    kept_mask = np.array([[flat_I[r_, c] in keep.reshape(-1, K_l)[r_] for c in range(K_prev)]
                          for r_ in range(flat_I.shape[0])])
    assert np.abs(b["dA_prev"].reshape(-1, K_prev)[~kept_mask]).max() < 1e-14


def window_tokens(x, win, shift):
    """[B, heads, H, W, d] -> [B*heads*nwin, N, d] tokens in slot order: roll by
    -shift, then cut win x win windows (raster inside the window)."""
    B, heads, H, W, d = x.shape
    x = torch.roll(x, shifts=(-shift, -shift), dims=(2, 3))
    x = x.reshape(B, heads, H // win, win, W // win, win, d).permute(0, 1, 2, 4, 3, 5, 6)
    return x.reshape(-1, win * win, d)


def test_all_candidates_matches_torch_autograd():
    """K_l = K_prev = N without a previous map is plain window softmax attention;
    its gradients (with a loss on both O and the map) come from torch autograd."""
    B, heads, H, W, d, win, shift = 1, 2, 8, 8, 8, 4, 1
    N = win * win
    Q, K, V = (rnd((B, heads, H, W, d), 30 + t) for t in range(3))
    r = oracle.layer(Q, K, V, win=win, shift=shift, K_l=N)
    keep = r["I"]
    assert np.array_equal(keep, np.broadcast_to(np.arange(N, dtype=np.int32), keep.shape))
    dO = rnd(Q.shape, 40)
    dA = rnd(keep.shape, 41)
    b = oracle.layer_backward(Q, K, V, win=win, shift=shift, keep=keep, dO=dO, dA=dA)

    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    q, k, v = (window_tokens(t, win, shift) for t in (tq, tk, tv))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    p = torch.softmax(q @ k.transpose(1, 2) / np.sqrt(d), dim=-1)
    go = window_tokens(torch.tensor(dO), win, shift)
    loss = (o * go).sum() + (p * torch.tensor(dA)).sum()
    loss.backward()
    for name, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        assert np.abs(b[name] - t.grad.numpy()).max() < 1e-12, name


def test_invariants():
    """Symmetries of the forward fix linear relations among the gradients."""
    B, heads, H, W, d, win, shift = 1, 2, 16, 16, 8, 8, 4
    N, K_prev, K_l = 64, 40, 10
    Q, K, V, I_prev, A_prev = case(B, heads, H, W, d, win, K_prev, 77)
    r = oracle.layer(Q, K, V, win=win, shift=shift, K_l=K_l, I_prev=I_prev, A_prev=A_prev)
    dO = rnd(Q.shape, 78)
    dA = rnd(r["I"].shape, 79)
    b = oracle.layer_backward(Q, K, V, win=win, shift=shift, keep=r["I"], dO=dO, dA=dA, I_prev=I_prev,
                              A_prev=A_prev)
    # scaling a row of A^{l-1} leaves the layer unchanged
    rs = (A_prev.reshape(-1, K_prev) * b["dA_prev"].reshape(-1, K_prev)).sum(axis=1)
    assert np.abs(rs).max() < 1e-12 * np.abs(b["dA_prev"]).max() * K_prev
    qt, kt, vt, gq, gk, gv, got = (window_tokens(torch.tensor(x), win, shift).numpy()
                                   for x in (Q, K, V, b["dQ"], b["dK"], b["dV"], dO))
    # a constant added to every key shifts each row's scores by a constant
    assert np.abs(gk.sum(axis=1)).max() < 1e-12 * np.abs(gk).sum(axis=1).max()
    # rows of A^l sum to one: the value gradients add up to the output gradients
    assert np.abs(gv.sum(axis=1) - got.sum(axis=1)).max() < 1e-12 * np.abs(got).sum(axis=1).max()
    # q -> (1+e) q, k -> k / (1+e) leaves every score unchanged
    lhs = (qt * gq).sum(axis=(1, 2))
    rhs = (kt * gk).sum(axis=(1, 2))
    assert np.abs(lhs - rhs).max() < 1e-11 * np.abs(lhs).max()


def test_rejects_kept_slot_outside_candidates():
    Q, K, V, I_prev, A_prev = case(1, 1, 4, 4, 4, 4, 6, 3)
    r = oracle.layer(Q, K, V, win=4, shift=0, K_l=3, I_prev=I_prev, A_prev=A_prev)
    keep = r["I"].copy()
    row = I_prev.reshape(-1, 6)[0]
    keep[0, 0, 0] = [t for t in range(16) if t not in row][0]
    with pytest.raises(ValueError):
        oracle.layer_backward(Q, K, V, win=4, shift=0, keep=keep, dO=rnd(Q.shape, 1), I_prev=I_prev,
                              A_prev=A_prev)
