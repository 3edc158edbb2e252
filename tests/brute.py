"""Brute-force masked-dense PFA layer for one window-head (numpy fp64).

A second, independent formulation used to pin the oracle: the full N x N score
matrix is formed densely, non-candidates are masked to -inf, the previous map is
scattered into a dense N x N matrix (zero off its support), and the top-K is taken
with a lexicographic sort. Only practical for tiny windows.
"""

import numpy as np


def masked_dense_layer(q, k, v, C=None, a=None, K_l=None, keep_override=None, bias=None):
    """q, k, v: [N, d] slot-ordered rows of one window-head.
    C: [N, K_prev] candidate slots (None = all); a: [N, K_prev] previous map (None = 1).
    keep_override: [N, N] bool, replaces the top-K choice when given.
    bias: [N, N] dense additive score bias (None = 0).
    Returns (keep [N, N] bool, A [N, N] dense, O [N, d])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    S = (q @ k.T) / np.sqrt(d)
    if bias is not None:
        S = S + np.asarray(bias, np.float64)
    mask = np.zeros((N, N), bool)
    prev = np.zeros((N, N))
    if C is None:
        mask[:] = True
        prev[:] = 1.0 if a is None else np.asarray(a, np.float64)
    else:
        rows = np.repeat(np.arange(N), C.shape[1])
        mask[rows, C.ravel()] = True
        prev[rows, C.ravel()] = 1.0 if a is None else np.asarray(a, np.float64).ravel()
    Sm = np.where(mask, S, -np.inf)
    E = np.exp(Sm - Sm.max(axis=1, keepdims=True))
    Acal = E / E.sum(axis=1, keepdims=True)
    P = prev * Acal
    Pn = P / P.sum(axis=1, keepdims=True)
    if keep_override is not None:
        keep = np.asarray(keep_override, bool)
    else:
        keep = np.zeros((N, N), bool)
        for i in range(N):
            cand = np.nonzero(mask[i])[0]
            order = cand[np.lexsort((cand, -Pn[i, cand]))]
            keep[i, order[:K_l]] = True
    A = np.where(keep, Pn, 0.0)
    A = A / A.sum(axis=1, keepdims=True)
    return keep, A, A @ v


def window_rows(x, b, h, wy, wx, win):
    """Slot-ordered [N, d] rows of window (wy, wx) of an unshifted map x [B, heads, H, W, d]."""
    return np.asarray(x[b, h, wy * win:(wy + 1) * win, wx * win:(wx + 1) * win, :]).reshape(win * win, -1)
