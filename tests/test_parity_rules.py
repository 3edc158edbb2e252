"""CPU checks of the parity helpers themselves (no GPU)."""

import numpy as np

from tests import parity


def _slots_brute(I, cand):
    out = np.full(I.shape, -1, dtype=np.int64)
    for r in np.ndindex(I.shape[:-1]):
        for k, v in enumerate(I[r]):
            hit = np.nonzero(cand[r] == v)[0]
            if len(hit):
                out[r + (k,)] = hit[0]
    return out


def test_candidate_slots_matches_brute_force():
    g = np.random.default_rng(5)
    n, N, Kc, Kl = 3, 17, 12, 5
    cand = np.stack([[g.permutation(40)[:Kc] for _ in range(N)] for _ in range(n)]).astype(np.int32)
    I = np.empty((n, N, Kl), dtype=np.int32)
    for a in range(n):
        for i in range(N):
            pick = np.sort(g.choice(Kc, Kl, replace=False))
            I[a, i] = cand[a, i, pick]
    I[1, 4, 2] = 39 if 39 not in cand[1, 4] else 41   # not a candidate
    I[2, 0, 0] = -1
    got = parity.candidate_slots(I, cand)
    assert (got == _slots_brute(I, cand)).all()
    assert got[1, 4, 2] == -1 and got[2, 0, 0] == -1
    assert (np.diff(got[0], axis=-1) > 0).all()


def test_candidate_slots_no_cross_row_match():
    # a value that is a candidate only in the next row must not be found
    cand = np.array([[[0, 1, 2]], [[3, 4, 5]]], dtype=np.int32)
    I = np.array([[[3]], [[5]]], dtype=np.int32)
    assert (parity.candidate_slots(I, cand).ravel() == [-1, 2]).all()
