"""Parity checks of HIP-path outputs against the fp64 oracle.

Rules (tolerances from the acceptance spec of the PFA layer chain):
  * index sets: a row passes if the GPU kept set equals the oracle's; otherwise
    every index in the symmetric difference must sit within GAP of the K_l-th
    largest oracle key (log-domain key ln P', a scale-free measure of the score
    gap). Such a row is a legitimate near-tie; its A and O are then checked
    against the oracle re-run on the GPU's kept set (conditional mode), which
    validates the alternative answer without taking any other GPU value.
  * every GPU row must list its kept indices as a subsequence of I^{l-1}(i) in
    that order (the layout contract of the C ABI).
  * A: elementwise |A_gpu - A_ref| <= tol * A_ref (+1e-30, fp32's normal floor).
  * O: per row max_c |O_gpu - O_ref| <= tol * max_c |O_ref| (+1e-30).
  tol = 1e-5 for fp32 inputs, 2e-3 for bf16 inputs.
"""

import numpy as np

import oracle

GAP = 1e-6
TOL = {"f32": 1e-5, "bf16": 2e-3}


def _rows_equal_sets(Ig, Ir):
    return (np.sort(Ig, axis=-1) == np.sort(Ir, axis=-1)).all(axis=-1)


def check_layer(*, gpu_I, gpu_A, gpu_O, ref, cand, wh_list, tol, rerun, O_ref=None, gap=GAP):
    """gpu_I, gpu_A: [n_sel, N, K_l] rows of the sampled window-heads (GPU);
    gpu_O: GPU O array [B, heads, H, W, d]; ref: oracle output for the same
    window-heads with keys; cand: [n_sel, N, K_prev] candidate lists (None = all
    slots); rerun(forced) -> oracle output with the kept set forced.
    Returns a dict of statistics; raises AssertionError on a violation."""
    Ig, Ag = np.asarray(gpu_I), np.asarray(gpu_A, dtype=np.float64)
    Ir, Ar, keys = ref["I"], ref["A"], ref["keys"]
    n_sel, N, K_l = Ir.shape
    K_prev = keys.shape[-1]
    same = _rows_equal_sets(Ig, Ir)
    tie_rows = np.argwhere(~same)
    stats = {"rows": int(n_sel * N), "tie_rows": int(len(tie_rows)), "max_gap_used": 0.0}

    # ordering contract: kept entries are a subsequence of the candidate list
    if cand is None:
        assert (np.diff(Ig, axis=-1) > 0).all(), "kept indices not in ascending slot order"
    else:
        slot = candidate_slots(Ig, cand)
        assert (slot >= 0).all(), "GPU kept an index that is not a candidate"
        assert (np.diff(slot, axis=-1) > 0).all(), "kept entries not in candidate-list order"

    # near-tie rows: every differing index must be within the gap of the K_l-th key
    if len(tie_rows):
        kth = -np.sort(-keys, axis=-1)[..., K_l - 1]
        for n, i in tie_rows:
            C = np.arange(N) if cand is None else cand[n, i]
            diff = set(Ig[n, i].tolist()) ^ set(Ir[n, i].tolist())
            for j in diff:
                c = int(np.nonzero(C == j)[0][0])
                g = abs(keys[n, i, c] - kth[n, i])
                stats["max_gap_used"] = max(stats["max_gap_used"], float(g))
                assert g < gap, f"row ({n},{i}): index {j} differs at key gap {g:.3e} >= {gap}"
        forced = np.where(same[..., None], Ir, Ig).astype(np.int32)
        cond = rerun(forced)
        Ar = np.where(same[..., None], Ar, cond["A"])
        O_ref = cond["O"] if O_ref is None else np.where(np.isnan(cond["O"]), O_ref, cond["O"])
        Ir = forced
    assert (Ig == Ir).all(), "kept indices differ in order"
    err_A = np.abs(Ag - Ar)
    bad = err_A > tol * Ar + 1e-30
    stats["max_rel_A"] = float((err_A / np.maximum(Ar, 1e-30)).max())
    assert not bad.any(), f"A mismatch: max rel {stats['max_rel_A']:.3e} > {tol}"

    O_ref = ref["O"] if O_ref is None else O_ref
    stats.update(check_O(gpu_O, O_ref, tol))
    return stats


def candidate_slots(I, cand):
    """Slot of each I[..., k] in its row's candidate list cand[..., :] (distinct
    entries per row), -1 where it is not a candidate. One global binary search:
    each row's values are offset by row * (max value + 1) so that the sorted
    rows concatenate into one sorted array."""
    I = np.asarray(I, dtype=np.int64)
    C = np.asarray(cand, dtype=np.int64)
    R, Kc, Kl = int(np.prod(C.shape[:-1])), C.shape[-1], I.shape[-1]
    span = int(max(C.max(initial=0), I.max(initial=0))) + 1
    off = (np.arange(R, dtype=np.int64) * span)[:, None]
    c = C.reshape(R, Kc) + off
    order = np.argsort(c, axis=-1, kind="stable")
    cs = np.take_along_axis(c, order, axis=-1).ravel()
    g = (I.reshape(R, Kl) + off).ravel()
    p = np.minimum(np.searchsorted(cs, g), cs.size - 1)
    found = (cs[p] == g) & (I.reshape(-1) >= 0)
    slot = np.where(found, order.ravel()[p], -1)
    return slot.reshape(I.shape)


def check_O(gpu_O, O_ref, tol):
    """Per pixel row (the d values of one token): max abs diff <= tol * max |O_ref|."""
    mask = ~np.isnan(O_ref[..., 0])
    g = np.asarray(gpu_O, dtype=np.float64)[mask]
    r = O_ref[mask]
    err = np.abs(g - r).max(axis=-1)
    scale = np.abs(r).max(axis=-1)
    worst = float((err / np.maximum(scale, 1e-30)).max()) if len(err) else 0.0
    assert (err <= tol * scale + 1e-30).all(), f"O mismatch: max row-relative {worst:.3e} > {tol}"
    return {"rows_O": int(mask.sum()), "max_rel_O": worst}


def rerun_fn(Q, K, V, *, win, shift, K_l, I_prev, A_prev, i_shared, prev_compact, wh_list):
    def rerun(forced):
        return oracle.layer(Q, K, V, win=win, shift=shift, K_l=K_l, I_prev=I_prev, A_prev=A_prev,
                            i_shared=i_shared, prev_compact=prev_compact, wh_list=wh_list,
                            forced_keep=forced)
    return rerun
