"""fp64 CPU oracle of the PFA layer chain (ctypes wrapper over ``pfa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it; the HIP library never does.

``layer`` computes one PFA layer (steps listed in ``pfa_oracle.c``) for a list of
window-heads; ``chain`` runs the layers of one chain for a list of window-heads,
feeding each layer's (I, A) to the next, all in fp64. ``dense_lse`` gives the
first layer's log softmax denominators. ``layer_backward`` is the reverse-mode
derivative of ``layer`` with the kept sets held fixed. ``iet_propagate`` is the
index-matrix propagation and sparsification step between attention blocks.
"""

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "pfa_oracle.c")
_LIB = os.path.join(_DIR, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over window-heads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_layer.argtypes = [i32] * 7 + [P, P, P, P, i32, P, i32, i32, i32, P, i64, P, P, P, P, P, P]
        lib.oracle_layer.restype = ctypes.c_int
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_layer_backward.argtypes = ([i32] * 7 + [P, P, P, P, P, i32, i32, i32, P, i64, P, P, P, P]
                                              + [P, P, P, P, P])
        lib.oracle_layer_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (omp_set_num_threads of the runtime the
    library links; plumbing for timing the oracle on a given core count)."""
    lib = _load()
    fn = lib.omp_set_num_threads
    fn.argtypes = [ctypes.c_int]
    fn.restype = None
    fn(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def layer(Q, K, V, *, win, shift, K_l, I_prev=None, A_prev=None, i_shared=False,
          prev_compact=False, wh_list=None, forced_keep=None, want_keys=False, O_out=None, bias=None):
    """One PFA layer in fp64.

    Q, K, V: [B, heads, H, W, d] arrays (any float dtype; widened to fp64).
    I_prev: [B, heads|1, nwin, N, K_prev] int32 or None (all slots, K_prev = N).
    A_prev: [B, heads, nwin, N, K_prev] or None (all ones).
    prev_compact: I_prev/A_prev are [n_wh, N, K_prev], aligned with wh_list.
    bias: [heads, (2 win - 1)^2] relative position bias added to the scores
    (window mode), or None.
    Returns dict with I [n_wh, N, K_l] int32, A [n_wh, N, K_l] fp64,
    O [B, heads, H, W, d] fp64 (NaN where not computed), optionally keys
    [n_wh, N, K_prev] = ln P'.
    """
    lib = _load()
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    B, heads, H, W, d = Q.shape
    N = win * win if win else H * W
    nwin = (H // win) * (W // win) if win else 1
    if I_prev is not None:
        I_prev = np.ascontiguousarray(I_prev, dtype=np.int32)
        K_prev = I_prev.shape[-1]
    else:
        K_prev = N
    if A_prev is not None:
        A_prev = np.ascontiguousarray(A_prev, dtype=np.float64)
        assert A_prev.shape[-1] == K_prev
    if wh_list is None:
        wl = None
        n_wh = B * heads * nwin
    else:
        wl = np.ascontiguousarray(wh_list, dtype=np.int64)
        n_wh = len(wl)
    fk = None if forced_keep is None else np.ascontiguousarray(forced_keep, dtype=np.int32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float64)
        assert win and bias.shape == (heads, (2 * win - 1) ** 2)
    I_out = np.empty((n_wh, N, K_l), dtype=np.int32)
    A_out = np.empty((n_wh, N, K_l), dtype=np.float64)
    keys = np.empty((n_wh, N, K_prev), dtype=np.float64) if want_keys else None
    if O_out is None:
        O_out = np.full(Q.shape, np.nan, dtype=np.float64)
    rc = lib.oracle_layer(B, heads, H, W, d, win, shift, _ptr(Q), _ptr(K), _ptr(V),
                          _ptr(I_prev), int(bool(i_shared)), _ptr(A_prev), int(bool(prev_compact)),
                          K_prev, K_l,
                          _ptr(wl), n_wh, _ptr(fk), _ptr(bias), _ptr(I_out), _ptr(A_out), _ptr(keys),
                          _ptr(O_out))
    if rc != 0:
        raise ValueError("oracle_layer rejected the sizes")
    out = {"I": I_out, "A": A_out, "O": O_out}
    if want_keys:
        out["keys"] = keys
    return out


def layer_backward(Q, K, V, *, win, shift, keep, dO, dA=None, I_prev=None, A_prev=None,
                   prev_compact=False, wh_list=None, want_dA_prev=True, bias=None):
    """Gradients of one PFA layer in fp64 with the kept sets held fixed.

    keep: [n_wh, N, K_l] kept slot indices (the layer's I^l, compact over
    wh_list). dO: [B, heads, H, W, d] gradient of O. dA: [n_wh, N, K_l] gradient
    of A^l aligned with keep, or None. I_prev / A_prev / prev_compact as in
    ``layer``. Returns dict dQ, dK, dV ([B, heads, H, W, d], zero outside the
    listed window-heads) and dA_prev ([n_wh, N, K_prev] in I^{l-1} order, when
    A_prev is given and want_dA_prev), and dbias ([heads, (2 win - 1)^2]) when
    a bias is given."""
    lib = _load()
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    dO = np.ascontiguousarray(dO, dtype=np.float64)
    B, heads, H, W, d = Q.shape
    N = win * win if win else H * W
    nwin = (H // win) * (W // win) if win else 1
    if I_prev is not None:
        I_prev = np.ascontiguousarray(I_prev, dtype=np.int32)
        K_prev = I_prev.shape[-1]
    else:
        K_prev = N
    if A_prev is not None:
        A_prev = np.ascontiguousarray(A_prev, dtype=np.float64)
        assert A_prev.shape[-1] == K_prev
    if wh_list is None:
        wl = None
        n_wh = B * heads * nwin
    else:
        wl = np.ascontiguousarray(wh_list, dtype=np.int64)
        n_wh = len(wl)
    keep = np.ascontiguousarray(keep, dtype=np.int32)
    K_l = keep.shape[-1]
    assert keep.shape == (n_wh, N, K_l)
    if dA is not None:
        dA = np.ascontiguousarray(dA, dtype=np.float64)
        assert dA.shape == keep.shape
    dQ = np.zeros(Q.shape)
    dK = np.zeros(Q.shape)
    dV = np.zeros(Q.shape)
    dA_prev = (np.zeros((n_wh, N, K_prev)) if (A_prev is not None and want_dA_prev) else None)
    dbias = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float64)
        assert win and bias.shape == (heads, (2 * win - 1) ** 2)
        dbias = np.zeros(bias.shape)
    rc = lib.oracle_layer_backward(B, heads, H, W, d, win, shift, _ptr(Q), _ptr(K), _ptr(V),
                                   _ptr(I_prev), _ptr(A_prev), int(bool(prev_compact)), K_prev, K_l,
                                   _ptr(wl), n_wh, _ptr(keep), _ptr(dO), _ptr(dA), _ptr(bias),
                                   _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dA_prev), _ptr(dbias))
    if rc != 0:
        raise ValueError("oracle_layer_backward rejected the sizes or the kept sets")
    out = {"dQ": dQ, "dK": dK, "dV": dV}
    if dA_prev is not None:
        out["dA_prev"] = dA_prev
    if dbias is not None:
        out["dbias"] = dbias
    return out


def rel_index(win):
    """[N, N] index into a (2 win - 1)^2 relative position bias table for slots
    (i, j) of a window: (i/w - j/w + w - 1) (2w - 1) + (i%w - j%w + w - 1)."""
    t = np.arange(win * win)
    dy = (t // win)[:, None] - (t // win)[None, :]
    dx = (t % win)[:, None] - (t % win)[None, :]
    return (dy + win - 1) * (2 * win - 1) + (dx + win - 1)


def chain(layers_qkv, *, win, shifts, Ks, wh_list=None):
    """Run a whole chain: layer 0 dense (K^1 = Ks[0], no previous map), then each
    later layer on the previous layer's (I, A). ``layers_qkv`` is a list of
    (Q, K, V) arrays. Returns the list of per-layer output dicts (compact rows
    over ``wh_list``)."""
    Q0 = layers_qkv[0][0]
    B, heads, H, W, _ = Q0.shape
    nwin = (H // win) * (W // win) if win else 1
    wl = np.arange(B * heads * nwin) if wh_list is None else np.asarray(wh_list)
    outs = []
    I_prev = A_prev = None
    for l, (Q, K, V) in enumerate(layers_qkv):
        r = layer(Q, K, V, win=win, shift=shifts[l], K_l=Ks[l], I_prev=I_prev, A_prev=A_prev,
                  prev_compact=True, wh_list=wl)
        outs.append(r)
        I_prev, A_prev = r["I"], r["A"]
    return outs


def dense_lse(Q, K, *, win, shift, wh_list=None, bias=None):
    """ln sum_j exp(q_i . k_j / sqrt(d)) over the N slots of each window, per query
    slot i: the denominator of the first layer's full softmax map (paper notes,
    "Progressive focused resource allocation strategy": the first layer computes
    the complete map), i.e. A^1_ij = exp(s_ij - lse_i). Slot t of window (a, b)
    reads pixel ((a*win + t//win + shift) mod H, (b*win + t%win + shift) mod W).
    With ``bias`` ([heads, (2 win - 1)^2]) the scores carry the relative position
    bias of ``layer``. Returns [n_wh, N] fp64 in window-head order (b, head,
    window row, window col)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    B, heads, H, W, d = Q.shape
    N = win * win
    nwy, nwx = H // win, W // win
    n_all = B * heads * nwy * nwx
    wl = np.arange(n_all) if wh_list is None else np.asarray(wh_list)
    t = np.arange(N)
    out = np.empty((len(wl), N), dtype=np.float64)
    for n, wh in enumerate(wl):
        b, rest = divmod(int(wh), heads * nwy * nwx)
        h, win_id = divmod(rest, nwy * nwx)
        wy, wx = divmod(win_id, nwx)
        y = (wy * win + t // win + shift) % H
        x = (wx * win + t % win + shift) % W
        s = Q[b, h, y, x] @ K[b, h, y, x].T / np.sqrt(d)
        if bias is not None:
            s = s + np.asarray(bias, np.float64)[h][rel_index(win)]
        m = s.max(axis=1, keepdims=True)
        out[n] = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    return out


def iet_select_scores(A):
    """Selection score of each candidate: the maps of all heads added in fp32, in
    head order (one index matrix serves every head). A: [n_maps, N, k]."""
    A = np.asarray(A, dtype=np.float32)
    S = A[0].copy()
    for h in range(1, A.shape[0]):
        S = (S + A[h]).astype(np.float32)
    return S


def iet_propagate(I, A, k1, k2):
    """Propagation and sparsification of an individualized index matrix
    ("From Local Windows to Adaptive Candidates via Individualized Exploratory",
    the paragraphs on propagation and sparsification and on the architecture:
    one-hop neighbours are merged with the neighbours of neighbours and
    de-duplicated; low-similarity connections are pruned; per-block k1 / k2).

    Reading of the lost equation: T_k(i) = the k candidates of row i with the
    largest score (ties to the lower token index). The new candidate set is
        Dedup( T_k1(i)  U  union over u in T_k2(i) of T_k2(u) ).
    I: [N, k] token indices in [0, N); A: [n_maps, N, k] attention weights
    aligned with I (scores: ``iet_select_scores``). Returns (I_out, count):
    I_out [N, k1 + k2*k2] int32 with each row's set in ascending order, padded
    with -1; count [N] int32 = set sizes. Plain Python loops (test sizes)."""
    I = np.asarray(I)
    S = iet_select_scores(A)
    N, k = I.shape
    assert 1 <= k2 <= k1 <= k
    T1 = np.empty((N, k1), dtype=np.int64)
    T2 = np.empty((N, k2), dtype=np.int64)
    for i in range(N):
        order = sorted(range(k), key=lambda c: (-float(S[i, c]), int(I[i, c])))
        T1[i] = I[i, order[:k1]]
        T2[i] = I[i, order[:k2]]
    width = k1 + k2 * k2
    out = np.full((N, width), -1, dtype=np.int32)
    count = np.empty(N, dtype=np.int32)
    for i in range(N):
        cand = set(T1[i].tolist())
        for u in T2[i]:
            cand.update(T2[u].tolist())
        v = sorted(cand)
        out[i, :len(v)] = v
        count[i] = len(v)
    return out, count
