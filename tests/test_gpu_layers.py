"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on
small inputs: free-running chains with every row compared, ragged and extreme
sizes, exact ties, zeros in the previous map, shared index matrices, dense-layer
variants, determinism and error codes. Rules: tests/parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_progressive_window_amd import inputs, pfa, workloads
from tests import parity
from tests.test_gpu_workloads import to_dev

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# free-running GPU chains, every row compared
# ---------------------------------------------------------------------------
def run_chain(B, heads, H, W, d, win, Ks, shifts, dtype, seed):
    """GPU chain with its own (I, A) vs the oracle chain; rows that legitimately
    diverged at a near-tie are excluded from later layers (rows are independent)."""
    shape = (B, heads, H, W, d)
    qkvs = [tuple(inputs.draw(seed + 10 * l + t, shape, dtype) for t in range(3)) for l in range(len(Ks))]
    n_wh = B * heads * (H // win) * (W // win)
    N = win * win
    tol = parity.TOL[dtype]
    sel = np.arange(n_wh)
    I_g = A_g = None
    I_r = A_r = None
    alive = np.ones((n_wh, N), bool)
    for l, (qt, kt, vt) in enumerate(qkvs):
        Qd, Kd, Vd = to_dev(qt), to_dev(kt), to_dev(vt)
        if l == 0:
            I, A, O = pfa.dense_layer(Qd, Kd, Vd, Ks[0], win=win, shift=shifts[0], want_A=True, want_I=True)
        else:
            I, A, O = pfa.sparse_layer(Qd, Kd, Vd, None if (l == 1 and Ks[0] == N) else I_g, A_g, Ks[l],
                                       win=win, shift=shifts[l])
        torch.cuda.synchronize()
        # oracle on the GPU's own previous map would take GPU values: use the oracle's chain instead
        ref = oracle.layer(qt.exact, kt.exact, vt.exact, win=win, shift=shifts[l], K_l=Ks[l], I_prev=I_r,
                           A_prev=A_r, prev_compact=True, wh_list=sel, want_keys=True)
        Ig = I.view(n_wh, N, Ks[l]).cpu().numpy()
        Ag = A.view(n_wh, N, Ks[l]).cpu().numpy()
        # compare rows still on the oracle's path; near-tie divergence retires a row
        same = (np.sort(Ig, -1) == np.sort(ref["I"], -1)).all(-1)
        rows = alive & same
        diverged = alive & ~same
        if diverged.any():
            keys = ref["keys"]
            kth = -np.sort(-keys, -1)[..., Ks[l] - 1]
            for n, i in np.argwhere(diverged):
                C = np.arange(N) if I_r is None else I_r[n, i]
                for j in set(Ig[n, i].tolist()) ^ set(ref["I"][n, i].tolist()):
                    c = int(np.nonzero(C == j)[0][0])
                    assert abs(keys[n, i, c] - kth[n, i]) < parity.GAP, (l, n, i, j)
        np.testing.assert_array_equal(Ig[rows], ref["I"][rows])
        err = np.abs(Ag[rows] - ref["A"][rows])
        assert (err <= tol * ref["A"][rows] + 1e-30).all(), (l, float((err / ref["A"][rows]).max()))
        # O on the pixels of rows still on the oracle's path
        parity.check_O(O.cpu().numpy(), _mask_O(ref["O"], rows, B, heads, H, W, win, shifts[l]), tol)
        # invariants on every GPU row
        np.testing.assert_allclose(Ag.sum(-1), 1.0, rtol=1e-5 if dtype == "f32" else 1e-4)
        assert (Ig >= 0).all() and (Ig < N).all()
        alive = rows
        I_g, A_g = I, A
        I_r, A_r = ref["I"], ref["A"]
        del Qd, Kd, Vd
    return alive


def _mask_O(O_ref, rows, B, heads, H, W, win, shift):
    """NaN out the O rows of retired slots (slot -> pixel under the layer's shift)."""
    out = O_ref.copy()
    nwy, nwx = H // win, W // win
    for n, i in np.argwhere(~rows):
        wx = n % nwx
        wy = (n // nwx) % nwy
        bh = n // (nwx * nwy)
        y = (wy * win + i // win + shift) % H
        x = (wx * win + i % win + shift) % W
        out[bh // heads, bh % heads, y, x] = np.nan
    return out


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_free_running_small(dtype):
    alive = run_chain(2, 3, 64, 96, 32, 32, [1024, 256, 128, 64, 32, 16], [0, 16, 0, 16, 0, 16], dtype, 9100)
    assert alive.mean() > 0.97


@pytest.mark.timeout(300)
def test_chain_tiny_workload():
    w = workloads.TINY
    run_chain(w.B, w.heads, w.H, w.W, w.d, w.win, w.K, w.shifts, w.dtype, 9200)


# ---------------------------------------------------------------------------
# edge cases: ragged and extreme sizes, ties, zeros, shared index matrices
# ---------------------------------------------------------------------------
def _on_grid(t):
    """The tensor's values rounded to multiples of 1/8 (exact in bf16 and fp32)."""
    v = np.round(t.exact.astype(np.float64) * 8) / 8
    if t.dtype == "f32":
        return inputs.Tensor(v.astype(np.float32), v.astype(np.float32), "f32")
    bits = inputs.bf16_round_bits(v.astype(np.float32))
    return inputs.Tensor(bits, inputs.bf16_bits_to_f32(bits), "bf16")


def single_layer_case(B, heads, H, W, d, win, shift, K_prev, K_l, dtype, seed, *, sorted_c=False,
                      dup_keys=False, zero_frac=0.0, no_A=False, i_shared=False, implicit=False):
    """One sparse layer on random candidate lists (implicit: every slot, K_prev = N)
    and a random previous map, checked against the oracle."""
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(seed + t, shape, dtype) for t in range(3))
    if dup_keys:
        # identical key vectors on every pixel, and q, k on a 1/8 grid so that every
        # product and partial sum of q.k is exact in fp32: all scores of a row are
        # then equal bit for bit whatever the summation order
        qt = _on_grid(qt)
        kt = _on_grid(kt)
        kt = inputs.Tensor(np.broadcast_to(kt.device[:, :, :1, :1], shape).copy(),
                           np.broadcast_to(kt.exact[:, :, :1, :1], shape).copy(), dtype)
    N = win * win if win else H * W
    nwin = (H // win) * (W // win) if win else 1
    n_wh = B * heads * nwin
    g = np.random.Generator(np.random.PCG64(seed + 5))
    hI = 1 if i_shared else heads
    C = np.stack([g.permutation(N)[:K_prev] for _ in range(B * hI * nwin * N)]).astype(np.int32)
    if sorted_c:
        C = np.sort(C, axis=1)
    C = C.reshape(B, hI, nwin, N, K_prev)
    if implicit:
        assert K_prev == N
        C = None
    a = (g.random((n_wh, N, K_prev)) + 0.05).astype(np.float32)
    if dup_keys:   # a coarse previous map: many exactly equal weights in a row
        a = (np.floor(a * 4) / 4 + 0.25).astype(np.float32)
    if zero_frac:
        a[g.random(a.shape) < zero_frac] = 0.0
        a[..., 0] = np.maximum(a[..., 0], 0.5)
    a = a.reshape(B, heads, nwin, N, K_prev)
    I, A, O = pfa.sparse_layer(to_dev(qt), to_dev(kt), to_dev(vt), None if C is None else torch.from_numpy(C).cuda(),
                               None if no_A else torch.from_numpy(a).cuda(), K_l, win=win, shift=shift,
                               i_shared=i_shared, K_prev=K_prev)
    torch.cuda.synchronize()
    sel = np.arange(n_wh)
    kw = dict(win=win, shift=shift, K_l=K_l, I_prev=C, A_prev=None if no_A else a.astype(np.float64),
              i_shared=i_shared, prev_compact=False, wh_list=sel)
    ref = oracle.layer(qt.exact, kt.exact, vt.exact, want_keys=True, **kw)
    cand = None if C is None else np.stack([C[n // (heads * nwin), 0 if i_shared else (n // nwin) % heads, n % nwin]
                                            for n in range(n_wh)])
    return parity.check_layer(gpu_I=I.view(n_wh, N, K_l).cpu().numpy(), gpu_A=A.view(n_wh, N, K_l).cpu().numpy(),
                              gpu_O=O.cpu().numpy(), ref=ref, cand=cand, wh_list=sel,
                              tol=parity.TOL[dtype], rerun=parity.rerun_fn(qt.exact, kt.exact, vt.exact, **kw))


EDGE = [
    # B, heads, H, W, d, win, shift, K_prev, K_l, dtype
    (1, 2, 8, 12, 16, 4, 2, 16, 5, "f32"),        # N = 16, shifted, tiny window
    (1, 1, 16, 16, 32, 8, 3, 37, 36, "f32"),      # ragged K_prev, odd shift
    (2, 2, 32, 32, 32, 16, 8, 100, 37, "bf16"),   # ragged K_prev / K_l
    (1, 2, 32, 64, 32, 32, 16, 1024, 1024, "f32"),  # K_l = K_prev = N (two aggregation passes)
    (1, 2, 32, 32, 32, 32, 0, 1024, 1, "bf16"),   # K_l = 1
    (1, 3, 32, 32, 16, 32, 5, 300, 150, "bf16"),  # d = 16 bf16
    (1, 3, 32, 32, 16, 32, 31, 64, 64, "f32"),    # K_l = K_prev, max shift
    (1, 1, 24, 24, 32, 12, 6, 144, 20, "f32"),    # window side not a power of two
    # fp32, N = 1024 (K and V do not fit LDS together: selection + aggregation kernels)
    (1, 2, 32, 32, 32, 32, 16, 200, 77, "f32"),   # ragged K_prev, 32-lane rows
    (1, 2, 32, 32, 32, 32, 0, 100, 50, "f32"),    # ragged K_prev, 16-lane rows
    (1, 1, 32, 32, 32, 32, 5, 20, 7, "f32"),      # ragged small K_prev
    (1, 2, 32, 32, 32, 32, 16, 256, 128, "f32"),  # rows filled exactly (as in the chain)
    (1, 2, 32, 32, 32, 32, 16, 512, 200, "f32"),  # 64-lane rows
    # narrow row groups of the selection kernel (4 lanes up to K_prev 32, 8 up to 64)
    (1, 2, 32, 32, 32, 32, 7, 12, 5, "bf16"),     # ragged 4-lane rows, 4 candidates per lane
    (1, 2, 32, 32, 16, 32, 9, 29, 16, "f32"),     # ragged 4-lane rows, 8 candidates per lane
    (1, 2, 32, 32, 32, 32, 3, 48, 20, "bf16"),    # ragged 8-lane rows
    (1, 2, 32, 32, 32, 32, 16, 32, 16, "f32"),    # full 4-lane rows (as in the chain)
    (1, 2, 32, 32, 32, 32, 16, 64, 32, "bf16"),   # full 8-lane rows (as in the chain)
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", EDGE)
def test_edge_cases(case):
    single_layer_case(*case, seed=4000 + sum(case[:9]))


@pytest.mark.timeout(300)
def test_exact_ties_lower_index_wins():
    # every score of a row equal and A_prev with repeated values: ties everywhere
    st = single_layer_case(1, 2, 32, 32, 32, 32, 0, 256, 100, "f32", 51, dup_keys=True, zero_frac=0.3)
    assert st["tie_rows"] == 0


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,K_prev,K_l", [("f32", 16, 7), ("bf16", 32, 16), ("f32", 30, 11), ("bf16", 64, 32),
                                             ("f32", 50, 21)])
def test_exact_ties_narrow_row_groups(dtype, K_prev, K_l):
    # the same tie pattern on the 4- and 8-lane row groups of small candidate lists
    st = single_layer_case(1, 2, 32, 32, 32, 32, 5, K_prev, K_l, dtype, 52 + K_prev, dup_keys=True, zero_frac=0.3)
    assert st["tie_rows"] == 0


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,K_l,no_A", [("f32", 256, False), ("f32", 1000, False), ("f32", 1, True),
                                            ("f32", 1024, False), ("bf16", 256, False), ("bf16", 100, True)])
def test_all_candidates_layer_exact_ties(dtype, K_l, no_A):
    # candidate list = every slot (the layer after the dense one): identical key
    # vectors make every score of a row equal, so the ranking comes from a coarse
    # previous map with many equal weights (or, without one, every key ties)
    st = single_layer_case(1, 2, 32, 32, 32, 32, 16, 1024, K_l, dtype, 53, dup_keys=True, no_A=no_A,
                           implicit=True)
    assert st["tie_rows"] == 0


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,K_l", [("f32", 32, 256), ("bf16", 32, 256), ("f32", 16, 256), ("bf16", 16, 256),
                                         ("f32", 16, 32), ("bf16", 16, 32), ("bf16", 32, 32), ("f32", 32, 12)])
def test_all_candidates_layer_random(dtype, d, K_l):
    # N = 1024 rows over 2 parts of 512, 4-row batches; zeros in the map; d = 16
    # takes the padded (unswizzled) K layout; small K_l puts 8 or 16 rows in one
    # aggregation step (groups of 8 or 4 lanes, narrower than a DPP row)
    single_layer_case(1, 3, 32, 64, d, 32, 16, 1024, K_l, dtype, 54 + d + K_l, zero_frac=0.2, implicit=True)


@pytest.mark.timeout(300)
def test_zeros_in_previous_map():
    single_layer_case(1, 2, 32, 32, 32, 32, 16, 128, 100, "bf16", 52, zero_frac=0.5)


@pytest.mark.timeout(300)
def test_shared_index_window_mode_and_global_unshared():
    single_layer_case(2, 3, 32, 32, 32, 16, 4, 64, 16, "f32", 53, i_shared=True)
    single_layer_case(1, 2, 16, 32, 32, 0, 0, 96, 40, "bf16", 54)
    single_layer_case(1, 2, 16, 16, 32, 0, 0, 48, 48, "f32", 55, no_A=True, sorted_c=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,win", [("f32", 32, 32), ("bf16", 32, 32), ("f32", 16, 16), ("bf16", 16, 8),
                                         ("f32", 32, 12), ("f32", 32, 8)])
def test_dense_layer_variants(dtype, d, win):
    B, heads, H, W = 1, 2, 2 * win, 3 * win
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(600 + t + d + win, shape, dtype) for t in range(3))
    N = win * win
    n_wh = B * heads * 6
    sel = np.arange(n_wh)
    for shift, K1 in [(0, N), (win // 2, N), (win // 2, N // 3)]:
        I, A, O = pfa.dense_layer(to_dev(qt), to_dev(kt), to_dev(vt), K1, win=win, shift=shift, want_A=True,
                                  want_I=True)
        torch.cuda.synchronize()
        kw = dict(win=win, shift=shift, K_l=K1, wh_list=sel)
        ref = oracle.layer(qt.exact, kt.exact, vt.exact, want_keys=True, **kw)
        parity.check_layer(gpu_I=I.view(n_wh, N, K1).cpu().numpy(), gpu_A=A.view(n_wh, N, K1).cpu().numpy(),
                           gpu_O=O.cpu().numpy(), ref=ref, cand=None, wh_list=sel, tol=parity.TOL[dtype],
                           rerun=parity.rerun_fn(qt.exact, kt.exact, vt.exact, I_prev=None, A_prev=None,
                                                 i_shared=False, prev_compact=False, **kw))
    # O-only mode (one pass, online softmax) matches the oracle's O, and the log
    # softmax denominators match the oracle's (absolute error in the log domain =
    # relative error of the denominator)
    lse = torch.empty((n_wh, N), dtype=torch.float32, device="cuda")
    _, A0, O0 = pfa.dense_layer(to_dev(qt), to_dev(kt), to_dev(vt), N, win=win, shift=win // 2, want_A=False,
                                lse_out=lse)
    torch.cuda.synchronize()
    assert A0 is None
    ref0 = oracle.layer(qt.exact, kt.exact, vt.exact, win=win, shift=win // 2, K_l=N, wh_list=sel)
    parity.check_O(O0.cpu().numpy(), ref0["O"], parity.TOL[dtype])
    lse_ref = oracle.dense_lse(qt.exact, kt.exact, win=win, shift=win // 2)
    err = np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref)
    assert err.max() <= parity.TOL[dtype], float(err.max())


@pytest.mark.timeout(300)
def test_deterministic():
    w = workloads.PATCH64
    shape = (4, 6, 64, 64, 32)
    qt, kt, vt = (inputs.draw(700 + t, shape, "bf16") for t in range(3))
    Qd, Kd, Vd = to_dev(qt), to_dev(kt), to_dev(vt)
    _, A1, O1 = pfa.dense_layer(Qd, Kd, Vd, 1024, win=32, shift=16)
    I2, A2, O2 = pfa.sparse_layer(Qd, Kd, Vd, None, A1, 256, win=32, shift=16)
    I3, A3, O3 = pfa.sparse_layer(Qd, Kd, Vd, I2, A2, 128, win=32, shift=0)
    _, A1b, O1b = pfa.dense_layer(Qd, Kd, Vd, 1024, win=32, shift=16)
    I2b, A2b, O2b = pfa.sparse_layer(Qd, Kd, Vd, None, A1b, 256, win=32, shift=16)
    I3b, A3b, O3b = pfa.sparse_layer(Qd, Kd, Vd, I2b, A2b, 128, win=32, shift=0)
    for x, y in [(A1, A1b), (O1, O1b), (I2, I2b), (A2, A2b), (O2, O2b), (I3, I3b), (A3, A3b), (O3, O3b)]:
        assert torch.equal(x, y)


def test_error_codes():
    Q = torch.zeros((1, 1, 32, 32, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(pfa.PfaError) as e:
        pfa.sparse_layer(Q, Q, Q, None, None, 0, win=32)            # K_l < 1
    assert e.value.code == -1
    with pytest.raises(pfa.PfaError) as e:
        pfa.sparse_layer(Q, Q, Q, None, None, 10, win=32, shift=32)  # shift >= win
    assert e.value.code == -1
    Q5 = torch.zeros((1, 1, 32, 32, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(pfa.PfaError) as e:
        pfa.dense_layer(Q5, Q5, Q5, win=32)                          # d = 8
    assert e.value.code == -2
    with pytest.raises(pfa.PfaError) as e:
        pfa.dense_layer(Q, Q, Q, win=0)                              # dense layer in global mode
    assert e.value.code == -2


@pytest.mark.timeout(120)
def test_kernel_timing_records():
    # every launch of the layer calls is bracketed by events while timing is on
    shape = (1, 2, 64, 64, 32)
    Qd, Kd, Vd = (to_dev(inputs.draw(900 + t, shape, "f32")) for t in range(3))
    pfa.timing_enable(8)
    try:
        I1, A1, O1 = pfa.dense_layer(Qd, Kd, Vd, 1024, win=32, want_I=True)
        n1 = pfa.timing_count()
        I2, A2, O2 = pfa.sparse_layer(Qd, Kd, Vd, None, A1, 256, win=32, shift=16)
        I3, A3, O3 = pfa.sparse_layer(Qd, Kd, Vd, I2, A2, 128, win=32)
        recs, dropped = pfa.timing_read()
        assert pfa.timing_count() == 0
    finally:
        pfa.timing_enable(0)
    kinds = [k for k, _ in recs]
    names = [pfa.kernel_name(k) for k in kinds]
    assert n1 == 2 and dropped == 0
    assert names[:3] == ["dense_layer_kernel", "iota_rows_kernel", "all_cand"], names
    assert names[-1] == "aggregate", names
    assert all(ms > 0 for _, ms in recs)
    # results with timing on equal those with timing off
    _, A2b, O2b = pfa.sparse_layer(Qd, Kd, Vd, None, A1, 256, win=32, shift=16)
    assert torch.equal(A2, A2b) and torch.equal(O2, O2b)


@pytest.mark.timeout(120)
@pytest.mark.parametrize("K_prev,K_l", [(1024, 256), (256, 128), (64, 32)])
def test_nonfinite_previous_map_terminates(K_prev, K_l):
    # NaN, negative and infinite previous weights violate the preconditions; the
    # kernels must still return (such keys count as weight 0) with valid indices.
    shape = (1, 2, 32, 32, 32)
    qt, kt, vt = (inputs.draw(800 + t, shape, "f32") for t in range(3))
    g = np.random.Generator(np.random.PCG64(801))
    n_wh, N = 2, 1024
    a = g.standard_normal((n_wh, N, K_prev)).astype(np.float32)
    a[..., ::7] = np.nan
    a[..., 3::11] = np.inf
    C = None if K_prev == N else torch.from_numpy(
        np.stack([g.permutation(N)[:K_prev] for _ in range(n_wh * N)]).astype(np.int32)).cuda()
    I, A, O = pfa.sparse_layer(to_dev(qt), to_dev(kt), to_dev(vt), C, torch.from_numpy(a).cuda(), K_l, win=32,
                               shift=0)
    torch.cuda.synchronize()
    Ig = I.cpu().numpy()
    assert (Ig >= 0).all() and (Ig < N).all()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,K2,shifts", [("bf16", 32, 256, (0, 16)), ("bf16", 16, 256, (16, 0)),
                                              ("f32", 16, 256, (0, 16)), ("bf16", 32, 1000, (3, 29)),
                                              ("bf16", 32, 1, (0, 0))])
def test_first_two_layers_fused(dtype, d, K2, shifts):
    # fused layers 1-2 (no A^1 in memory) against the fp64 oracle chain run unfused
    shape = (1, 2, 64, 96, d)
    q1, k1, v1, q2, k2, v2 = (inputs.draw(950 + t + d, shape, dtype) for t in range(6))
    n_wh, N = 2 * 6, 1024
    sel = np.arange(n_wh)
    tol = parity.TOL[dtype]
    lse = torch.empty((n_wh, N), dtype=torch.float32, device="cuda")
    O1, I2, A2, O2 = pfa.first_two_layers(*(to_dev(t) for t in (q1, k1, v1, q2, k2, v2)), K2, win=32,
                                          shift1=shifts[0], shift2=shifts[1], lse_out=lse)
    torch.cuda.synchronize()
    ref1 = oracle.layer(q1.exact, k1.exact, v1.exact, win=32, shift=shifts[0], K_l=N, wh_list=sel)
    parity.check_O(O1.cpu().numpy(), ref1["O"], tol)
    lse_ref = oracle.dense_lse(q1.exact, k1.exact, win=32, shift=shifts[0])
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= tol
    kw = dict(win=32, shift=shifts[1], K_l=K2, I_prev=None, A_prev=ref1["A"], i_shared=False, prev_compact=True,
              wh_list=sel)
    ref2 = oracle.layer(q2.exact, k2.exact, v2.exact, want_keys=True, **kw)
    st = parity.check_layer(gpu_I=I2.view(n_wh, N, K2).cpu().numpy(), gpu_A=A2.view(n_wh, N, K2).cpu().numpy(),
                            gpu_O=O2.cpu().numpy(), ref=ref2, cand=None, wh_list=sel, tol=tol,
                            rerun=parity.rerun_fn(q2.exact, k2.exact, v2.exact, **kw))
    assert st["rows"] == n_wh * N


@pytest.mark.timeout(120)
def test_first_two_layers_rejects_fp32_d32():
    Q = torch.zeros((1, 1, 32, 32, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(pfa.PfaError) as e:
        pfa.first_two_layers(Q, Q, Q, Q, Q, Q, 256, win=32)
    assert e.value.code == -2


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,K_prev,K_l", [("bf16", 64, 20), ("bf16", 128, 40), ("bf16", 256, 100),
                                              ("f32", 128, 12), ("f32", 100, 7)])
def test_nonfinite_V_row_reaches_only_rows_that_keep_it(dtype, K_prev, K_l):
    # V of slot 0 of every window holds +inf. Rows that did not keep slot 0 must get
    # the oracle's finite O, also where K_l is not a multiple of the aggregation
    # kernels' entry blocks (padding entries must add no 0 * inf term).
    B, heads, H, W, d, win = 1, 2, 64, 64, 32, 32
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(1200 + t + K_l, shape, dtype) for t in range(3))
    vdev, vex = vt.device.copy(), vt.exact.copy()
    vdev[:, :, ::win, ::win, 3] = np.float32(np.inf) if dtype == "f32" else np.uint16(0x7F80)
    vex[:, :, ::win, ::win, 3] = np.inf
    vt = inputs.Tensor(vdev, vex, dtype)
    N, nwin = win * win, (H // win) * (W // win)
    n_wh = B * heads * nwin
    g = np.random.Generator(np.random.PCG64(1300 + K_l))
    C = np.stack([np.sort(g.permutation(N)[:K_prev]) for _ in range(n_wh * N)]).astype(np.int32)
    C = C.reshape(B, heads, nwin, N, K_prev)
    a = (g.random((B, heads, nwin, N, K_prev)) + 0.05).astype(np.float32)
    I, A, O = pfa.sparse_layer(to_dev(qt), to_dev(kt), to_dev(vt), torch.from_numpy(C).cuda(),
                               torch.from_numpy(a).cuda(), K_l, win=win, shift=0)
    torch.cuda.synchronize()
    ref = oracle.layer(qt.exact, kt.exact, vex, win=win, shift=0, K_l=K_l, I_prev=C, A_prev=a.astype(np.float64),
                       wh_list=np.arange(n_wh), want_keys=True)
    Og = O.cpu().numpy()
    fin = np.isfinite(ref["O"]).all(-1)
    assert fin.sum() > 0.5 * fin.size and (~fin).sum() > 0, "case must mix rows with and without slot 0"
    # near-ties would change which rows keep slot 0: compare the kept sets first
    Ig = I.view(n_wh, N, K_l).cpu().numpy()
    same = (np.sort(Ig, -1) == np.sort(ref["I"], -1)).all(-1)
    assert same.mean() > 0.99
    keeps0 = (Ig == 0).any(-1)
    # pixel rows of window-head rows that kept slot 0 on the GPU or differ from the oracle are masked
    O_ref = ref["O"].copy()
    nwx = W // win
    for n, i in np.argwhere(keeps0 | ~same):
        b, h, wn = n // (heads * nwin), (n // nwin) % heads, n % nwin
        y, x = (wn // nwx) * win + i // win, (wn % nwx) * win + i % win
        O_ref[b, h, y, x] = np.nan
    mask = ~np.isnan(O_ref[..., 0])
    assert np.isfinite(Og[mask]).all(), "a row that did not keep slot 0 is not finite"
    parity.check_O(Og, O_ref, parity.TOL[dtype])
