"""GPU parity of the sparse-layer backward pass (through the C ABI) against the
fp64 backward oracle (``oracle.layer_backward``), whose pins are in
tests/test_oracle_backward_pins.py.

Every input comes from the seeded generators or from the oracle: the kept sets
I^l are the oracle forward's (the backward holds them fixed) and the GPU takes
the oracle's A^l rounded to fp32, while the oracle backward recomputes A^l in
fp64 from Q, K and A^{l-1}.

Rules (a reading of the forward's tolerances for gradients, which the pages do
not cover): tol = 1e-5 for fp32 inputs, 2e-3 for bf16 inputs;
  * dQ, dK, dV: per window-head, max |gpu - ref| over the window's pixels and
    the d columns <= tol * max |ref| over the same set (norm-relative: the
    gradients are sums with cancellation, so elementwise relative error is
    ill-posed where an entry is near zero);
  * dA^{l-1}: per row, max |gpu - ref| <= tol * max |ref row|, and exactly 0
    at every slot the layer dropped;
  * dbias (relative position bias): per head, max |gpu - ref| over the table
    <= tol * max |ref| over the head's table (each entry is a sum with
    cancellation over many pairs, as dQ's are).
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_progressive_window_amd import inputs, pfa, workloads
from tests import parity
from tests.test_gpu_workloads import sample_wh, to_dev

pytestmark = pytest.mark.gpu


def window_pixels(wh, heads, H, W, win, shift):
    """(b, h, y, x) index arrays of the N slots of window-head `wh`, slot order."""
    nwy, nwx = H // win, W // win
    wx = wh % nwx
    wy = (wh // nwx) % nwy
    h = (wh // (nwx * nwy)) % heads
    b = wh // (nwx * nwy * heads)
    t = np.arange(win * win)
    y = (wy * win + t // win + shift) % H
    x = (wx * win + t % win + shift) % W
    return b, h, y, x


def check_grads(gpu, ref, wh_list, heads, win, shift, tol):
    """dQ/dK/dV dicts of [B, heads, H, W, d] arrays; returns the worst ratios."""
    H, W = ref["dQ"].shape[2:4]
    worst = {}
    for name in ("dQ", "dK", "dV"):
        g = np.asarray(gpu[name], dtype=np.float64)
        r = ref[name]
        w_max = 0.0
        for wh in wh_list:
            b, h, y, x = window_pixels(int(wh), heads, H, W, win, shift)
            err = np.abs(g[b, h, y, x] - r[b, h, y, x]).max()
            scale = np.abs(r[b, h, y, x]).max()
            assert err <= tol * scale + 1e-30, f"{name} window-head {wh}: {err / scale:.3e} > {tol}"
            w_max = max(w_max, float(err / max(scale, 1e-30)))
        worst[name] = w_max
    return worst


def check_dA_prev(gpu, ref, tol):
    """gpu, ref: [n, N, K_prev] (ref fp64)."""
    g = np.asarray(gpu, dtype=np.float64)
    dropped = ref == 0.0
    assert (g[dropped] == 0.0).all(), "nonzero gradient at a dropped slot"
    err = np.abs(g - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    ok = err <= tol * scale + 1e-30
    worst = float((err / np.maximum(scale, 1e-30)).max())
    assert ok.all(), f"dA_prev mismatch: worst row {worst:.3e} > {tol}"
    return worst


def check_dbias(gpu, ref, tol):
    """gpu, ref: [heads, (2 win - 1)^2]."""
    g = np.asarray(gpu, dtype=np.float64)
    worst = 0.0
    for h in range(ref.shape[0]):
        err = np.abs(g[h] - ref[h]).max()
        scale = np.abs(ref[h]).max()
        assert err <= tol * scale + 1e-30, f"dbias head {h}: {err / scale:.3e} > {tol}"
        worst = max(worst, float(err / max(scale, 1e-30)))
    return worst


def bias_table(heads, win, seed, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((heads, (2 * win - 1) ** 2)) * scale).astype(np.float32)


def rand_lists(n_rows, N, K_prev, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.stack([g.permutation(N)[:K_prev] for _ in range(n_rows)]).astype(np.int32)


def rand_map(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.random(shape) + 1e-3
    return (a / a.sum(axis=-1, keepdims=True)).astype(np.float32)


def run_case(B, heads, H, W, d, win, shift, K_prev, K_l, dtype, seed, *, implicit=False, with_dA=True,
             want_dA_prev=True, zero_frac=0.0, subnormal_frac=0.0, with_bias=False):
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(seed + t, shape, dtype) for t in range(3))
    N = win * win
    nwin = (H // win) * (W // win)
    n_wh = B * heads * nwin
    lead = (B, heads, nwin)
    I_prev = None if implicit else rand_lists(n_wh * N, N, K_prev, seed + 5).reshape(lead + (N, K_prev))
    A_prev = rand_map(lead + (N, K_prev), seed + 6)
    if zero_frac or subnormal_frac:
        # zero (and subnormal) previous weights; with K_l above a row's positive
        # weights, slots of weight 0 are kept (their A^l is 0, their dA^{l-1} is not)
        g = np.random.Generator(np.random.PCG64(seed + 9))
        u = g.random(A_prev.shape)
        A_prev[u < zero_frac] = 0.0
        A_prev[(u >= zero_frac) & (u < zero_frac + subnormal_frac)] = np.float32(3e-41)
        A_prev[..., 0] = np.maximum(A_prev[..., 0], np.float32(0.5 / K_prev))
    Qd, Kd, Vd = to_dev(qt), to_dev(kt), to_dev(vt)
    Ipd = None if I_prev is None else torch.from_numpy(I_prev).cuda()
    Apd = torch.from_numpy(A_prev).cuda()
    table = bias_table(heads, win, seed + 10) if with_bias else None
    fwd = oracle.layer(qt.exact, kt.exact, vt.exact, win=win, shift=shift, K_l=K_l, I_prev=I_prev,
                       A_prev=A_prev.astype(np.float64), bias=table)
    I_l = torch.from_numpy(fwd["I"].reshape(lead + (N, K_l))).cuda()
    A_l = torch.from_numpy(fwd["A"].astype(np.float32).reshape(lead + (N, K_l))).cuda()
    dO = inputs.draw(seed + 7, shape, "f32").exact
    dA = inputs.draw(seed + 8, lead + (N, K_l), "f32").exact if with_dA else None
    dOd = torch.from_numpy(dO).cuda()
    dAd = None if dA is None else torch.from_numpy(dA).cuda()
    if with_bias:
        dQ, dK, dV, dAp, dbias = pfa.sparse_layer_backward_rpb(
            Qd, Kd, Vd, torch.from_numpy(table).cuda(), Ipd, Apd, I_l, A_l, dOd, dAd, win=win, shift=shift,
            K_prev=K_prev, want_dA_prev=want_dA_prev)
        again = pfa.sparse_layer_backward_rpb(Qd, Kd, Vd, torch.from_numpy(table).cuda(), Ipd, Apd, I_l, A_l, dOd,
                                              dAd, win=win, shift=shift, K_prev=K_prev, want_dA_prev=want_dA_prev)
        assert torch.equal(again[4], dbias), "the bias gradient differs between two calls"
    else:
        dQ, dK, dV, dAp = pfa.sparse_layer_backward(Qd, Kd, Vd, Ipd, Apd, I_l, A_l, dOd, dAd, win=win, shift=shift,
                                                    K_prev=K_prev, want_dA_prev=want_dA_prev)
    torch.cuda.synchronize()
    keep = fwd["I"]
    ref = oracle.layer_backward(qt.exact, kt.exact, vt.exact, win=win, shift=shift, keep=keep, dO=dO,
                                dA=None if dA is None else dA.reshape(n_wh, N, K_l),
                                I_prev=None if I_prev is None else I_prev.reshape(n_wh, N, K_prev),
                                A_prev=A_prev.reshape(n_wh, N, K_prev), prev_compact=True, bias=table)
    tol = parity.TOL[dtype]
    gpu = {"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}
    st = check_grads(gpu, ref, range(n_wh), heads, win, shift, tol)
    if want_dA_prev:
        st["dA_prev"] = check_dA_prev(dAp.view(n_wh, N, K_prev).cpu().numpy(), ref["dA_prev"], tol)
    else:
        assert dAp is None
    if with_bias:
        st["dbias"] = check_dbias(dbias.cpu().numpy(), ref["dbias"], tol)
    return st


CASES = [
    # dtype, d, win, shift, K_prev, K_l, implicit, with_dA
    ("f32", 32, 32, 16, 1024, 256, True, True),     # K and V passes in two kernels, dK/dV in column halves
    ("bf16", 32, 32, 16, 1024, 256, True, True),    # one row kernel with K and V in LDS
    ("f32", 16, 32, 0, 1024, 256, True, False),
    ("bf16", 16, 32, 16, 256, 128, False, True),
    ("f32", 32, 32, 16, 256, 128, False, True),
    ("f32", 32, 32, 0, 128, 64, False, True),
    ("bf16", 32, 32, 16, 64, 32, False, True),
    ("f32", 32, 32, 16, 32, 16, False, True),
    ("bf16", 32, 32, 0, 12, 5, False, True),        # ragged K_l (rows not 16-byte aligned)
    ("f32", 32, 16, 8, 256, 256, False, True),      # N = 256, nothing dropped
    ("f32", 16, 8, 4, 64, 13, False, False),        # N = 64
    ("bf16", 16, 16, 0, 100, 37, False, True),
    ("f32", 16, 6, 3, 20, 7, False, True),          # N = 36: dK/dV by LDS compare-and-swap adds
]


ZERO_CASES = [
    # dtype, d, win, shift, K_prev, K_l, implicit, zero_frac, subnormal_frac
    ("f32", 32, 32, 16, 1024, 256, True, 0.9, 0.0),   # K pass alone (fp32, d = 32), layer-2 shape
    ("bf16", 32, 32, 16, 1024, 256, True, 0.85, 0.05),  # K and V passes in one kernel
    ("f32", 32, 32, 0, 128, 64, False, 0.7, 0.1),
    ("bf16", 16, 16, 0, 100, 37, False, 0.75, 0.0),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,win,shift,K_prev,K_l,implicit,zero_frac,subnormal_frac", ZERO_CASES)
def test_backward_zero_previous_weights(dtype, d, win, shift, K_prev, K_l, implicit, zero_frac, subnormal_frac,
                                        capsys):
    """Previous maps with many zero (and subnormal) weights, so that rows keep
    slots of weight 0: their dA^{l-1} is exp(s) / sum_kept A^{l-1} exp(s) * g,
    not 0 (pinned by finite differences in the oracle's pins)."""
    st = run_case(1, 2, 2 * win, 2 * win, d, win, shift, K_prev, K_l, dtype, 900 + K_l + d, implicit=implicit,
                  zero_frac=zero_frac, subnormal_frac=subnormal_frac)
    with capsys.disabled():
        print(f"  zero weights {dtype} d={d} win={win} K={K_prev}->{K_l}: {st}", flush=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,win,shift,K_prev,K_l,implicit,with_dA", CASES)
def test_backward_random(dtype, d, win, shift, K_prev, K_l, implicit, with_dA, capsys):
    H = W = 2 * win
    st = run_case(1, 2, H, W, d, win, shift, K_prev, K_l, dtype, 700 + K_l + d, implicit=implicit,
                  with_dA=with_dA)
    with capsys.disabled():
        print(f"  backward {dtype} d={d} win={win} K {K_prev}->{K_l}: {st}", flush=True)


RPB_CASES = [
    # dtype, d, win, shift, K_prev, K_l, implicit, zero_frac
    ("f32", 32, 32, 16, 256, 128, False, 0.0),
    ("bf16", 32, 32, 0, 1024, 256, True, 0.0),
    ("f32", 32, 32, 16, 1024, 256, True, 0.9),     # zero weights: exact dA^{l-1} from scores with the bias
    ("bf16", 32, 32, 16, 64, 16, False, 0.0),
    ("f32", 16, 16, 8, 100, 37, False, 0.0),
    ("bf16", 16, 16, 0, 256, 64, True, 0.0),
    ("f32", 16, 16, 0, 64, 40, False, 0.7),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,win,shift,K_prev,K_l,implicit,zero_frac", RPB_CASES)
def test_backward_with_bias(dtype, d, win, shift, K_prev, K_l, implicit, zero_frac, capsys):
    """Sparse layer computed with a relative position bias: every gradient,
    including the bias table's, against the oracle backward with the same bias."""
    st = run_case(2, 2, 2 * win, 2 * win, d, win, shift, K_prev, K_l, dtype, 1500 + K_l + d, implicit=implicit,
                  zero_frac=zero_frac, with_bias=True)
    with capsys.disabled():
        print(f"  backward with bias {dtype} d={d} win={win} K {K_prev}->{K_l}: {st}", flush=True)


@pytest.mark.timeout(300)
def test_backward_without_dA_prev():
    run_case(1, 2, 64, 64, 32, 32, 16, 256, 64, "f32", 811, want_dA_prev=False)


@pytest.mark.timeout(300)
def test_backward_kernel_timing_records():
    pfa.timing_enable(16)
    try:
        run_case(1, 1, 32, 32, 32, 32, 0, 1024, 256, "f32", 901, implicit=True)
        recs, dropped = pfa.timing_read()
    finally:
        pfa.timing_enable(0)
    kinds = [k for k, _ in recs]
    assert kinds[-4:] == [6, 6, 11, 7], kinds      # V pass, K pass, exact dA^{l-1} rows, dK/dV (fp32, d = 32)
    assert dropped == 0 and all(ms > 0 for _, ms in recs)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers", [(workloads.PATCH64.name, (1, 2, 4, 5)), (workloads.MAP256.name, (1, 2, 4, 5))])
def test_backward_full_size(name, layers, capsys):
    """Full-size workload, every window-head on the GPU; 12 sampled window-heads
    carry the oracle chain's maps (previous map and the layer's I^l, A^l), the
    others a valid uniform map, as in the forward full-size tests."""
    w = workloads.BY_NAME[name]
    sel = sample_wh(w, 12)
    selt = torch.from_numpy(sel).cuda()
    N = w.N
    lead = (w.B, w.heads, w.n_windows)
    tol = parity.TOL[w.dtype]
    I_ref = A_ref = None
    for l in range(max(layers) + 1):
        qkv = inputs.qkv(w, 0, l)
        Q, K, V = (t.exact for t in qkv)
        fwd = oracle.layer(Q, K, V, win=w.win, shift=w.shifts[l], K_l=w.K[l], I_prev=I_ref,
                           A_prev=None if A_ref is None else A_ref.astype(np.float32).astype(np.float64),
                           prev_compact=True, wh_list=sel)
        if l in layers:
            K_prev, K_l = w.K[l - 1], w.K[l]
            Qd, Kd, Vd = (to_dev(t) for t in qkv)

            def full(values, fill, dtype):   # [n_wh, N, K]: the oracle's rows at sel, `fill` elsewhere
                t = fill.clone()
                t[selt] = torch.from_numpy(values.astype(dtype)).cuda()
                return t.view(lead + values.shape[1:])
            A_prev = full(A_ref.astype(np.float32), torch.full((w.n_wh, N, K_prev), 1.0 / K_prev, device="cuda"),
                          np.float32)
            I_prev = None if I_ref is None else full(
                I_ref, torch.arange(K_prev, dtype=torch.int32, device="cuda").expand(w.n_wh, N, K_prev), np.int32)
            I_l = full(fwd["I"], torch.arange(K_l, dtype=torch.int32, device="cuda").expand(w.n_wh, N, K_l), np.int32)
            A_l = full(fwd["A"].astype(np.float32), torch.full((w.n_wh, N, K_l), 1.0 / K_l, device="cuda"), np.float32)
            dO = torch.randn(Qd.shape, generator=torch.Generator().manual_seed(50 + l)).cuda()
            dA = torch.randn(lead + (N, K_l), generator=torch.Generator().manual_seed(60 + l)).cuda()
            dQ, dK, dV, dAp = pfa.sparse_layer_backward(Qd, Kd, Vd, I_prev, A_prev, I_l, A_l, dO, dA, win=w.win,
                                                        shift=w.shifts[l], K_prev=K_prev)
            torch.cuda.synchronize()
            ref = oracle.layer_backward(Q, K, V, win=w.win, shift=w.shifts[l], keep=fwd["I"], dO=dO.cpu().numpy(),
                                        dA=dA.view(-1, N, K_l)[selt].cpu().numpy(), I_prev=I_ref,
                                        A_prev=A_ref.astype(np.float32).astype(np.float64), prev_compact=True,
                                        wh_list=sel)
            gpu = {"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}
            st = check_grads(gpu, ref, sel, w.heads, w.win, w.shifts[l], tol)
            st["dA_prev"] = check_dA_prev(dAp.view(-1, N, K_prev)[selt].cpu().numpy(), ref["dA_prev"], tol)
            with capsys.disabled():
                print(f"  {w.name} layer {l + 1} backward: {st}", flush=True)
            del Qd, Kd, Vd, dQ, dK, dV, dAp, I_prev, A_prev, I_l, A_l
        I_ref, A_ref = fwd["I"], fwd["A"]


DENSE = [
    # dtype, d, win, shift, with_dA, with_bias
    ("f32", 32, 32, 16, True, False),
    ("bf16", 32, 32, 0, True, False),
    ("f32", 16, 16, 8, False, False),
    ("bf16", 16, 8, 4, True, False),
    ("f32", 32, 32, 16, True, True),
    ("bf16", 16, 16, 0, True, True),
    ("bf16", 32, 32, 0, False, True),
    ("f32", 16, 16, 8, False, True),
    ("f32", 32, 24, 12, True, False),        # N = 576: the last workgroup has idle waves
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,win,shift,with_dA,with_bias", DENSE)
def test_dense_backward(dtype, d, win, shift, with_dA, with_bias, capsys):
    """Backward of the dense first layer (all N slots kept, no previous map),
    against the oracle backward with every slot kept; the GPU takes the oracle's
    log denominators (fp64 rounded to fp32)."""
    B, heads, H, W = 1, 2, 2 * win, 2 * win
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(1300 + d + win + t, shape, dtype) for t in range(3))
    N = win * win
    n_wh = B * heads * 4
    lead = (B, heads, 4)
    table = None
    if with_bias:
        table = (np.random.Generator(np.random.PCG64(1310)).standard_normal((heads, (2 * win - 1) ** 2))
                 ).astype(np.float32)
    lse = oracle.dense_lse(qt.exact, kt.exact, win=win, shift=shift, bias=table).astype(np.float32)
    dO = inputs.draw(1320, shape, "f32").exact
    dA = inputs.draw(1321, lead + (N, N), "f32").exact if with_dA else None
    args = (to_dev(qt), to_dev(kt), to_dev(vt))
    lse_d = torch.from_numpy(lse).cuda().view(lead + (N,))
    dA_d = None if dA is None else torch.from_numpy(dA).cuda()
    if with_bias:   # with the bias gradient (the plain call is checked against it below)
        dQ, dK, dV, dbias = pfa.dense_layer_backward_rpb(*args, torch.from_numpy(table).cuda(), lse_d,
                                                         torch.from_numpy(dO).cuda(), dA_d, win=win, shift=shift)
        plain = pfa.dense_layer_backward(*args, lse_d, torch.from_numpy(dO).cuda(), dA_d, win=win, shift=shift,
                                         bias=torch.from_numpy(table).cuda())
        torch.cuda.synchronize()
        for x, y in zip((dQ, dK, dV), plain):
            assert torch.equal(x, y), "the bias gradient changed the other gradients"
        again = pfa.dense_layer_backward_rpb(*args, torch.from_numpy(table).cuda(), lse_d, torch.from_numpy(dO).cuda(),
                                             dA_d, win=win, shift=shift)
        assert torch.equal(again[3], dbias), "the bias gradient differs between two calls"
    else:
        dQ, dK, dV = pfa.dense_layer_backward(*args, lse_d, torch.from_numpy(dO).cuda(), dA_d, win=win, shift=shift)
    torch.cuda.synchronize()
    keep = np.broadcast_to(np.arange(N, dtype=np.int32), (n_wh, N, N)).copy()
    ref = oracle.layer_backward(qt.exact, kt.exact, vt.exact, win=win, shift=shift, keep=keep, dO=dO,
                                dA=None if dA is None else dA.reshape(n_wh, N, N), bias=table)
    gpu = {"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}
    st = check_grads(gpu, ref, range(n_wh), heads, win, shift, parity.TOL[dtype])
    if with_bias:
        st["dbias"] = check_dbias(dbias.cpu().numpy(), ref["dbias"], parity.TOL[dtype])
    with capsys.disabled():
        print(f"  dense backward {dtype} d={d} win={win} dA={with_dA} bias={with_bias}: {st}", flush=True)


def check_grads_global(gpu, ref, tol):
    """Global mode: per (image, head) plane, max |gpu - ref| <= tol * max |ref|."""
    worst = {}
    for name in ("dQ", "dK", "dV"):
        g = np.asarray(gpu[name], dtype=np.float64)
        r = ref[name]
        w_max = 0.0
        for b in range(r.shape[0]):
            for h in range(r.shape[1]):
                err = np.abs(g[b, h] - r[b, h]).max()
                scale = np.abs(r[b, h]).max()
                assert err <= tol * scale + 1e-30, f"{name} plane ({b}, {h}): {err / scale:.3e} > {tol}"
                w_max = max(w_max, float(err / max(scale, 1e-30)))
        worst[name] = w_max
    return worst


def run_global_case(B, heads, H, W, d, K_prev, K_l, dtype, seed, *, with_A_prev, with_dA=True, zero_frac=0.0,
                    I_shared=None):
    """Global mode (win = 0): each token's candidates are K_prev tokens of the whole
    map (seeded distinct random lists per row and head, or I_shared [N, K_prev]
    for every head)."""
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(seed + t, shape, dtype) for t in range(3))
    N = H * W
    n_wh = B * heads
    lead = (B, heads)
    if I_shared is not None:
        I_prev = np.broadcast_to(I_shared, lead + (N, K_prev)).copy()
    else:
        I_prev = rand_lists(n_wh * N, N, K_prev, seed + 5).reshape(lead + (N, K_prev))
    A_prev = None
    if with_A_prev:
        A_prev = rand_map(lead + (N, K_prev), seed + 6)
        if zero_frac:
            u = np.random.Generator(np.random.PCG64(seed + 9)).random(A_prev.shape)
            A_prev[u < zero_frac] = 0.0
            A_prev[..., 0] = np.maximum(A_prev[..., 0], np.float32(0.5 / K_prev))
    fwd = oracle.layer(qt.exact, kt.exact, vt.exact, win=0, shift=0, K_l=K_l,
                       I_prev=I_prev.reshape(B, heads, 1, N, K_prev),
                       A_prev=None if A_prev is None else A_prev.reshape(B, heads, 1, N, K_prev).astype(np.float64))
    I_l = torch.from_numpy(fwd["I"].reshape(lead + (N, K_l))).cuda()
    A_l = torch.from_numpy(fwd["A"].astype(np.float32).reshape(lead + (N, K_l))).cuda()
    dO = inputs.draw(seed + 7, shape, "f32").exact
    dA = inputs.draw(seed + 8, lead + (N, K_l), "f32").exact if with_dA else None
    dQ, dK, dV, dAp = pfa.sparse_layer_backward(
        to_dev(qt), to_dev(kt), to_dev(vt), torch.from_numpy(I_prev).cuda(),
        None if A_prev is None else torch.from_numpy(A_prev).cuda(), I_l, A_l, torch.from_numpy(dO).cuda(),
        None if dA is None else torch.from_numpy(dA).cuda(), win=0, shift=0, K_prev=K_prev)
    torch.cuda.synchronize()
    ref = oracle.layer_backward(qt.exact, kt.exact, vt.exact, win=0, shift=0, keep=fwd["I"], dO=dO,
                                dA=None if dA is None else dA.reshape(n_wh, N, K_l),
                                I_prev=I_prev.reshape(n_wh, N, K_prev),
                                A_prev=None if A_prev is None else A_prev.reshape(n_wh, N, K_prev),
                                prev_compact=True)
    tol = parity.TOL[dtype]
    st = check_grads_global({"dQ": dQ.cpu().numpy(), "dK": dK.cpu().numpy(), "dV": dV.cpu().numpy()}, ref, tol)
    if with_A_prev:
        st["dA_prev"] = check_dA_prev(dAp.view(n_wh, N, K_prev).cpu().numpy(), ref["dA_prev"], tol)
    else:
        assert dAp is None
    return st


GLOBAL_CASES = [
    # dtype, d, H, W, K_prev, K_l, with_A_prev, zero_frac
    ("bf16", 32, 64, 64, 64, 64, False, 0.0),      # 4096 tokens: gathers from L2, 4 token ranges for dK/dV
    ("f32", 32, 64, 64, 64, 32, True, 0.0),        # selection and dA^{l-1}
    ("bf16", 16, 48, 64, 100, 37, True, 0.7),      # zero weights: exact dA^{l-1}, slots found by search
    ("f32", 32, 32, 32, 256, 64, True, 0.0),       # 1024 tokens: staged like a window
    ("bf16", 32, 18, 18, 40, 40, False, 0.0),      # 324 tokens (not a multiple of 16)
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,H,W,K_prev,K_l,with_A_prev,zero_frac", GLOBAL_CASES)
def test_backward_global_mode(dtype, d, H, W, K_prev, K_l, with_A_prev, zero_frac, capsys):
    st = run_global_case(1, 2, H, W, d, K_prev, K_l, dtype, 1600 + K_l + d, with_A_prev=with_A_prev,
                         zero_frac=zero_frac)
    with capsys.disabled():
        print(f"  global backward {dtype} d={d} {H}x{W} K {K_prev}->{K_l}: {st}", flush=True)


@pytest.mark.timeout(300)
def test_backward_global_workload(capsys):
    """The individualized-attention workload (one index matrix shared by the 6
    heads, k = 64 kept of 64): its backward against the oracle's."""
    w = workloads.GLOBAL64
    st = run_global_case(w.B, w.heads, w.H, w.W, w.d, w.k_global, w.k_global, w.dtype, 1650, with_A_prev=False,
                         I_shared=inputs.global_index(w))
    with capsys.disabled():
        print(f"  {w.name} backward: {st}", flush=True)


FUSED_BWD = [
    # dtype, d, (shift1, shift2), K2
    ("bf16", 32, (0, 16), 256),
    ("bf16", 16, (16, 0), 128),
    ("f32", 16, (0, 16), 256),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,d,shifts,K2", FUSED_BWD)
def test_first_two_layers_backward(dtype, d, shifts, K2, capsys):
    """Backward of the fused first two layers against the oracle's unfused chain:
    the second layer's backward (every slot a candidate, A^{l-1} = the first
    layer's map) and then the dense first layer's with that dA^1. The GPU takes the
    oracle's lse1, I2 and A2 (rounded to fp32), as the forward would give them."""
    B, heads, win, H, W = 1, 2, 32, 64, 64
    shape = (B, heads, H, W, d)
    q1, k1, v1, q2, k2, v2 = (inputs.draw(1700 + d + K2 + t, shape, dtype) for t in range(6))
    N, n_wh, lead = win * win, B * heads * 4, (B, heads, 4)
    s1, s2 = shifts
    ref1 = oracle.layer(q1.exact, k1.exact, v1.exact, win=win, shift=s1, K_l=N)
    lse1 = oracle.dense_lse(q1.exact, k1.exact, win=win, shift=s1).astype(np.float32)
    ref2 = oracle.layer(q2.exact, k2.exact, v2.exact, win=win, shift=s2, K_l=K2, I_prev=None, A_prev=ref1["A"],
                        prev_compact=True)
    dO1 = inputs.draw(1790, shape, "f32").exact
    dO2 = inputs.draw(1791, shape, "f32").exact
    dA2 = inputs.draw(1792, lead + (N, K2), "f32").exact
    outs = pfa.first_two_layers_backward(
        *(to_dev(t) for t in (q1, k1, v1, q2, k2, v2)), torch.from_numpy(lse1).cuda().view(lead + (N,)),
        torch.from_numpy(ref2["I"].reshape(lead + (N, K2))).cuda(),
        torch.from_numpy(ref2["A"].astype(np.float32).reshape(lead + (N, K2))).cuda(),
        torch.from_numpy(dO1).cuda(), torch.from_numpy(dO2).cuda(), torch.from_numpy(dA2).cuda(), win=win,
        shift1=s1, shift2=s2)
    torch.cuda.synchronize()
    bwd2 = oracle.layer_backward(q2.exact, k2.exact, v2.exact, win=win, shift=s2, keep=ref2["I"], dO=dO2,
                                 dA=dA2.reshape(n_wh, N, K2), I_prev=None, A_prev=ref1["A"], prev_compact=True)
    keep1 = np.broadcast_to(np.arange(N, dtype=np.int32), (n_wh, N, N)).copy()
    bwd1 = oracle.layer_backward(q1.exact, k1.exact, v1.exact, win=win, shift=s1, keep=keep1, dO=dO1,
                                 dA=bwd2["dA_prev"])
    tol = parity.TOL[dtype]
    g = [t.cpu().numpy() for t in outs]
    st1 = check_grads({"dQ": g[0], "dK": g[1], "dV": g[2]}, bwd1, range(n_wh), heads, win, s1, tol)
    st2 = check_grads({"dQ": g[3], "dK": g[4], "dV": g[5]}, bwd2, range(n_wh), heads, win, s2, tol)
    with capsys.disabled():
        print(f"  fused layers 1-2 backward {dtype} d={d} shifts={shifts} K2={K2}: layer 1 {st1}; layer 2 {st2}",
              flush=True)
