"""GPU parity at the full workload sizes (through the C ABI) against the fp64 oracle.

Per-layer tests run each workload at its full size, in the launch configuration
the benchmark times, and compare every window-head (the 640x384 map: every
window-head of one block, a sample of the other five): the previous map
(I^{l-1}, A^{l-1}) comes from the oracle's own chain (rounded to fp32, the
dtype the C ABI takes), so both sides see identical inputs; window-heads
outside the compared set get a valid uniform map. Chain tests run the
GPU free-running at small sizes and compare every row. Rules: tests/parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_progressive_window_amd import inputs, pfa, workloads
from tests import parity

pytestmark = pytest.mark.gpu


def to_dev(t: inputs.Tensor):
    if t.dtype == "f32":
        return torch.from_numpy(t.device).cuda()
    return torch.from_numpy(t.device.view(np.int16)).cuda().view(torch.bfloat16)


def sample_wh(w: workloads.Workload, count: int):
    """Spread of window-heads: first, last, the wrapping window of each head
    (last row and column of windows), and a seeded random rest."""
    n = w.n_wh
    nwin = w.n_windows
    picks = {0, n - 1}
    for h in range(w.heads):
        picks.add(h * nwin + nwin - 1)
    g = np.random.Generator(np.random.PCG64(w.seed_base + 77))
    while len(picks) < min(count, n):
        picks.add(int(g.integers(0, n)))
    return np.array(sorted(picks), dtype=np.int64)


def gpu_rows(x, sel):
    t = x.reshape(-1, x.shape[-2], x.shape[-1])
    return t[torch.from_numpy(sel).cuda()].cpu().numpy()


def run_layer_parity(w, block, layers, sel, log, chunk=48):
    """The workload's chain at full size on the GPU, layer by layer, with the
    previous map of the window-heads in `sel` taken from the oracle's own chain
    (teacher forcing; rounded to fp32, the dtype the C ABI takes) and a valid
    uniform map elsewhere. Every row of every window-head in `sel` is compared;
    the oracle runs `chunk` window-heads at a time (its fp64 keys per chunk)."""
    N, tol = w.N, parity.TOL[w.dtype]
    I_ref = A_ref = None              # oracle's previous map on the window-heads of sel
    selt = torch.from_numpy(sel).cuda()
    for l in range(layers):
        qkv = inputs.qkv(w, block, l)
        Qd, Kd, Vd = (to_dev(t) for t in qkv)
        Q, K, V = (t.exact for t in qkv)
        shift, K_l = w.shifts[l], w.K[l]
        A32 = None if A_ref is None else A_ref.astype(np.float32)
        if l == 0:
            I, A, O = pfa.dense_layer(Qd, Kd, Vd, K_l, win=w.win, shift=shift, want_A=True,
                                      want_I=K_l < N)
            if I is None:
                I = torch.arange(N, dtype=torch.int32, device="cuda").expand(A.shape).contiguous()
        else:
            K_prev = w.K[l - 1]
            shape = (w.n_wh, N, K_prev)
            A_dev = torch.full(shape, 1.0 / K_prev, dtype=torch.float32, device="cuda")
            A_dev[selt] = torch.from_numpy(A32).cuda()
            if l == 1 and K_prev == N:
                I_dev = None
            else:
                I_dev = torch.arange(K_prev, dtype=torch.int32, device="cuda").expand(shape).contiguous()
                I_dev[selt] = torch.from_numpy(I_ref).cuda()
            lead = (w.B, w.heads, w.n_windows)
            I, A, O = pfa.sparse_layer(Qd, Kd, Vd, None if I_dev is None else I_dev.view(lead + (N, K_prev)),
                                       A_dev.view(lead + (N, K_prev)), K_l, win=w.win, shift=shift)
            del A_dev, I_dev
        torch.cuda.synchronize()
        Ig, Ag, Og = gpu_rows(I, sel), gpu_rows(A, sel), O.cpu().numpy()
        del Qd, Kd, Vd, I, A, O
        total = {"rows": 0, "tie_rows": 0, "max_gap_used": 0.0, "max_rel_A": 0.0, "rows_O": 0, "max_rel_O": 0.0}
        I_next, A_next = [], []
        for c0 in range(0, len(sel), chunk):
            cs = sel[c0:c0 + chunk]
            Ip = None if I_ref is None else I_ref[c0:c0 + chunk]
            Ap = None if A32 is None else A32[c0:c0 + chunk].astype(np.float64)
            kw = dict(win=w.win, shift=shift, K_l=K_l, I_prev=Ip, A_prev=Ap, i_shared=False, prev_compact=True,
                      wh_list=cs)
            ref = oracle.layer(Q, K, V, want_keys=True, **kw)
            st = parity.check_layer(gpu_I=Ig[c0:c0 + chunk], gpu_A=Ag[c0:c0 + chunk], gpu_O=Og, ref=ref, cand=Ip,
                                    wh_list=cs, tol=tol, rerun=parity.rerun_fn(Q, K, V, **kw))
            for k in ("rows", "tie_rows", "rows_O"):
                total[k] += st[k]
            for k in ("max_gap_used", "max_rel_A", "max_rel_O"):
                total[k] = max(total[k], st[k])
            I_next.append(ref["I"])
            A_next.append(ref["A"])
            del ref
        log(f"{w.name} block {block} layer {l + 1} ({len(sel)} of {w.n_wh} window-heads): {total}")
        I_ref, A_ref = np.concatenate(I_next), np.concatenate(A_next)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", [workloads.TINY.name, workloads.MAP256.name, workloads.PATCH64.name])
def test_layers_full_size_every_window_head(name, capsys):
    w = workloads.BY_NAME[name]
    with capsys.disabled():
        run_layer_parity(w, 0, w.layers, np.arange(w.n_wh), lambda s: print(s, flush=True))


@pytest.mark.timeout(900)
def test_layers_full_size_map640(capsys):
    # every window-head of block 5, a sample of each other block
    w = workloads.MAP640
    with capsys.disabled():
        log = lambda s: print(s, flush=True)   # noqa: E731
        run_layer_parity(w, 5, w.layers, np.arange(w.n_wh), log)
        for block in range(5):
            run_layer_parity(w, block, w.layers, sample_wh(w, 8), log)


@pytest.mark.timeout(300)
def test_global_individualized(capsys):
    w = workloads.GLOBAL64
    Qt, Kt, Vt = inputs.qkv(w, 0, 0)
    Iidx = inputs.global_index(w)
    N, k = w.N, w.k_global
    I_dev = torch.from_numpy(Iidx).cuda().view(1, 1, N, k)
    I, A, O = pfa.sparse_layer(to_dev(Qt), to_dev(Kt), to_dev(Vt), I_dev, None, k, win=0, i_shared=True)
    torch.cuda.synchronize()
    sel = np.arange(w.heads)
    Ip = Iidx.reshape(1, 1, 1, N, k)
    ref = oracle.layer(Qt.exact, Kt.exact, Vt.exact, win=0, shift=0, K_l=k, I_prev=Ip, i_shared=True,
                       wh_list=sel, want_keys=True)
    st = parity.check_layer(gpu_I=gpu_rows(I, sel), gpu_A=gpu_rows(A, sel), gpu_O=O.cpu().numpy(), ref=ref,
                            cand=np.broadcast_to(Iidx, (w.heads, N, k)), wh_list=sel,
                            tol=parity.TOL[w.dtype],
                            rerun=parity.rerun_fn(Qt.exact, Kt.exact, Vt.exact, win=0, shift=0, K_l=k,
                                                  I_prev=Ip, A_prev=None, i_shared=True,
                                                  prev_compact=False, wh_list=sel))
    with capsys.disabled():
        print(f"{w.name}: {st}", flush=True)


@pytest.mark.timeout(600)
def test_first_two_layers_fused_full_size(capsys):
    # the bf16 training-patch batch at full size with layers 1-2 fused (no A^1),
    # sampled window-heads against the fp64 oracle's unfused chain
    w = workloads.PATCH64
    sel = sample_wh(w, 12)
    q1, k1, v1 = inputs.qkv(w, 0, 0)
    q2, k2, v2 = inputs.qkv(w, 0, 1)
    O1, I2, A2, O2 = pfa.first_two_layers(*(to_dev(t) for t in (q1, k1, v1, q2, k2, v2)), w.K[1], win=w.win,
                                          shift1=w.shifts[0], shift2=w.shifts[1])
    torch.cuda.synchronize()
    tol = parity.TOL[w.dtype]
    ref1 = oracle.layer(q1.exact, k1.exact, v1.exact, win=w.win, shift=w.shifts[0], K_l=w.N, wh_list=sel)
    st1 = parity.check_O(O1.cpu().numpy(), ref1["O"], tol)
    kw = dict(win=w.win, shift=w.shifts[1], K_l=w.K[1], I_prev=None, A_prev=ref1["A"], i_shared=False,
              prev_compact=True, wh_list=sel)
    ref2 = oracle.layer(q2.exact, k2.exact, v2.exact, want_keys=True, **kw)
    st2 = parity.check_layer(gpu_I=gpu_rows(I2, sel), gpu_A=gpu_rows(A2, sel), gpu_O=O2.cpu().numpy(), ref=ref2,
                             cand=None, wh_list=sel, tol=tol, rerun=parity.rerun_fn(q2.exact, k2.exact, v2.exact, **kw))
    with capsys.disabled():
        print(f"{w.name} fused layers 1-2: layer 1 {st1}; layer 2 {st2}", flush=True)
