"""GPU test of the entry point that allocates nothing,
pfa_dense_layer_backward_noalloc (its scratch memory is the library's static
device array): two calls in a row, the second on a smaller input, must give
exactly what pfa_dense_layer_backward (same kernels, caller-owned workspace)
gives on the same inputs, and match the fp64 oracle within the dtype's
tolerance (parity rules of tests/parity.py)."""

import numpy as np
import pytest
import torch

import oracle
from sparse_progressive_window_amd import inputs, pfa
from tests import parity
from tests.test_gpu_backward import check_grads
from tests.test_gpu_workloads import to_dev

pytestmark = pytest.mark.gpu


def _case(B, heads, H, W, d, win, shift, dtype, seed, with_dA):
    shape = (B, heads, H, W, d)
    qt, kt, vt = (inputs.draw(seed + t, shape, dtype) for t in range(3))
    N = win * win
    nwin = (H // win) * (W // win)
    lead = (B, heads, nwin)
    lse = oracle.dense_lse(qt.exact, kt.exact, win=win, shift=shift).astype(np.float32)
    dO = inputs.draw(seed + 10, shape, "f32").exact
    dA = inputs.draw(seed + 11, lead + (N, N), "f32").exact if with_dA else None
    dev = dict(Q=to_dev(qt), K=to_dev(kt), V=to_dev(vt), lse=torch.from_numpy(lse).cuda().view(lead + (N,)),
               dO=torch.from_numpy(dO).cuda(), dA=None if dA is None else torch.from_numpy(dA).cuda())
    host = dict(q=qt.exact, k=kt.exact, v=vt.exact, dO=dO, dA=dA, n_wh=B * heads * nwin, N=N)
    return dict(dev=dev, host=host, win=win, shift=shift, heads=heads, dtype=dtype)


def _call(fn, c):
    t = c["dev"]
    return fn(t["Q"], t["K"], t["V"], t["lse"], t["dO"], t["dA"], win=c["win"], shift=c["shift"])


@pytest.mark.timeout(300)
def test_noalloc_dense_backward_matches_workspace_entry_point():
    big = _case(2, 3, 64, 96, 32, 32, 16, "f32", 1500, True)     # 36 window-heads of 1024 slots
    small = _case(1, 2, 32, 48, 16, 16, 8, "bf16", 1600, False)  # 12 window-heads of 256 slots
    # two calls in a row on the static scratch array, the second smaller
    got = [_call(pfa.dense_layer_backward_noalloc, big), _call(pfa.dense_layer_backward_noalloc, small)]
    torch.cuda.synchronize()
    for c, g in zip((big, small), got):
        want = _call(pfa.dense_layer_backward, c)
        torch.cuda.synchronize()
        for name, x, y in zip(("dQ", "dK", "dV"), g, want):
            assert torch.equal(x, y), f"{name} differs from pfa_dense_layer_backward"
        h = c["host"]
        N, n_wh = h["N"], h["n_wh"]
        keep = np.broadcast_to(np.arange(N, dtype=np.int32), (n_wh, N, N)).copy()
        ref = oracle.layer_backward(h["q"], h["k"], h["v"], win=c["win"], shift=c["shift"], keep=keep, dO=h["dO"],
                                    dA=None if h["dA"] is None else h["dA"].reshape(n_wh, N, N))
        st = check_grads({"dQ": g[0].cpu().numpy(), "dK": g[1].cpu().numpy(), "dV": g[2].cpu().numpy()}, ref,
                         range(n_wh), c["heads"], c["win"], c["shift"], parity.TOL[c["dtype"]])
        print(f"  no-allocation dense backward {c['dtype']} win={c['win']}: {st}", flush=True)
