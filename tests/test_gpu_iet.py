"""GPU parity of the index-matrix propagation (through the C ABI) against the
oracle (``oracle.iet_propagate``; pins in tests/test_oracle_iet_pins.py).
Integer outputs: compared bit-exactly (both sides rank on the same fp32 score,
the heads' maps added in head order)."""

import numpy as np
import pytest
import torch

import oracle
from sparse_progressive_window_amd import inputs, pfa, workloads

pytestmark = pytest.mark.gpu


def rand_index(B, N, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.stack([g.permutation(N)[:k] for _ in range(B * N)]).astype(np.int32).reshape(B, N, k)


def check(I, A, k1, k2):
    out, cnt = pfa.iet_propagate(torch.from_numpy(I).cuda(), torch.from_numpy(A).cuda(), k1, k2)
    torch.cuda.synchronize()
    out, cnt = out.cpu().numpy(), cnt.cpu().numpy()
    for b in range(I.shape[0]):
        ro, rc = oracle.iet_propagate(I[b], A[b], k1, k2)
        np.testing.assert_array_equal(cnt[b], rc)
        np.testing.assert_array_equal(out[b], ro)
    return float(cnt.mean())


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B,N,k,n_maps,k1,k2,scores", [
    (2, 300, 16, 3, 9, 4, "random"),
    (1, 1000, 64, 6, 22, 12, "random"),
    (1, 777, 64, 2, 64, 64, "random"),     # every candidate kept, widest output
    (1, 200, 1, 1, 1, 1, "random"),        # one candidate per row
    (1, 500, 32, 4, 20, 10, "equal"),      # all scores tie: lowest token indices
    (2, 129, 24, 3, 14, 7, "grid"),        # many ties on a coarse grid
])
def test_propagate_random(B, N, k, n_maps, k1, k2, scores):
    I = rand_index(B, N, k, 100 + N)
    g = np.random.Generator(np.random.PCG64(200 + N))
    if scores == "equal":
        A = np.full((B, n_maps, N, k), 0.25, np.float32)
    elif scores == "grid":
        A = (g.integers(0, 4, (B, n_maps, N, k)) / 4).astype(np.float32)
    else:
        A = g.random((B, n_maps, N, k)).astype(np.float32)
    check(I, A, k1, k2)


@pytest.mark.timeout(600)
def test_propagate_global_workload(capsys):
    """The global workload (64x64 map, 6 heads, k = 64, one index matrix): the
    maps of its individualized attention layer (fp64 oracle, rounded to fp32)
    drive the propagation with each block's (k1, k2)."""
    w = workloads.GLOBAL64
    Qt, Kt, Vt = inputs.qkv(w, 0, 0)
    Iidx = inputs.global_index(w)
    N, k = w.N, w.k_global
    ref = oracle.layer(Qt.exact, Kt.exact, Vt.exact, win=0, shift=0, K_l=k, I_prev=Iidx.reshape(1, 1, 1, N, k),
                       i_shared=True, wh_list=np.arange(w.heads))
    # the layer keeps every candidate in I order: its map is aligned with I
    assert (ref["I"] == Iidx[None]).all()
    A = ref["A"].astype(np.float32).reshape(1, w.heads, N, k)
    I = Iidx.reshape(1, N, k)
    sizes = []
    for k1, k2 in zip((22, 20, 14, 12), (12, 10, 7, 6)):
        sizes.append(check(I, A, k1, k2))
    with capsys.disabled():
        print(f"  {w.name}: mean propagated set sizes {sizes}", flush=True)
