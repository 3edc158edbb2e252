"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/pfa.h declares, and rejects bad arguments with the documented
codes before touching any pointer or the HIP runtime."""

import ctypes
import os
import re

import pytest

from sparse_progressive_window_amd import pfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pfa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pfa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pfa._LIB_PATH):
        from sparse_progressive_window_amd import build
        build.build()
    return pfa.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"pfa_dense_layer", "pfa_sparse_layer", "pfa_first_two_layers", "pfa_sparse_layer_backward",
            "pfa_sparse_layer_backward_workspace", "pfa_iet_propagate", "pfa_iet_propagate_workspace",
            "pfa_dense_layer_rpb", "pfa_sparse_layer_rpb", "pfa_dense_layer_backward",
            "pfa_dense_layer_backward_workspace", "pfa_sparse_layer_backward_rpb",
            "pfa_sparse_layer_backward_rpb_workspace", "pfa_dense_layer_backward_rpb",
            "pfa_dense_layer_backward_rpb_workspace", "pfa_first_two_layers_backward",
            "pfa_first_two_layers_backward_workspace",
            "pfa_strerror", "pfa_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_timing_calls_without_device(lib):
    # enabling with 0 / reading an empty record list touch no HIP state
    assert lib.pfa_timing_enable(-1) == -1
    assert lib.pfa_timing_enable(1 << 21) == -1
    assert lib.pfa_timing_enable(0) == 0
    assert lib.pfa_timing_count() == 0
    n, dropped = ctypes.c_int32(7), ctypes.c_int32(7)
    assert lib.pfa_timing_read(None, None, 0, ctypes.byref(n), ctypes.byref(dropped)) == 0
    assert (n.value, dropped.value) == (0, 0)
    assert lib.pfa_timing_read(None, None, 0, None, None) == -1
    assert lib.pfa_timing_read(None, None, 4, ctypes.byref(n), None) == -1
    assert lib.pfa_timing_read(None, None, -1, ctypes.byref(n), None) == -1
    names = [lib.pfa_kernel_name(k).decode() for k in range(14)]
    assert names == ["dense_layer_kernel", "all_cand", "sparse_layer_kernel",
                     "sparse_layer_kernel(select)", "aggregate", "iota_rows_kernel", "bwd_rows_kernel",
                     "bwd_dkv", "iet_rank_kernel", "iet_union_kernel", "dense_bwd", "bwd_exact_dap_kernel",
                     "dbias", "first_map_kept_kernel"]
    assert lib.pfa_kernel_name(99) == b"unknown"


def test_version_and_strerror(lib):
    assert lib.pfa_version() == 10000
    assert lib.pfa_strerror(0) == b"ok"
    assert lib.pfa_strerror(-1) == b"invalid argument"
    assert lib.pfa_strerror(-2) == b"unsupported configuration"
    assert lib.pfa_strerror(-3) == b"HIP runtime error"
    assert lib.pfa_strerror(12345) == b"unknown error code"


def shape(B=1, heads=1, H=32, W=32, d=32, win=32, shift=0, dtype=0):
    return pfa.PfaShape(B, heads, H, W, d, win, shift, dtype)


def sparse(lib, s, K_prev=64, K_l=16, I_prev=FAKE, outs=(FAKE, FAKE, FAKE)):
    return lib.pfa_sparse_layer(ctypes.byref(s) if s is not None else None, FAKE, FAKE, FAKE, I_prev, 0,
                                FAKE, K_prev, K_l, *outs, None)


def dense(lib, s, K1=1024, I=None, A=None, O=FAKE, lse=None):
    return lib.pfa_dense_layer(ctypes.byref(s) if s is not None else None, FAKE, FAKE, FAKE, K1, I, A, lse, O,
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=8), -2), (dict(d=64), -2), (dict(dtype=7), -2), (dict(win=64, H=64, W=64), -2),
    (dict(H=33), -1), (dict(shift=32), -1), (dict(shift=-1), -1), (dict(B=0), -1), (dict(heads=0), -1),
    (dict(win=0, shift=1), -1), (dict(win=0, H=4096, W=4096), -2), (dict(win=-1), -1),
])
def test_sparse_shape_validation(lib, kw, code):
    assert sparse(lib, shape(**kw)) == code


def test_sparse_size_validation(lib):
    assert sparse(lib, None) == -1
    assert sparse(lib, shape(), K_l=0) == -1
    assert sparse(lib, shape(), K_l=65, K_prev=64) == -1
    assert sparse(lib, shape(), K_prev=0) == -1
    assert sparse(lib, shape(), K_prev=2000) == -1                 # K_prev > N
    assert sparse(lib, shape(), K_prev=64, I_prev=None) == -1      # implicit list needs K_prev == N
    assert sparse(lib, shape(win=0, H=64, W=64), K_prev=1025, K_l=5) == -2
    assert sparse(lib, shape(), outs=(None, FAKE, FAKE)) == -1
    assert sparse(lib, shape(), outs=(FAKE, None, FAKE)) == -1
    assert sparse(lib, shape(), outs=(FAKE, FAKE, None)) == -1


def test_dense_validation(lib):
    assert dense(lib, None) == -1
    assert dense(lib, shape(win=0)) == -2
    assert dense(lib, shape(d=8)) == -2
    assert dense(lib, shape(), K1=0) == -1
    assert dense(lib, shape(), K1=1025) == -1
    assert dense(lib, shape(), O=None) == -1
    assert dense(lib, shape(), K1=100) == -1                       # K1 < N needs I and A
    assert dense(lib, shape(), K1=100, I=FAKE, A=FAKE, lse=FAKE) == -2   # no log-normaliser when K1 < N
    assert dense(lib, shape(), K1=100, I=FAKE) == -1
    assert dense(lib, shape(win=6, H=12, W=12), K1=36) == -2       # K1 == N needs win % 4 == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pfa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pfa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        pfa.load()


def test_plain_c_client(lib, tmp_path):
    # the header is plain C99 and the library links into a C program
    import subprocess
    src = os.path.join(ROOT, "tests", "c", "abi_check.c")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(pfa._LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                           src, "-o", exe, "-L", libdir, "-lpfa", "-Wl,-rpath," + libdir])
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout


def test_first_two_layers_validation(lib):
    def fused(s, shift1=0, shift2=16, K2=256, outs=(FAKE, FAKE, FAKE, FAKE)):
        return lib.pfa_first_two_layers(ctypes.byref(s) if s is not None else None, shift1, shift2, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, K2, None, *outs, None)
    bf = dict(dtype=1)
    assert fused(None) == -1
    assert fused(shape(shift=16, **bf)) == -1                     # shifts go in shift1/shift2
    assert fused(shape(**bf), shift1=32) == -1
    assert fused(shape(**bf), shift2=-1) == -1
    assert fused(shape(**bf), K2=0) == -1
    assert fused(shape(**bf), K2=1025) == -1
    assert fused(shape(**bf), outs=(None, FAKE, FAKE, FAKE)) == -1
    assert fused(shape(**bf), outs=(FAKE, FAKE, FAKE, None)) == -1
    assert fused(shape()) == -2                                   # fp32, d = 32: K1 and K2 exceed LDS together
    assert fused(shape(win=16, H=32, W=32, **bf)) == -2           # N != 1024
    assert fused(shape(win=0, H=32, W=32, **bf)) == -2            # global mode


def test_backward_validation(lib):
    ws_full = 1 * 1 * 1024 * (64 + 1) * 4

    def bwd(s, K_prev=256, K_l=64, I_prev=FAKE, A_prev=FAKE, dA_prev=FAKE, ws=FAKE, ws_bytes=ws_full,
            grads=(FAKE, FAKE, FAKE), dO=FAKE):
        return lib.pfa_sparse_layer_backward(ctypes.byref(s) if s is not None else None, FAKE, FAKE, FAKE, I_prev,
                                             A_prev, K_prev, K_l, FAKE, FAKE, dO, None, *grads, dA_prev, ws,
                                             ws_bytes, None)
    assert bwd(None) == -1
    assert bwd(shape(win=0, H=128, W=128), K_prev=64, K_l=16, ws_bytes=1 << 30) == -2   # global: dA_prev <= 8192 tokens
    assert bwd(shape(d=8)) == -2
    assert bwd(shape(), K_l=0) == -1
    assert bwd(shape(), K_l=300, K_prev=256) == -1               # K_l > K_prev
    assert bwd(shape(), K_prev=512, I_prev=None) == -1           # implicit list needs K_prev == N
    assert bwd(shape(), A_prev=None) == -1                       # dA_prev needs A_prev
    assert bwd(shape(), ws=None) == -1
    assert bwd(shape(), ws_bytes=ws_full - 4) == -1              # workspace too small
    assert bwd(shape(), dO=None) == -1
    assert bwd(shape(), grads=(FAKE, None, FAKE)) == -1
    assert bwd(shape(), K_prev=1024, K_l=512, I_prev=None, ws_bytes=1 << 30) == -2   # K_l > 256
    assert lib.pfa_sparse_layer_backward_workspace(ctypes.byref(shape()), 64) == ws_full
    assert lib.pfa_sparse_layer_backward_workspace(ctypes.byref(shape(B=2, heads=3, H=64, W=32)), 16) == \
        2 * 3 * 2 * 1024 * (16 + 1) * 4   # g per kept pair, one flag per row
    assert lib.pfa_sparse_layer_backward_workspace(ctypes.byref(shape()), 0) == -1
    assert lib.pfa_sparse_layer_backward_workspace(ctypes.byref(shape(d=8)), 16) == -2


def test_backward_rpb_validation(lib):
    nrel = 63 * 63
    ws_full = 1 * 1 * 1024 * (64 + 1) * 4 + nrel * 4

    def bwd(s, bias=FAKE, dbias=FAKE, ws_bytes=ws_full):
        return lib.pfa_sparse_layer_backward_rpb(ctypes.byref(s), FAKE, FAKE, FAKE, bias, FAKE, FAKE, 256, 64, FAKE,
                                                 FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, dbias, FAKE, ws_bytes,
                                                 None)
    assert bwd(shape(), bias=None) == -1                          # dbias needs the bias
    assert bwd(shape(), ws_bytes=ws_full - 4) == -1               # no room for the per-window-head tables
    assert bwd(shape(win=0)) == -2                                # no bias in global mode
    assert lib.pfa_sparse_layer_backward_rpb_workspace(ctypes.byref(shape(win=0)), 64) == -2
    assert lib.pfa_sparse_layer_backward_rpb_workspace(ctypes.byref(shape()), 64) == ws_full
    assert lib.pfa_sparse_layer_backward_rpb_workspace(ctypes.byref(shape(B=2, heads=3, H=64, W=32, win=16)),
                                                       16) == 2 * 3 * 8 * (256 * 17 * 4 + 31 * 31 * 4)

    def db(s, bias=FAKE, dbias=FAKE, ws_bytes=1 << 30):
        return lib.pfa_dense_layer_backward_rpb(ctypes.byref(s), FAKE, FAKE, FAKE, bias, FAKE, FAKE, None, FAKE,
                                                FAKE, FAKE, dbias, FAKE, ws_bytes, None)
    dws = 1024 * 4 + 64 * 32 * 64 * 4 + nrel * 4                  # D_i, per-wave rows, one table
    assert lib.pfa_dense_layer_backward_rpb_workspace(ctypes.byref(shape())) == dws
    assert lib.pfa_dense_layer_backward_rpb_workspace(ctypes.byref(shape(win=0))) == -2
    assert db(shape(), bias=None) == -1
    assert db(shape(), ws_bytes=dws - 4) == -1
    assert db(shape(win=8, H=16, W=16)) == -2                     # a bias needs win % 16 == 0


def test_first_two_layers_backward_validation(lib):
    ws = 2 * 1024 * 256 * 4 + 1024 * 1024 * 4 + 1024 * 257 * 4 + 1024 * 4   # kept A^1, dA^1; dense dA^1; the passes

    def fb(s, shifts=(0, 16), K2=256, ptrs=(FAKE,) * 6, ws_ptr=FAKE, ws_bytes=ws):
        return lib.pfa_first_two_layers_backward(ctypes.byref(s), shifts[0], shifts[1], *([FAKE] * 6), K2, FAKE,
                                                 FAKE, FAKE, FAKE, FAKE, None, *ptrs, ws_ptr, ws_bytes, None)
    assert lib.pfa_first_two_layers_backward_workspace(ctypes.byref(shape()), 256) == ws
    assert lib.pfa_first_two_layers_backward_workspace(ctypes.byref(shape(win=0)), 256) == -2
    assert lib.pfa_first_two_layers_backward_workspace(ctypes.byref(shape()), 0) == -1
    assert fb(shape(shift=16)) == -1                              # shifts come as arguments
    assert fb(shape(), shifts=(0, 32)) == -1
    assert fb(shape(), K2=0) == -1
    assert fb(shape(), ptrs=(FAKE, FAKE, None, FAKE, FAKE, FAKE)) == -1
    assert fb(shape(), ws_bytes=ws - 4) == -1
    assert fb(shape(), ws_ptr=None) == -1
    assert fb(shape(win=0)) == -2
    assert fb(shape(), K2=512, ws_bytes=1 << 30) == -2           # K2 > 256
    assert fb(shape(win=12, H=24, W=24), shifts=(0, 6), K2=64, ws_bytes=1 << 30) == -2   # win % 8 != 0


def test_iet_validation(lib):
    def prop(B=1, N=4096, k=64, n_maps=6, k1=22, k2=12, ptrs=(FAKE, FAKE, FAKE, FAKE), ws=FAKE,
             ws_bytes=4096 * 34 * 4):
        return lib.pfa_iet_propagate(B, N, k, n_maps, ptrs[0], ptrs[1], k1, k2, ptrs[2], ptrs[3], ws, ws_bytes,
                                     None)
    assert prop(B=0) == -1
    assert prop(N=0) == -1
    assert prop(n_maps=0) == -1
    assert prop(k1=10, k2=12) == -1                              # k2 > k1
    assert prop(k=16) == -1                                      # k1 > k
    assert prop(k2=0) == -1
    assert prop(ptrs=(None, FAKE, FAKE, FAKE)) == -1
    assert prop(ptrs=(FAKE, FAKE, FAKE, None)) == -1
    assert prop(ws=None) == -1
    assert prop(ws_bytes=4096 * 34 * 4 - 4) == -1
    assert prop(k=65, ws_bytes=1 << 20) == -2
    assert prop(N=65537, ws_bytes=1 << 30) == -2
    assert lib.pfa_iet_propagate_workspace(2, 4096, 22, 12) == 2 * 4096 * 34 * 4
    assert lib.pfa_iet_propagate_workspace(1, 0, 22, 12) == -1


def test_rpb_validation(lib):
    def sp(s, bias=FAKE, K_prev=64, K_l=16):
        return lib.pfa_sparse_layer_rpb(ctypes.byref(s), FAKE, FAKE, FAKE, bias, FAKE, 0, FAKE, K_prev, K_l,
                                        FAKE, FAKE, FAKE, None)

    def de(s, bias=FAKE, K1=1024):
        return lib.pfa_dense_layer_rpb(ctypes.byref(s), FAKE, FAKE, FAKE, bias, K1, None, None, None, FAKE, None)
    assert sp(shape(win=0, H=64, W=64)) == -2                   # no bias in global mode
    assert sp(shape(), K_l=0) == -1
    assert de(shape(win=12, H=24, W=24), K1=144) == -2          # dense with a bias needs win % 16 == 0
    assert de(shape(d=8)) == -2
    assert de(shape(), K1=0) == -1


def test_dense_backward_validation(lib):
    def db(s, bias=None, ptr=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return lib.pfa_dense_layer_backward(ctypes.byref(s), FAKE, FAKE, FAKE, bias, ptr, FAKE, None, FAKE, FAKE, FAKE,
                                            ws, ws_bytes, None)
    assert db(shape(win=0, H=32, W=32)) == -2
    assert db(shape(win=12, H=24, W=24)) == -2                  # win % 8 != 0
    assert db(shape(win=8, H=16, W=16), bias=FAKE) == -2        # a bias needs win % 16 == 0
    assert db(shape(), ptr=None) == -1                          # lse required
    assert db(shape(), ws=None) == -1
    assert db(shape(), ws_bytes=1024 * 4 - 4) == -1
    assert db(shape(d=8)) == -2
    assert lib.pfa_dense_layer_backward_workspace(ctypes.byref(shape(B=2, heads=3))) == 2 * 3 * 1024 * 4


def test_noalloc_dense_backward_validation(lib):
    # The no-allocation entry point rejects, before any HIP call, what its static
    # scratch array cannot hold: 4096 windows of 32x32 (4194304 query slots) fit,
    # one more row of windows does not. NULL and shape errors as the workspace form.
    def call(s, q=FAKE):
        return lib.pfa_dense_layer_backward_noalloc(ctypes.byref(s), q, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                                                    FAKE, FAKE, None)
    assert call(shape(H=2080, W=2048, d=16)) == -4
    assert call(shape(), q=None) == -1
    assert call(shape(win=0)) == -2
    assert call(shape(win=12, H=24, W=24)) == -2                  # win % 8 != 0
    assert lib.pfa_strerror(-4).startswith(b"problem larger than the static scratch")
