"""Thin Python binding of libpfa.so (ctypes): argument marshalling only.

Every step of a layer runs in the HIP kernels behind the C ABI declared in
``include/pfa.h``; this module allocates output tensors with torch, passes raw
device pointers and the current HIP stream, and turns error codes into
exceptions. There is no fallback: without the built library every call raises.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpfa.so")
_lib = None

PFA_F32, PFA_BF16 = 0, 1


class PfaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "heads", "H", "W", "d", "win", "shift", "dtype")]


class PfaError(RuntimeError):
    def __init__(self, fn, code):
        msg = load().pfa_strerror(code).decode()
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


def load():
    """Load libpfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m sparse_progressive_window_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.pfa_dense_layer.argtypes = [ctypes.POINTER(PfaShape), P, P, P, i32, P, P, P, P, P]
        lib.pfa_dense_layer.restype = ctypes.c_int
        lib.pfa_sparse_layer.argtypes = [ctypes.POINTER(PfaShape), P, P, P, P, i32, P, i32, i32, P, P, P, P]
        lib.pfa_sparse_layer.restype = ctypes.c_int
        lib.pfa_dense_layer_rpb.argtypes = [ctypes.POINTER(PfaShape), P, P, P, P, i32, P, P, P, P, P]
        lib.pfa_dense_layer_rpb.restype = ctypes.c_int
        lib.pfa_sparse_layer_rpb.argtypes = [ctypes.POINTER(PfaShape), P, P, P, P, P, i32, P, i32, i32, P, P, P, P]
        lib.pfa_sparse_layer_rpb.restype = ctypes.c_int
        lib.pfa_first_two_layers.argtypes = [ctypes.POINTER(PfaShape), i32, i32, P, P, P, P, P, P, i32, P, P, P, P,
                                             P, P]
        lib.pfa_first_two_layers.restype = ctypes.c_int
        lib.pfa_sparse_layer_backward.argtypes = ([ctypes.POINTER(PfaShape), P, P, P, P, P, i32, i32]
                                                  + [P] * 9 + [ctypes.c_int64, P])
        lib.pfa_sparse_layer_backward.restype = ctypes.c_int
        lib.pfa_sparse_layer_backward_workspace.argtypes = [ctypes.POINTER(PfaShape), i32]
        lib.pfa_sparse_layer_backward_workspace.restype = ctypes.c_int64
        lib.pfa_dense_layer_backward.argtypes = [ctypes.POINTER(PfaShape)] + [P] * 11 + [ctypes.c_int64, P]
        lib.pfa_dense_layer_backward.restype = ctypes.c_int
        lib.pfa_dense_layer_backward_noalloc.argtypes = [ctypes.POINTER(PfaShape)] + [P] * 11
        lib.pfa_dense_layer_backward_noalloc.restype = ctypes.c_int
        lib.pfa_dense_layer_backward_workspace.argtypes = [ctypes.POINTER(PfaShape)]
        lib.pfa_dense_layer_backward_workspace.restype = ctypes.c_int64
        lib.pfa_sparse_layer_backward_rpb.argtypes = ([ctypes.POINTER(PfaShape), P, P, P, P, P, P, i32, i32]
                                                      + [P] * 10 + [ctypes.c_int64, P])
        lib.pfa_sparse_layer_backward_rpb.restype = ctypes.c_int
        lib.pfa_sparse_layer_backward_rpb_workspace.argtypes = [ctypes.POINTER(PfaShape), i32]
        lib.pfa_sparse_layer_backward_rpb_workspace.restype = ctypes.c_int64
        lib.pfa_dense_layer_backward_rpb.argtypes = [ctypes.POINTER(PfaShape)] + [P] * 12 + [ctypes.c_int64, P]
        lib.pfa_dense_layer_backward_rpb.restype = ctypes.c_int
        lib.pfa_dense_layer_backward_rpb_workspace.argtypes = [ctypes.POINTER(PfaShape)]
        lib.pfa_dense_layer_backward_rpb_workspace.restype = ctypes.c_int64
        lib.pfa_first_two_layers_backward.argtypes = ([ctypes.POINTER(PfaShape), i32, i32] + [P] * 6 + [i32]
                                                      + [P] * 13 + [ctypes.c_int64, P])
        lib.pfa_first_two_layers_backward.restype = ctypes.c_int
        lib.pfa_first_two_layers_backward_workspace.argtypes = [ctypes.POINTER(PfaShape), i32]
        lib.pfa_first_two_layers_backward_workspace.restype = ctypes.c_int64
        lib.pfa_iet_propagate.argtypes = [i32, i32, i32, i32, P, P, i32, i32, P, P, P, ctypes.c_int64, P]
        lib.pfa_iet_propagate.restype = ctypes.c_int
        lib.pfa_iet_propagate_workspace.argtypes = [i32, i32, i32, i32]
        lib.pfa_iet_propagate_workspace.restype = ctypes.c_int64
        lib.pfa_strerror.argtypes = [ctypes.c_int]
        lib.pfa_strerror.restype = ctypes.c_char_p
        lib.pfa_version.restype = ctypes.c_int
        lib.pfa_timing_enable.argtypes = [i32]
        lib.pfa_timing_enable.restype = ctypes.c_int
        lib.pfa_timing_count.restype = i32
        lib.pfa_timing_read.argtypes = [P, P, i32, P, P]
        lib.pfa_timing_read.restype = ctypes.c_int
        lib.pfa_kernel_name.argtypes = [i32]
        lib.pfa_kernel_name.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def version() -> int:
    return load().pfa_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PFA_F32
    if t.dtype == torch.bfloat16:
        return PFA_BF16
    raise TypeError(f"Q/K/V must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_qkv(Q, K, V):
    for t in (Q, K, V):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 5:
            raise ValueError("Q, K, V must be contiguous 5-d [B, heads, H, W, d] device tensors")
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError("Q, K, V must share shape and dtype")


def make_shape(Q: torch.Tensor, win: int, shift: int) -> PfaShape:
    B, heads, H, W, d = Q.shape
    return PfaShape(B, heads, H, W, d, win, shift, _dtype_code(Q))


def _prod(xs):
    r = 1
    for x in xs:
        r *= x
    return r


def _geometry(Q, win):
    B, heads, H, W, _ = Q.shape
    if win:
        return (B, heads, (H // win) * (W // win)), win * win
    return (B, heads), H * W


def _expect(t, numel, dtype, name):
    """The C ABI sees raw pointers only: check every buffer's size here."""
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor with {numel} elements, got "
                         f"{tuple(t.shape)} {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_bias(bias, Q, win):
    if bias is None:
        return
    if not win:
        raise ValueError("a relative position bias needs window mode")
    _expect(bias, Q.shape[1] * (2 * win - 1) ** 2, torch.float32, "bias")


def dense_layer(Q, K, V, K1=None, *, win, shift=0, want_A=True, want_I=False, out=None, lse_out=None, bias=None):
    """First (dense) layer. Returns (I, A, O); I and A are None when not requested
    (K1 == N) and always returned when K1 < N. ``out`` = optional preallocated
    (I or None, A or None, O). ``lse_out``: optional [B, heads, nwin, N] fp32
    tensor filled with each row's log softmax denominator (K1 == N only).
    ``bias``: optional [heads, (2 win - 1)^2] fp32 relative position bias."""
    _check_qkv(Q, K, V)
    lead, N = _geometry(Q, win)
    K1 = N if K1 is None else K1
    dev = Q.device
    if out is not None:
        I, A, O = out
    else:
        if K1 < N:
            want_A = want_I = True
        O = torch.empty(Q.shape, dtype=torch.float32, device=dev)
        A = torch.empty(lead + (N, K1), dtype=torch.float32, device=dev) if want_A else None
        I = torch.empty(lead + (N, K1), dtype=torch.int32, device=dev) if want_I else None
    rows = _prod(lead) * N
    _expect(I, rows * K1, torch.int32, "I_out")
    _expect(A, rows * K1, torch.float32, "A_out")
    _expect(O, Q.numel(), torch.float32, "O_out")
    _expect(lse_out, rows, torch.float32, "lse_out")
    _check_bias(bias, Q, win)
    shape = make_shape(Q, win, shift)
    rc = load().pfa_dense_layer_rpb(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(bias), K1, _ptr(I), _ptr(A),
                                    _ptr(lse_out), _ptr(O), _stream())
    if rc != 0:
        raise PfaError("pfa_dense_layer", rc)
    return I, A, O


def sparse_layer(Q, K, V, I_prev, A_prev, K_l, *, win, shift=0, i_shared=False, K_prev=None, out=None, bias=None):
    """Sparse layer: scores only over I_prev, Hadamard with A_prev, top-K_l.
    I_prev None = all slots (K_prev = N); A_prev None = all ones.
    ``out`` = optional preallocated (I, A, O); ``bias`` = optional [heads,
    (2 win - 1)^2] fp32 relative position bias. Returns (I, A, O)."""
    _check_qkv(Q, K, V)
    lead, N = _geometry(Q, win)
    if I_prev is not None:
        K_prev = I_prev.shape[-1]
    elif K_prev is None:
        K_prev = N
    dev = Q.device
    if out is None:
        I = torch.empty(lead + (N, K_l), dtype=torch.int32, device=dev)
        A = torch.empty(lead + (N, K_l), dtype=torch.float32, device=dev)
        O = torch.empty(Q.shape, dtype=torch.float32, device=dev)
    else:
        I, A, O = out
    rows = _prod(lead) * N
    hI = 1 if i_shared else Q.shape[1]
    _expect(I_prev, rows // Q.shape[1] * hI * K_prev, torch.int32, "I_prev")
    _expect(A_prev, rows * K_prev, torch.float32, "A_prev")
    _expect(I, rows * K_l, torch.int32, "I_out")
    _expect(A, rows * K_l, torch.float32, "A_out")
    _expect(O, Q.numel(), torch.float32, "O_out")
    _check_bias(bias, Q, win)
    shape = make_shape(Q, win, shift)
    rc = load().pfa_sparse_layer_rpb(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(bias), _ptr(I_prev),
                                     int(bool(i_shared)), _ptr(A_prev), K_prev, K_l, _ptr(I), _ptr(A),
                                     _ptr(O), _stream())
    if rc != 0:
        raise PfaError("pfa_sparse_layer", rc)
    return I, A, O


def first_two_layers(Q1, K1, V1, Q2, K2, V2, K2_keep, *, win, shift1=0, shift2=0, out=None, lse_out=None):
    """Layers 1 and 2 of a chain without materialising layer 1's map. Returns
    (O1, I2, A2, O2); ``out`` = optional preallocated (O1, I2, A2, O2);
    ``lse_out`` = optional [B, heads, nwin, N] fp32 tensor for layer 1's log
    softmax denominators."""
    _check_qkv(Q1, K1, V1)
    _check_qkv(Q2, K2, V2)
    if Q2.shape != Q1.shape or Q2.dtype != Q1.dtype:
        raise ValueError("both layers' Q/K/V must share shape and dtype")
    lead, N = _geometry(Q1, win)
    dev = Q1.device
    if out is None:
        O1 = torch.empty(Q1.shape, dtype=torch.float32, device=dev)
        I2 = torch.empty(lead + (N, K2_keep), dtype=torch.int32, device=dev)
        A2 = torch.empty(lead + (N, K2_keep), dtype=torch.float32, device=dev)
        O2 = torch.empty(Q1.shape, dtype=torch.float32, device=dev)
    else:
        O1, I2, A2, O2 = out
    rows = _prod(lead) * N
    _expect(O1, Q1.numel(), torch.float32, "O1_out")
    _expect(I2, rows * K2_keep, torch.int32, "I2_out")
    _expect(A2, rows * K2_keep, torch.float32, "A2_out")
    _expect(O2, Q1.numel(), torch.float32, "O2_out")
    _expect(lse_out, rows, torch.float32, "lse1_out")
    shape = make_shape(Q1, win, 0)
    rc = load().pfa_first_two_layers(ctypes.byref(shape), shift1, shift2, _ptr(Q1), _ptr(K1), _ptr(V1), _ptr(Q2),
                                     _ptr(K2), _ptr(V2), K2_keep, _ptr(lse_out), _ptr(O1), _ptr(I2), _ptr(A2),
                                     _ptr(O2), _stream())
    if rc != 0:
        raise PfaError("pfa_first_two_layers", rc)
    return O1, I2, A2, O2


def first_two_layers_backward(Q1, K1, V1, Q2, K2, V2, lse1, I2, A2, dO1, dO2, dA2=None, *, win, shift1=0,
                              shift2=0, out=None, workspace=None):
    """Backward of first_two_layers: lse1, I2, A2 = the forward's outputs (lse1
    [B, heads, nwin, N]); dO1, dO2 fp32; dA2 = gradient of A2 or None. Returns
    (dQ1, dK1, dV1, dQ2, dK2, dV2) in fp32."""
    _check_qkv(Q1, K1, V1)
    _check_qkv(Q2, K2, V2)
    if Q1.shape != Q2.shape or Q1.dtype != Q2.dtype:
        raise ValueError("both layers' inputs must share shape and dtype")
    lead, N = _geometry(Q1, win)
    K2_keep = I2.shape[-1]
    rows = _prod(lead) * N
    _expect(lse1, rows, torch.float32, "lse1")
    _expect(I2, rows * K2_keep, torch.int32, "I2")
    _expect(A2, rows * K2_keep, torch.float32, "A2")
    _expect(dO1, Q1.numel(), torch.float32, "dO1")
    _expect(dO2, Q1.numel(), torch.float32, "dO2")
    _expect(dA2, rows * K2_keep, torch.float32, "dA2")
    dev = Q1.device
    outs = out if out is not None else tuple(torch.empty(Q1.shape, dtype=torch.float32, device=dev)
                                             for _ in range(6))
    for t, n in zip(outs, ("dQ1", "dK1", "dV1", "dQ2", "dK2", "dV2")):
        _expect(t, Q1.numel(), torch.float32, n)
    shape = make_shape(Q1, win, 0)
    need = int(load().pfa_first_two_layers_backward_workspace(ctypes.byref(shape), int(K2_keep)))
    if need < 0:
        raise PfaError("pfa_first_two_layers_backward_workspace", need)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device tensor of at least {need} bytes")
    rc = load().pfa_first_two_layers_backward(ctypes.byref(shape), int(shift1), int(shift2), _ptr(Q1), _ptr(K1),
                                              _ptr(V1), _ptr(Q2), _ptr(K2), _ptr(V2), int(K2_keep), _ptr(lse1),
                                              _ptr(I2), _ptr(A2), _ptr(dO1), _ptr(dO2), _ptr(dA2),
                                              *(_ptr(t) for t in outs), _ptr(workspace),
                                              workspace.numel() * workspace.element_size(), _stream())
    if rc != 0:
        raise PfaError("pfa_first_two_layers_backward", rc)
    return tuple(outs)


def sparse_layer_backward(Q, K, V, I_prev, A_prev, I_l, A_l, dO, dA_l=None, *, win, shift=0, K_prev=None,
                          want_dA_prev=True, out=None, workspace=None):
    """Backward pass of a window-mode sparse layer with its kept sets fixed.

    Q, K, V, I_prev (None = every slot), A_prev: the forward call's inputs;
    I_l, A_l: its outputs; dO: fp32 gradient of O; dA_l: fp32 gradient of A^l or
    None. Returns (dQ, dK, dV, dA_prev) in fp32; dA_prev is None when not wanted
    (or A_prev is None). ``out`` = optional preallocated (dQ, dK, dV, dA_prev or
    None); ``workspace`` = optional uint8 device tensor of at least
    ``backward_workspace_bytes`` bytes."""
    return _sparse_backward(Q, K, V, I_prev, A_prev, I_l, A_l, dO, dA_l, win, shift, K_prev, want_dA_prev, out,
                            workspace, None, False)[:4]


def sparse_layer_backward_rpb(Q, K, V, bias, I_prev, A_prev, I_l, A_l, dO, dA_l=None, *, win, shift=0,
                              K_prev=None, want_dA_prev=True, want_dbias=True, out=None, workspace=None):
    """sparse_layer_backward of a layer computed with the relative position bias
    ``bias`` [heads, (2 win - 1)^2] (fp32, device). Returns (dQ, dK, dV, dA_prev,
    dbias); dbias [heads, (2 win - 1)^2] fp32, or None when not wanted."""
    return _sparse_backward(Q, K, V, I_prev, A_prev, I_l, A_l, dO, dA_l, win, shift, K_prev, want_dA_prev, out,
                            workspace, bias, want_dbias)


def _sparse_backward(Q, K, V, I_prev, A_prev, I_l, A_l, dO, dA_l, win, shift, K_prev, want_dA_prev, out,
                     workspace, bias, want_dbias):
    _check_qkv(Q, K, V)
    lead, N = _geometry(Q, win)
    K_l = I_l.shape[-1]
    if I_prev is not None:
        K_prev = I_prev.shape[-1]
    elif K_prev is None:
        K_prev = N
    dev = Q.device
    want = want_dA_prev and A_prev is not None
    if out is None:
        dQ, dK, dV = (torch.empty(Q.shape, dtype=torch.float32, device=dev) for _ in range(3))
        dAp = torch.empty(lead + (N, K_prev), dtype=torch.float32, device=dev) if want else None
    else:
        dQ, dK, dV, dAp = out
    rows = _prod(lead) * N
    _expect(I_prev, rows * K_prev, torch.int32, "I_prev")
    _expect(A_prev, rows * K_prev, torch.float32, "A_prev")
    _expect(I_l, rows * K_l, torch.int32, "I_l")
    _expect(A_l, rows * K_l, torch.float32, "A_l")
    _expect(dO, Q.numel(), torch.float32, "dO")
    _expect(dA_l, rows * K_l, torch.float32, "dA_l")
    for t, n in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _expect(t, Q.numel(), torch.float32, n)
    _expect(dAp, rows * K_prev, torch.float32, "dA_prev")
    _check_bias(bias, Q, win)
    dbias = None
    if want_dbias:
        if bias is None:
            raise ValueError("the bias gradient needs the forward's bias")
        dbias = torch.empty(bias.shape, dtype=torch.float32, device=dev)
    shape = make_shape(Q, win, shift)
    if dbias is not None:
        need = int(load().pfa_sparse_layer_backward_rpb_workspace(ctypes.byref(shape), int(K_l)))
        if need < 0:
            raise PfaError("pfa_sparse_layer_backward_rpb_workspace", need)
    else:
        need = backward_workspace_bytes(Q, K_l, win=win, shift=shift)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device tensor of at least {need} bytes")
    nbytes = workspace.numel() * workspace.element_size()
    if bias is None:
        rc = load().pfa_sparse_layer_backward(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(I_prev),
                                              _ptr(A_prev), K_prev, K_l, _ptr(I_l), _ptr(A_l), _ptr(dO), _ptr(dA_l),
                                              _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dAp), _ptr(workspace), nbytes,
                                              _stream())
        if rc != 0:
            raise PfaError("pfa_sparse_layer_backward", rc)
    else:
        rc = load().pfa_sparse_layer_backward_rpb(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(bias),
                                                  _ptr(I_prev), _ptr(A_prev), K_prev, K_l, _ptr(I_l), _ptr(A_l),
                                                  _ptr(dO), _ptr(dA_l), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dAp),
                                                  _ptr(dbias), _ptr(workspace), nbytes, _stream())
        if rc != 0:
            raise PfaError("pfa_sparse_layer_backward_rpb", rc)
    return dQ, dK, dV, dAp, dbias


def dense_layer_backward(Q, K, V, lse, dO, dA=None, *, win, shift=0, bias=None, out=None, workspace=None):
    """Backward of the dense first layer: lse = the forward's lse_out
    [B, heads, nwin, N]; dO fp32; dA = gradient of A^1 [B, heads, nwin, N, N]
    or None. Returns (dQ, dK, dV) in fp32."""
    _check_qkv(Q, K, V)
    lead, N = _geometry(Q, win)
    dev = Q.device
    if out is None:
        dQ, dK, dV = (torch.empty(Q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    else:
        dQ, dK, dV = out
    rows = _prod(lead) * N
    _expect(lse, rows, torch.float32, "lse")
    _expect(dO, Q.numel(), torch.float32, "dO")
    _expect(dA, rows * N, torch.float32, "dA")
    for t, n in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _expect(t, Q.numel(), torch.float32, n)
    _check_bias(bias, Q, win)
    shape = make_shape(Q, win, shift)
    need = int(load().pfa_dense_layer_backward_workspace(ctypes.byref(shape)))
    if need < 0:
        raise PfaError("pfa_dense_layer_backward_workspace", need)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device tensor of at least {need} bytes")
    rc = load().pfa_dense_layer_backward(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(bias), _ptr(lse),
                                         _ptr(dO), _ptr(dA), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream())
    if rc != 0:
        raise PfaError("pfa_dense_layer_backward", rc)
    return dQ, dK, dV


def dense_layer_backward_rpb(Q, K, V, bias, lse, dO, dA=None, *, win, shift=0, out=None, workspace=None):
    """dense_layer_backward of a layer computed with the relative position bias
    ``bias`` [heads, (2 win - 1)^2], with its gradient: returns (dQ, dK, dV, dbias)."""
    _check_qkv(Q, K, V)
    lead, N = _geometry(Q, win)
    dev = Q.device
    if out is None:
        dQ, dK, dV = (torch.empty(Q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    else:
        dQ, dK, dV = out
    rows = _prod(lead) * N
    _expect(lse, rows, torch.float32, "lse")
    _expect(dO, Q.numel(), torch.float32, "dO")
    _expect(dA, rows * N, torch.float32, "dA")
    for t, n in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _expect(t, Q.numel(), torch.float32, n)
    if bias is None:
        raise ValueError("the bias gradient needs the forward's bias")
    _check_bias(bias, Q, win)
    dbias = torch.empty(bias.shape, dtype=torch.float32, device=dev)
    shape = make_shape(Q, win, shift)
    need = int(load().pfa_dense_layer_backward_rpb_workspace(ctypes.byref(shape)))
    if need < 0:
        raise PfaError("pfa_dense_layer_backward_rpb_workspace", need)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device tensor of at least {need} bytes")
    rc = load().pfa_dense_layer_backward_rpb(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(bias), _ptr(lse),
                                             _ptr(dO), _ptr(dA), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dbias),
                                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if rc != 0:
        raise PfaError("pfa_dense_layer_backward_rpb", rc)
    return dQ, dK, dV, dbias


def dense_layer_backward_noalloc(Q, K, V, lse, dO, dA=None, *, win, shift=0, bias=None, out=None):
    """dense_layer_backward through the entry point that allocates nothing (its
    scratch memory is the library's static device array). ``out`` = optional
    preallocated (dQ, dK, dV); when given, this call allocates nothing either."""
    _check_qkv(Q, K, V)
    lead, N = _geometry(Q, win)
    dev = Q.device
    if out is None:
        dQ, dK, dV = (torch.empty(Q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    else:
        dQ, dK, dV = out
    rows = _prod(lead) * N
    _expect(lse, rows, torch.float32, "lse")
    _expect(dO, Q.numel(), torch.float32, "dO")
    _expect(dA, rows * N, torch.float32, "dA")
    for t, n in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _expect(t, Q.numel(), torch.float32, n)
    _check_bias(bias, Q, win)
    shape = make_shape(Q, win, shift)
    rc = load().pfa_dense_layer_backward_noalloc(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(bias),
                                                 _ptr(lse), _ptr(dO), _ptr(dA), _ptr(dQ), _ptr(dK), _ptr(dV),
                                                 _stream())
    if rc != 0:
        raise PfaError("pfa_dense_layer_backward_noalloc", rc)
    return dQ, dK, dV


def first_two_layers_backward_workspace_bytes(Q1, K2_keep, *, win) -> int:
    shape = make_shape(Q1, win, 0)
    n = int(load().pfa_first_two_layers_backward_workspace(ctypes.byref(shape), int(K2_keep)))
    if n < 0:
        raise PfaError("pfa_first_two_layers_backward_workspace", n)
    return n


def backward_workspace_bytes(Q, K_l, *, win, shift=0) -> int:
    shape = make_shape(Q, win, shift)
    n = int(load().pfa_sparse_layer_backward_workspace(ctypes.byref(shape), int(K_l)))
    if n < 0:
        raise PfaError("pfa_sparse_layer_backward_workspace", n)
    return n


def iet_propagate(I, A, k1, k2, *, out=None, workspace=None):
    """Propagation and sparsification of an index matrix: I [B, N, k] (or [N, k])
    int32, A [B, n_maps, N, k] (or [n_maps, N, k]) fp32. Returns (I_out
    [.., N, k1 + k2*k2] int32 ascending and -1 padded, count [.., N] int32)."""
    squeeze = I.dim() == 2
    if squeeze:
        I, A = I.unsqueeze(0), A.unsqueeze(0)
    if I.dim() != 3 or A.dim() != 4:
        raise ValueError("I must be [B, N, k] and A [B, n_maps, N, k]")
    B, N, k = I.shape
    n_maps = A.shape[1]
    if A.shape != (B, n_maps, N, k):
        raise ValueError(f"A must be [{B}, n_maps, {N}, {k}], got {tuple(A.shape)}")
    width = k1 + k2 * k2
    dev = I.device
    if out is None:
        I_out = torch.empty((B, N, width), dtype=torch.int32, device=dev)
        count = torch.empty((B, N), dtype=torch.int32, device=dev)
    else:
        I_out, count = out
    _expect(I, B * N * k, torch.int32, "I")
    _expect(A, B * n_maps * N * k, torch.float32, "A")
    _expect(I_out, B * N * width, torch.int32, "I_out")
    _expect(count, B * N, torch.int32, "count_out")
    need = int(load().pfa_iet_propagate_workspace(B, N, k1, k2))
    if need < 0:
        raise PfaError("pfa_iet_propagate_workspace", need)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be a device tensor of at least {need} bytes")
    rc = load().pfa_iet_propagate(B, N, k, n_maps, _ptr(I), _ptr(A), k1, k2, _ptr(I_out), _ptr(count),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if rc != 0:
        raise PfaError("pfa_iet_propagate", rc)
    if squeeze:
        return I_out[0], count[0]
    return I_out, count


KERNEL_KINDS = ("dense", "all_candidates", "sparse", "select", "aggregate", "iota", "bwd_rows", "bwd_scatter",
                "iet_rank", "iet_union", "dense_bwd")


def kernel_name(kind: int) -> str:
    return load().pfa_kernel_name(kind).decode()


def timing_enable(capacity: int) -> None:
    """Bracket every kernel the layer calls launch with HIP events on its stream
    (capacity = launches kept until the next read; 0 switches timing off)."""
    rc = load().pfa_timing_enable(int(capacity))
    if rc != 0:
        raise PfaError("pfa_timing_enable", rc)


def timing_count() -> int:
    return int(load().pfa_timing_count())


def timing_read(cap: int = 4096):
    """Wait for the recorded launches; returns ([(kind, ms), ...] in launch order, dropped)."""
    kinds = (ctypes.c_int32 * max(cap, 1))()
    ms = (ctypes.c_float * max(cap, 1))()
    n, dropped = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = load().pfa_timing_read(kinds, ms, int(cap), ctypes.byref(n), ctypes.byref(dropped))
    if rc != 0:
        raise PfaError("pfa_timing_read", rc)
    return [(int(kinds[i]), float(ms[i])) for i in range(n.value)], int(dropped.value)
