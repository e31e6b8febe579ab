"""Thin ctypes binding of libbitlinear.so (declared in include/bitlinear.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the BitLinear path runs in the library's kernels.
There is no fallback: if the library is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libbitlinear.so"

NM_DENSE = (0, 0)
NM_2_4 = (2, 4)
NM_6_8 = (6, 8)

OK, EINVAL, EUNSUPPORTED, ESIZE, EHIP = 0, -1, -2, -3, -4
_STATUS = {OK: "OK", EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", ESIZE: "ESIZE", EHIP: "EHIP"}

# every entry point include/bitlinear.h declares
EXPORTED = (
    "bitlinear_packed_size",
    "bitlinear_pack_weights",
    "bitlinear_pack_weights_masked",
    "bitlinear_quant_act",
    "bitlinear_quant_act_ex",
    "bitlinear_quant_act_multi",
    "bitlinear_quant_act_h4",
    "bitlinear_quant_act_a48",
    "bitlinear_combine_a48",
    "bitlinear_forward_workspace_size",
    "bitlinear_forward",
    "bitlinear_forward_noalloc",
    "bitlinear_forward_grouped",
    "bitlinear_forward_fused",
    "bitlinear_forward_fused_ex",
    "bitlinear_forward_fused_multi",
    "bitlinear_forward_grouped_multi",
    "bitlinear_packed_size_trit24",
    "bitlinear_pack_weights_trit24",
    "bitlinear_forward_trit24_workspace_size",
    "bitlinear_forward_trit24",
    "bitlinear_last_error",
    "bitlinear_last_dispatch",
)


class BitLinearError(RuntimeError):
    def __init__(self, fn, status, message):
        self.status = status
        super().__init__("%s failed: %s (%d): %s" % (fn, _STATUS.get(status, "?"), status, message))


class NM(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("m", ctypes.c_int32)]


class ActTransform(ctypes.Structure):
    _fields_ = [("up", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("eps", ctypes.c_float)]


class Proj(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("w_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("Y", ctypes.c_void_p), ("acc", ctypes.c_void_p)]


class QuantGroup(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("Xq", ctypes.c_void_p),
                ("x_scale", ctypes.c_void_p), ("x_rowsum", ctypes.c_void_p)]


class ActGroup(ctypes.Structure):
    _fields_ = [("Xq", ctypes.c_void_p), ("x_scale", ctypes.c_void_p), ("x_rowsum", ctypes.c_void_p),
                ("K", ctypes.c_int64), ("projs", ctypes.POINTER(Proj)), ("nproj", ctypes.c_int32)]


class InputGroup(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("K", ctypes.c_int64), ("projs", ctypes.POINTER(Proj)),
                ("nproj", ctypes.c_int32), ("x_scale", ctypes.c_void_p)]


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


_lib = None


def load_library():
    """Load libbitlinear.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "libbitlinear.so is not built (%s); run __graft_entry__.build() first -- "
            "there is no fallback implementation" % path)
    lib = ctypes.CDLL(path)
    i64, sz, vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    lib.bitlinear_packed_size.argtypes = [i64, i64, NM, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.bitlinear_pack_weights.argtypes = [vp, i64, i64, NM, vp, sz, vp, vp, sz, vp]
    lib.bitlinear_pack_weights_masked.argtypes = [vp, i64, i64, NM, vp, sz, vp, vp, sz, vp]
    lib.bitlinear_quant_act.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.bitlinear_forward_workspace_size.argtypes = [i64, i64, i64, NM, ctypes.POINTER(sz)]
    lib.bitlinear_forward.argtypes = [vp, vp, vp, vp, vp, NM, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.bitlinear_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, NM, i64, i64, i64, vp, vp, vp]
    lib.bitlinear_forward_grouped.argtypes = [vp, vp, vp, i64, i64, NM, ctypes.POINTER(Proj), ctypes.c_int32, vp]
    lib.bitlinear_forward_fused.argtypes = [vp, i64, i64, NM, ctypes.POINTER(Proj), ctypes.c_int32, vp, vp]
    lib.bitlinear_quant_act_ex.argtypes = [vp, ctypes.POINTER(ActTransform), i64, i64, vp, vp, vp, vp]
    lib.bitlinear_quant_act_h4.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    lib.bitlinear_quant_act_a48.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    lib.bitlinear_combine_a48.argtypes = [vp, i64, i64, vp, vp]
    lib.bitlinear_forward_fused_ex.argtypes = [vp, ctypes.POINTER(ActTransform), i64, i64, NM,
                                               ctypes.POINTER(Proj), ctypes.c_int32, vp, vp]
    lib.bitlinear_quant_act_multi.argtypes = [ctypes.POINTER(QuantGroup), ctypes.c_int32, vp]
    lib.bitlinear_forward_grouped_multi.argtypes = [ctypes.POINTER(ActGroup), ctypes.c_int32, ctypes.c_int64, NM,
                                                    vp]
    lib.bitlinear_forward_fused_multi.argtypes = [ctypes.POINTER(InputGroup), ctypes.c_int32, NM, vp]
    lib.bitlinear_packed_size_trit24.argtypes = [i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.bitlinear_pack_weights_trit24.argtypes = [vp, i64, i64, vp, sz, vp, vp, sz, vp]
    lib.bitlinear_forward_trit24_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(sz)]
    lib.bitlinear_forward_trit24.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    for f in EXPORTED:
        if f not in ("bitlinear_last_error", "bitlinear_last_dispatch"):
            getattr(lib, f).restype = ctypes.c_int
    lib.bitlinear_last_error.restype = ctypes.c_char_p
    lib.bitlinear_last_dispatch.restype = ctypes.c_char_p
    lib.bitlinear_last_error.argtypes = []
    lib.bitlinear_last_dispatch.argtypes = []
    _lib = lib
    return lib


def _check(fn, status):
    if status != OK:
        msg = load_library().bitlinear_last_error()
        raise BitLinearError(fn, status, msg.decode() if msg else "")


def last_dispatch() -> str:
    s = load_library().bitlinear_last_dispatch()
    return s.decode() if s else ""


def _nm(nm):
    n, m = nm
    return NM(int(n), int(m))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, dtype, shape, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def packed_size(N: int, K: int, nm=NM_DENSE):
    """(packed_bytes, workspace_bytes) for an N x K weight matrix."""
    lib = load_library()
    pb, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("bitlinear_packed_size", lib.bitlinear_packed_size(N, K, _nm(nm), ctypes.byref(pb), ctypes.byref(wb)))
    return pb.value, wb.value


def pack_weights(W, nm=NM_DENSE, out=None, w_scale=None, workspace=None, stream=None):
    """Ternarise and pack an N x K fp32 device matrix.  Returns (packed uint8, w_scale fp32[1])."""
    import torch
    _require(W, torch.float32, None, "W")
    N, K = W.shape
    pb, wb = packed_size(N, K, nm)
    if out is None:
        out = torch.empty(pb, dtype=torch.uint8, device=W.device)
    if w_scale is None:
        w_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    if workspace is None and wb:
        workspace = torch.empty(wb, dtype=torch.uint8, device=W.device)
    _require(out, torch.uint8, None, "packed")
    _require(w_scale, torch.float32, (1,), "w_scale")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bitlinear_pack_weights", load_library().bitlinear_pack_weights(
        _ptr(W), N, K, _nm(nm), _ptr(out), out.numel(), _ptr(w_scale), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return out, w_scale


def pack_weights_masked(W, nm, out=None, w_scale=None, workspace=None, stream=None):
    """N:M-masked ternary weights (nm = (2, 4) or (6, 8)) in the dense 2-bit
    layout, for forward() with nm = (0, 0).  Returns (packed uint8, w_scale)."""
    import torch
    _require(W, torch.float32, None, "W")
    N, K = W.shape
    pb, wb = packed_size(N, K, NM_DENSE)
    if out is None:
        out = torch.empty(pb, dtype=torch.uint8, device=W.device)
    if w_scale is None:
        w_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    if workspace is None and wb:
        workspace = torch.empty(wb, dtype=torch.uint8, device=W.device)
    _require(out, torch.uint8, None, "packed")
    _require(w_scale, torch.float32, (1,), "w_scale")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bitlinear_pack_weights_masked", load_library().bitlinear_pack_weights_masked(
        _ptr(W), N, K, _nm(nm), _ptr(out), out.numel(), _ptr(w_scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, w_scale


def packed_size_trit24(N: int, K: int):
    """(packed bytes, pack workspace bytes) of the trit-packed 2:4 layout."""
    pb, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("bitlinear_packed_size_trit24", load_library().bitlinear_packed_size_trit24(
        N, K, ctypes.byref(pb), ctypes.byref(wb)))
    return pb.value, wb.value


def pack_weights_trit24(W, out=None, w_scale=None, workspace=None, stream=None):
    """2:4 ternary weights of an N x K fp32 device matrix, one 6-bit code per
    group of 4 (3*N*K/16 bytes), for forward_trit24().  Returns (packed uint8,
    w_scale fp32[1])."""
    import torch
    _require(W, torch.float32, None, "W")
    N, K = W.shape
    pb, wb = packed_size_trit24(N, K)
    if out is None:
        out = torch.empty(pb, dtype=torch.uint8, device=W.device)
    if w_scale is None:
        w_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    if workspace is None and wb:
        workspace = torch.empty(wb, dtype=torch.uint8, device=W.device)
    _require(out, torch.uint8, None, "packed")
    _require(w_scale, torch.float32, (1,), "w_scale")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bitlinear_pack_weights_trit24", load_library().bitlinear_pack_weights_trit24(
        _ptr(W), N, K, _ptr(out), out.numel(), _ptr(w_scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, w_scale


def forward_trit24_workspace_size(M: int, N: int, K: int) -> int:
    """Device scratch bytes bitlinear_forward_trit24 needs for an M x N x K call."""
    wb = ctypes.c_size_t(0)
    _check("bitlinear_forward_trit24_workspace_size", load_library().bitlinear_forward_trit24_workspace_size(
        M, N, K, ctypes.byref(wb)))
    return wb.value


def forward_trit24(Xq, x_scale, x_rowsum, packed, w_scale, N, Y=None, acc=None, want_acc=False, workspace=None,
                   stream=None):
    """forward() on weights packed by pack_weights_trit24.  Returns Y or (Y, acc)."""
    import torch
    _require(Xq, torch.int8, None, "Xq")
    M, K = Xq.shape
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    _require(packed, torch.uint8, None, "packed")
    _require(w_scale, torch.float32, (1,), "w_scale")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    _require(Y, torch.float32, (M, N), "Y")
    if acc is None and want_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    if acc is not None:
        _require(acc, torch.int32, (M, N), "acc")
    pb, _ = packed_size_trit24(N, K)
    if packed.numel() < pb:
        raise ValueError("packed buffer holds %d bytes, %d needed" % (packed.numel(), pb))
    if workspace is None:
        wb = forward_trit24_workspace_size(M, N, K)
        if wb:
            workspace = torch.empty(wb, dtype=torch.uint8, device=Xq.device)
    if workspace is not None:
        _require(workspace, torch.uint8, None, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("bitlinear_forward_trit24", load_library().bitlinear_forward_trit24(
        _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), _ptr(packed), _ptr(w_scale), M, N, K, _ptr(Y), _ptr(acc),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return (Y, acc) if (want_acc or acc is not None) else Y


def quant_act(X, Xq=None, x_scale=None, x_rowsum=None, stream=None):
    """Per-row absmax int8 quantisation of an M x K fp32 device matrix.

    Returns (Xq int8 M x K, x_scale fp32[M], x_rowsum int32[M]).
    """
    import torch
    _require(X, torch.float32, None, "X")
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_rowsum is None:
        x_rowsum = torch.empty(M, dtype=torch.int32, device=X.device)
    _require(Xq, torch.int8, (M, K), "Xq")
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    _check("bitlinear_quant_act", load_library().bitlinear_quant_act(
        _ptr(X), M, K, _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), _stream(stream)))
    return Xq, x_scale, x_rowsum


def _transform(X, up, gamma, eps):
    """The row transform struct (None when there is none)."""
    import torch
    M, K = X.shape
    if up is not None:
        _require(up, torch.float32, (M, K), "up")
    if gamma is not None:
        _require(gamma, torch.float32, (K,), "gamma")
        if eps is None:
            raise ValueError("eps is required with gamma")
    if up is None and gamma is None:
        return None
    return ActTransform(None if up is None else up.data_ptr(), None if gamma is None else gamma.data_ptr(),
                        0.0 if eps is None else float(eps))


def quant_act_ex(X, up=None, gamma=None, eps=None, Xq=None, x_scale=None, x_rowsum=None, stream=None):
    """quant_act on transformed rows: h = ReLU(X)^2 * up when `up` is given,
    then RMSNorm with weight `gamma` (K) and `eps` when `gamma` is given; the
    codes are taken from h * gamma and 1/rms goes into x_scale."""
    import torch
    _require(X, torch.float32, None, "X")
    M, K = X.shape
    tr = _transform(X, up, gamma, eps)
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_rowsum is None:
        x_rowsum = torch.empty(M, dtype=torch.int32, device=X.device)
    _require(Xq, torch.int8, (M, K), "Xq")
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    _check("bitlinear_quant_act_ex", load_library().bitlinear_quant_act_ex(
        _ptr(X), None if tr is None else ctypes.byref(tr), M, K, _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum),
        _stream(stream)))
    return Xq, x_scale, x_rowsum


def quant_act_h4(X, block, Xq=None, x_scale=None, x_rowsum=None, stream=None):
    """H-BitLinear activations: block Hadamard transform of each row (block a
    power of two dividing K), then 4-bit absmax codes stored one per int8.
    Returns (Xq, x_scale, x_rowsum) for forward()."""
    import torch
    _require(X, torch.float32, None, "X")
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_rowsum is None:
        x_rowsum = torch.empty(M, dtype=torch.int32, device=X.device)
    _require(Xq, torch.int8, (M, K), "Xq")
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    _check("bitlinear_quant_act_h4", load_library().bitlinear_quant_act_h4(
        _ptr(X), M, K, int(block), _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), _stream(stream)))
    return Xq, x_scale, x_rowsum


def forward_workspace_size(M: int, N: int, K: int, nm=NM_DENSE) -> int:
    """Device scratch bytes bitlinear_forward needs for an M x N x K call (often 0)."""
    wb = ctypes.c_size_t(0)
    _check("bitlinear_forward_workspace_size", load_library().bitlinear_forward_workspace_size(
        M, N, K, _nm(nm), ctypes.byref(wb)))
    return wb.value


def quant_act_a48(X, n_outliers, Xq=None, x_scale=None, x_rowsum=None, stream=None):
    """BitNet a4.8 hybrid activations: for each row the n_outliers largest |x|
    at 8 bits, the rest at 4 bits.  Returns (Xq int8 2M x K, x_scale fp32 2M,
    x_rowsum int32 2M): rows 2m / 2m+1 are token m's 8-bit / 4-bit parts."""
    import torch
    _require(X, torch.float32, None, "X")
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty((2 * M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(2 * M, dtype=torch.float32, device=X.device)
    if x_rowsum is None:
        x_rowsum = torch.empty(2 * M, dtype=torch.int32, device=X.device)
    _require(Xq, torch.int8, (2 * M, K), "Xq")
    _require(x_scale, torch.float32, (2 * M,), "x_scale")
    _require(x_rowsum, torch.int32, (2 * M,), "x_rowsum")
    _check("bitlinear_quant_act_a48", load_library().bitlinear_quant_act_a48(
        _ptr(X), M, K, int(n_outliers), _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), _stream(stream)))
    return Xq, x_scale, x_rowsum


def combine_a48(Y2, Y=None, stream=None):
    """Y[m] = Y2[2m] + Y2[2m+1]: token m's output from the forward of its two parts."""
    import torch
    _require(Y2, torch.float32, None, "Y2")
    M2, N = Y2.shape
    if M2 % 2:
        raise ValueError("Y2 must have an even number of rows")
    if Y is None:
        Y = torch.empty((M2 // 2, N), dtype=torch.float32, device=Y2.device)
    _require(Y, torch.float32, (M2 // 2, N), "Y")
    _check("bitlinear_combine_a48", load_library().bitlinear_combine_a48(
        _ptr(Y2), M2 // 2, N, _ptr(Y), _stream(stream)))
    return Y


def forward(Xq, x_scale, x_rowsum, packed, w_scale, N, nm=NM_DENSE, Y=None, acc=None,
            want_acc=False, workspace=None, stream=None):
    """Y = (Xq . W_eff^T) * w_scale * x_scale, fp32 M x N.  Returns Y or (Y, acc).

    `workspace`: a uint8 device tensor for the call's scratch; when None, one
    of the size forward_workspace_size() reports is taken from torch's
    allocator on the call's device (none when that size is 0).
    """
    import torch
    _require(Xq, torch.int8, None, "Xq")
    M, K = Xq.shape
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    _require(packed, torch.uint8, None, "packed")
    _require(w_scale, torch.float32, (1,), "w_scale")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    _require(Y, torch.float32, (M, N), "Y")
    if acc is None and want_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    if acc is not None:
        _require(acc, torch.int32, (M, N), "acc")
    pb, _ = packed_size(N, K, nm)
    if packed.numel() < pb:
        raise ValueError("packed buffer holds %d bytes, %d needed" % (packed.numel(), pb))
    if workspace is None:
        wb = forward_workspace_size(M, N, K, nm)
        if wb:
            workspace = torch.empty(wb, dtype=torch.uint8, device=Xq.device)
    if workspace is not None:
        _require(workspace, torch.uint8, None, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("bitlinear_forward", load_library().bitlinear_forward(
        _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), _ptr(packed), _ptr(w_scale), _nm(nm),
        M, N, K, _ptr(Y), _ptr(acc), _ptr(workspace), ws_bytes, _stream(stream)))
    return (Y, acc) if (want_acc or acc is not None) else Y


def forward_noalloc(Xq, x_scale, x_rowsum, packed, w_scale, N, nm=NM_DENSE, Y=None, acc=None, stream=None):
    """forward() through bitlinear_forward_noalloc: the library's fixed
    per-GPU scratch instead of a workspace (at most 32 MiB of it; calls must
    not overlap on one GPU).  Y and acc must be given (this allocates nothing);
    returns Y, or (Y, acc) with acc."""
    import torch
    _require(Xq, torch.int8, None, "Xq")
    M, K = Xq.shape
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    _require(packed, torch.uint8, None, "packed")
    _require(w_scale, torch.float32, (1,), "w_scale")
    _require(Y, torch.float32, (M, N), "Y")
    if acc is not None:
        _require(acc, torch.int32, (M, N), "acc")
    pb, _ = packed_size(N, K, nm)
    if packed.numel() < pb:
        raise ValueError("packed buffer holds %d bytes, %d needed" % (packed.numel(), pb))
    _check("bitlinear_forward_noalloc", load_library().bitlinear_forward_noalloc(
        _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), _ptr(packed), _ptr(w_scale), _nm(nm),
        M, N, K, _ptr(Y), _ptr(acc), _stream(stream)))
    return (Y, acc) if acc is not None else Y


def _proj_array(projs, M, Ys, accs, device):
    """Proj structs for (packed, w_scale, N) triples, with their outputs."""
    import torch
    n = len(projs)
    if Ys is None:
        Ys = [torch.empty((M, N), dtype=torch.float32, device=device) for (_, _, N) in projs]
    arr = (Proj * max(n, 1))()
    for i, (packed, ws, N) in enumerate(projs):
        _require(packed, torch.uint8, None, "packed")
        _require(ws, torch.float32, (1,), "w_scale")
        _require(Ys[i], torch.float32, (M, N), "Y")
        if accs is not None:
            _require(accs[i], torch.int32, (M, N), "acc")
        arr[i] = Proj(packed.data_ptr(), ws.data_ptr(), N, Ys[i].data_ptr(),
                      accs[i].data_ptr() if accs is not None else None)
    return arr, Ys


def forward_grouped(Xq, x_scale, x_rowsum, projs, nm=NM_DENSE, Ys=None, accs=None, want_acc=False, stream=None):
    """forward() of every projection in `projs` -- a list of (packed, w_scale,
    N) sharing the quantised input -- in one launch.  Returns the list of Y
    tensors, or (Ys, accs) when accumulators are wanted."""
    import torch
    _require(Xq, torch.int8, None, "Xq")
    M, K = Xq.shape
    _require(x_scale, torch.float32, (M,), "x_scale")
    _require(x_rowsum, torch.int32, (M,), "x_rowsum")
    if accs is None and want_acc:
        accs = [torch.empty((M, N), dtype=torch.int32, device=Xq.device) for (_, _, N) in projs]
    arr, Ys = _proj_array(projs, M, Ys, accs, Xq.device)
    _check("bitlinear_forward_grouped", load_library().bitlinear_forward_grouped(
        _ptr(Xq), _ptr(x_scale), _ptr(x_rowsum), M, K, _nm(nm), arr, len(projs), _stream(stream)))
    return (Ys, accs) if accs is not None else Ys


def forward_fused(X, projs, nm=NM_DENSE, Ys=None, accs=None, want_acc=False, x_scale=None, stream=None):
    """Quantise X (M x K fp32, M <= 16) and apply every projection in `projs`
    -- a list of (packed, w_scale, N) sharing X -- in one launch.

    Returns the list of Y tensors, or (Ys, accs) when accumulators are wanted.
    """
    return forward_fused_ex(X, projs, nm=nm, Ys=Ys, accs=accs, want_acc=want_acc, x_scale=x_scale,
                            stream=stream)


def forward_fused_ex(X, projs, up=None, gamma=None, eps=None, nm=NM_DENSE, Ys=None, accs=None, want_acc=False,
                     x_scale=None, stream=None):
    """forward_fused on transformed rows (see quant_act_ex): with `up` the
    rows are ReLU(X)^2 * up, with `gamma` and `eps` they are RMS-normalised
    before the quantiser.  A transform is served at M = 1, K <= 16384."""
    import torch
    _require(X, torch.float32, None, "X")
    M, K = X.shape
    tr = _transform(X, up, gamma, eps)
    n = len(projs)
    if Ys is None:
        Ys = [torch.empty((M, N), dtype=torch.float32, device=X.device) for (_, _, N) in projs]
    if accs is None and want_acc:
        accs = [torch.empty((M, N), dtype=torch.int32, device=X.device) for (_, _, N) in projs]
    arr = (Proj * max(n, 1))()
    for i, (packed, ws, N) in enumerate(projs):
        _require(packed, torch.uint8, None, "packed")
        _require(ws, torch.float32, (1,), "w_scale")
        _require(Ys[i], torch.float32, (M, N), "Y")
        if accs is not None:
            _require(accs[i], torch.int32, (M, N), "acc")
        arr[i] = Proj(packed.data_ptr(), ws.data_ptr(), N, Ys[i].data_ptr(),
                      accs[i].data_ptr() if accs is not None else None)
    if x_scale is not None:
        _require(x_scale, torch.float32, (M,), "x_scale")
    if tr is None:
        _check("bitlinear_forward_fused", load_library().bitlinear_forward_fused(
            _ptr(X), M, K, _nm(nm), arr, n, _ptr(x_scale), _stream(stream)))
    else:
        _check("bitlinear_forward_fused_ex", load_library().bitlinear_forward_fused_ex(
            _ptr(X), ctypes.byref(tr), M, K, _nm(nm), arr, n, _ptr(x_scale), _stream(stream)))
    return (Ys, accs) if accs is not None else Ys


def forward_fused_multi(groups, nm=NM_DENSE, stream=None):
    """forward_fused at M = 1 for several input groups in one call: `groups`
    is a list of (X, projs, Ys, accs, x_scale), X a 1 x K fp32 row, projs a
    list of (packed, w_scale, N) reading X, Ys their 1 x N outputs, accs None
    or their 1 x N int32 accumulators, x_scale None or a 1-element fp32
    output.  Dense weights run as one launch (each K <= 16384)."""
    import torch
    keep = []
    garr = (InputGroup * max(len(groups), 1))()
    for g, (X, projs, Ys, accs, x_scale) in enumerate(groups):
        _require(X, torch.float32, None, "X")
        M, K = X.shape
        if M != 1:
            raise ValueError("forward_fused_multi takes one token per group (X is %d x %d)" % (M, K))
        arr = (Proj * max(len(projs), 1))()
        for i, (packed, ws, N) in enumerate(projs):
            _require(packed, torch.uint8, None, "packed")
            _require(ws, torch.float32, (1,), "w_scale")
            _require(Ys[i], torch.float32, (1, N), "Y")
            if accs is not None:
                _require(accs[i], torch.int32, (1, N), "acc")
            arr[i] = Proj(packed.data_ptr(), ws.data_ptr(), N, Ys[i].data_ptr(),
                          accs[i].data_ptr() if accs is not None else None)
        if x_scale is not None:
            _require(x_scale, torch.float32, (1,), "x_scale")
        keep.append(arr)
        garr[g] = InputGroup(_ptr(X), K, arr, len(projs), _ptr(x_scale))
    _check("bitlinear_forward_fused_multi", load_library().bitlinear_forward_fused_multi(
        garr, len(groups), _nm(nm), _stream(stream)))


def quant_act_multi(groups, stream=None):
    """quant_act for several independent inputs in one call: `groups` is a
    list of (X, Xq, x_scale, x_rowsum) with X an M x K fp32 tensor and the
    outputs preallocated (M x K int8, M fp32, M int32 or None)."""
    import torch
    arr = (QuantGroup * max(len(groups), 1))()
    for g, (X, Xq, xs, rs) in enumerate(groups):
        _require(X, torch.float32, None, "X")
        M, K = X.shape
        _require(Xq, torch.int8, (M, K), "Xq")
        _require(xs, torch.float32, (M,), "x_scale")
        if rs is not None:
            _require(rs, torch.int32, (M,), "x_rowsum")
        arr[g] = QuantGroup(_ptr(X), M, K, _ptr(Xq), _ptr(xs), _ptr(rs))
    _check("bitlinear_quant_act_multi", load_library().bitlinear_quant_act_multi(arr, len(groups),
                                                                                 _stream(stream)))


def forward_grouped_multi(groups, nm=NM_DENSE, stream=None):
    """forward_grouped for several quantised inputs in one call: `groups` is a
    list of (Xq, x_scale, x_rowsum, projs, Ys, accs) with Xq an M x K int8
    tensor (M the same for every group), projs a list of (packed, w_scale, N)
    reading it, Ys their M x N fp32 outputs and accs None or their M x N
    int32 accumulators."""
    import torch
    keep = []
    garr = (ActGroup * max(len(groups), 1))()
    M = None
    for g, (Xq, xs, rs, projs, Ys, accs) in enumerate(groups):
        _require(Xq, torch.int8, None, "Xq")
        m, K = Xq.shape
        if M is None:
            M = m
        elif m != M:
            raise ValueError("every group of forward_grouped_multi has the same token count (%d, %d)" % (M, m))
        _require(xs, torch.float32, (M,), "x_scale")
        _require(rs, torch.int32, (M,), "x_rowsum")
        arr = (Proj * max(len(projs), 1))()
        for i, (packed, ws, N) in enumerate(projs):
            _require(packed, torch.uint8, None, "packed")
            _require(ws, torch.float32, (1,), "w_scale")
            _require(Ys[i], torch.float32, (M, N), "Y")
            if accs is not None:
                _require(accs[i], torch.int32, (M, N), "acc")
            arr[i] = Proj(packed.data_ptr(), ws.data_ptr(), N, Ys[i].data_ptr(),
                          accs[i].data_ptr() if accs is not None else None)
        keep.append(arr)
        garr[g] = ActGroup(_ptr(Xq), _ptr(xs), _ptr(rs), K, arr, len(projs))
    _check("bitlinear_forward_grouped_multi", load_library().bitlinear_forward_grouped_multi(
        garr, len(groups), M or 0, _nm(nm), _stream(stream)))
