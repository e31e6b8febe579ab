"""ctypes wrapper around the plain C oracle in bitlinear_oracle.c.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function takes
and returns numpy arrays; the arithmetic lives in the C file, whose header
cites the pages each step follows:

* "BitNet b1.58 2B4T Technical Report 요약 설명", sec. 2 Architecture and
  sec. 5.1 GPU Inference;
* "BitNet 논문 분석: 1-Bit LLM의 시대", sections "Absmean 양자화 함수" and
  "bitnet.cpp 추론 프레임워크" (I2_S code);
* "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to Semi-Structured
  Sparsity" (review), sec. 3.2 (N:M mask, quant-then-mask).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
# BITLINEAR_ORACLE_LIB lets the mutation test load a deliberately broken copy
LIB_PATH = os.environ.get("BITLINEAR_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]

OK = 0
EINVAL = -1
ENONFINITE = -5


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE arithmetic, no FMA contraction)."""
    if os.environ.get("BITLINEAR_ORACLE_LIB"):
        return LIB_PATH
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_absmean.argtypes = [vp, i64, i64, vp]
        lib.oracle_ternarize.argtypes = [vp, i64, ctypes.c_float, vp]
        lib.oracle_nm_keep.argtypes = [vp, i64, i64, i32, i32, vp]
        lib.oracle_apply_mask.argtypes = [vp, vp, i64, vp]
        lib.oracle_packed_bytes.argtypes = [i64, i64, i32, i32]
        lib.oracle_packed_bytes.restype = i64
        lib.oracle_pack_dense.argtypes = [vp, i64, i64, vp]
        lib.oracle_packed_bytes_trit24.argtypes = [i64, i64]
        lib.oracle_packed_bytes_trit24.restype = i64
        lib.oracle_pack_trit24.argtypes = [vp, vp, i64, i64, vp]
        lib.oracle_unpack_trit24.argtypes = [vp, i64, i64, vp]
        lib.oracle_pack_nm.argtypes = [vp, vp, i64, i64, i32, i32, vp]
        lib.oracle_quant_act.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        lib.oracle_quant_act_ex.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, vp, vp, vp]
        lib.oracle_hadamard_rows.argtypes = [vp, i64, i64, i64]
        lib.oracle_quant_act_h4.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        lib.oracle_quant_act_a48.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
        lib.oracle_forward.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, i64, vp, vp]
        for f in ("oracle_absmean", "oracle_ternarize", "oracle_nm_keep", "oracle_apply_mask",
                  "oracle_pack_dense", "oracle_pack_nm", "oracle_quant_act", "oracle_quant_act_ex",
                  "oracle_hadamard_rows", "oracle_quant_act_h4", "oracle_quant_act_a48", "oracle_forward"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != OK:
        raise ValueError("oracle %s failed with status %d" % (what, rc))


def absmean(W: np.ndarray) -> np.float32:
    """beta = mean |W| (binary64 row sums, then over rows), rounded to fp32."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.zeros(1, np.float32)
    _check(_L().oracle_absmean(_p(W), N, K, _p(out)), "absmean")
    return out[0]


def ternarize(W: np.ndarray, beta) -> np.ndarray:
    """t = clamp(round(W / fl32(beta + 1e-5)), -1, 1) as int8."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    t = np.empty(W.shape, np.int8)
    _check(_L().oracle_ternarize(_p(W), W.size, float(np.float32(beta)), _p(t)), "ternarize")
    return t


def nm_keep(W: np.ndarray, n: int, m: int) -> np.ndarray:
    """uint8 keep mask (1 = kept): top-n |W| per group of m along K, ties to lower k."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    keep = np.empty(W.shape, np.uint8)
    _check(_L().oracle_nm_keep(_p(W), N, K, n, m, _p(keep)), "nm_keep")
    return keep


def apply_mask(t: np.ndarray, keep: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.int8)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    out = np.empty(t.shape, np.int8)
    _check(_L().oracle_apply_mask(_p(t), _p(keep), t.size, _p(out)), "apply_mask")
    return out


def packed_bytes(N: int, K: int, n: int = 0, m: int = 0) -> int:
    return int(_L().oracle_packed_bytes(N, K, n, m))


def pack_dense(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    out = np.empty(packed_bytes(N, K), np.uint8)
    _check(_L().oracle_pack_dense(_p(t), N, K, _p(out)), "pack_dense")
    return out


def pack_nm(t: np.ndarray, keep: np.ndarray, n: int, m: int) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.int8)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    N, K = t.shape
    out = np.empty(packed_bytes(N, K, n, m), np.uint8)
    _check(_L().oracle_pack_nm(_p(t), _p(keep), N, K, n, m, _p(out)), "pack_nm")
    return out


def packed_bytes_trit24(N: int, K: int) -> int:
    return int(_L().oracle_packed_bytes_trit24(N, K))


def pack_trit24(t: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """2:4 trit pack: one 6-bit code per group of 4 (the pair of kept inputs
    and their two ternary values), 16 codes per 12 bytes."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    N, K = t.shape
    out = np.empty(packed_bytes_trit24(N, K), np.uint8)
    _check(_L().oracle_pack_trit24(_p(t), _p(keep), N, K, _p(out)), "pack_trit24")
    return out


def unpack_trit24(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((N, K), np.int8)
    _check(_L().oracle_unpack_trit24(_p(packed), N, K, _p(out)), "unpack_trit24")
    return out


def quantize_weights_trit24(W: np.ndarray):
    """The 2:4 pack-time path in the trit-packed storage: (beta, w_eff, bytes)."""
    beta = absmean(W)
    t = ternarize(W, beta)
    keep = nm_keep(W, 2, 4)
    return beta, apply_mask(t, keep), pack_trit24(t, keep)


def quantize_weights(W: np.ndarray, n: int = 0, m: int = 0):
    """The whole pack-time path: returns (beta, w_eff int8 N x K, packed bytes).

    Ternarise with the full-matrix absmean, then (for N:M) mask by the latent
    magnitudes -- quant-then-mask -- and pack.
    """
    beta = absmean(W)
    t = ternarize(W, beta)
    if n == 0 and m == 0:
        return beta, t, pack_dense(t)
    keep = nm_keep(W, n, m)
    return beta, apply_mask(t, keep), pack_nm(t, keep, n, m)


def quant_act(X: np.ndarray, variant: int = 0):
    """Per-row absmax int8 quantisation: returns (q int8, x_scale fp32, rowsum int32)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    q = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    _check(_L().oracle_quant_act(_p(X), M, K, variant, _p(q), _p(xs), _p(rs)), "quant_act")
    return q, xs, rs


def quant_act_ex(X: np.ndarray, up=None, gamma=None, eps: float = 0.0):
    """Absmax int8 quantisation of the transformed rows: h = ReLU(X)^2 * up when
    `up` is given (else h = X), then RMSNorm with weight `gamma` (length K) and
    epsilon `eps` when `gamma` is given.  Returns (q int8, x_scale fp32, rowsum
    int32); see step 6b of the C file."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    if up is not None:
        up = np.ascontiguousarray(up, dtype=np.float32)
        if up.shape != X.shape:
            raise ValueError("up must have the shape of X")
    if gamma is not None:
        gamma = np.ascontiguousarray(gamma, dtype=np.float32)
        if gamma.shape != (K,):
            raise ValueError("gamma must have K entries")
    q = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    null = ctypes.c_void_p(None)
    _check(_L().oracle_quant_act_ex(_p(X), _p(up) if up is not None else null,
                                    _p(gamma) if gamma is not None else null, float(eps), M, K,
                                    _p(q), _p(xs), _p(rs)), "quant_act_ex")
    return q, xs, rs


def hadamard_rows(X: np.ndarray, B: int) -> np.ndarray:
    """H_B (Sylvester, entries +-1, unnormalised) applied to each block of B
    inputs of each row, with binary32 butterflies in the fixed order."""
    V = np.array(X, dtype=np.float32, copy=True, order="C")
    M, K = V.shape
    _check(_L().oracle_hadamard_rows(_p(V), M, K, int(B)), "hadamard_rows")
    return V


def quant_act_h4(X: np.ndarray, B: int):
    """4-bit absmax codes (int8 storage) of the block-Hadamard-transformed rows;
    returns (q int8, x_scale fp32 incl. 1/sqrt(B), rowsum int32)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    q = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    _check(_L().oracle_quant_act_h4(_p(X), M, K, int(B), _p(q), _p(xs), _p(rs)), "quant_act_h4")
    return q, xs, rs


def quant_act_a48(X: np.ndarray, T: int):
    """BitNet a4.8 hybrid activations with T outliers per row: returns
    (q int8 2M x K, x_scale fp32 2M, rowsum int32 2M, sel uint8 M x K); row
    2m holds token m's 8-bit outlier codes, row 2m+1 its 4-bit codes, sel
    marks the outliers.  See step 6d of the C file."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    q = np.empty((2 * M, K), np.int8)
    xs = np.empty(2 * M, np.float32)
    rs = np.empty(2 * M, np.int32)
    sel = np.empty((M, K), np.uint8)
    _check(_L().oracle_quant_act_a48(_p(X), M, K, int(T), _p(q), _p(xs), _p(rs), _p(sel)), "quant_act_a48")
    return q, xs, rs, sel


def forward_a48(q2: np.ndarray, xs2: np.ndarray, w_eff: np.ndarray, beta):
    """The linear on the 2M hybrid rows, each pair summed: returns (acc int32
    2M x N, Y binary64 M x N, Y_parts binary64 2M x N)."""
    acc, Yp = forward(q2, xs2, w_eff, beta)
    return acc, Yp[0::2] + Yp[1::2], Yp


def forward(q: np.ndarray, x_scale: np.ndarray, w_eff: np.ndarray, beta):
    """Exact int acc (int32) and Y = acc * beta * x_scale in binary64."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    x_scale = np.ascontiguousarray(x_scale, dtype=np.float32)
    w_eff = np.ascontiguousarray(w_eff, dtype=np.int8)
    M, K = q.shape
    N, K2 = w_eff.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.empty((M, N), np.int32)
    Y = np.empty((M, N), np.float64)
    _check(_L().oracle_forward(_p(q), _p(x_scale), _p(w_eff), float(np.float32(beta)),
                               M, N, K, _p(acc), _p(Y)), "forward")
    return acc, Y
