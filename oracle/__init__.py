"""Plain CPU oracle for C[M,N] = A[M,K] * B[N,K]^T (bf16 and fp8-e4m3 inputs).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``dense_gemm_linear_amd``) never imports it and shares no code with it.

This module is a thin ctypes wrapper over ``oracle.c`` (plain C, fp64
accumulation, built with ``-O2 -fno-fast-math -ffp-contract=off``); every piece
of arithmetic lives in that file and is cited there.  The wrappers below only
marshal numpy arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

ORC_BF16 = 0
ORC_E4M3 = 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b

        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f64.restype = ctypes.c_double
    lib.orc_bf16_from_f64.argtypes = [ctypes.c_double]
    lib.orc_bf16_from_f64.restype = ctypes.c_uint16
    lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_to_f64.restype = ctypes.c_double
    lib.orc_e4m3_from_f64.argtypes = [ctypes.c_double]
    lib.orc_e4m3_from_f64.restype = ctypes.c_uint8
    for name in ("orc_bf16_encode_array", "orc_bf16_decode_array",
                 "orc_e4m3_encode_array", "orc_e4m3_decode_array"):
        getattr(lib, name).argtypes = [P, P, I64]
        getattr(lib, name).restype = None
    lib.orc_gemm_bf16.argtypes = [P, I64, P, I64, I64, I64, I64, P, I64, ctypes.c_int]
    lib.orc_gemm_bf16.restype = I64
    lib.orc_gemm_e4m3.argtypes = [P, I64, P, I64, I64, I64, I64, ctypes.c_float,
                                  ctypes.c_float, P, I64, ctypes.c_int]
    lib.orc_gemm_e4m3.restype = I64
    lib.orc_gemm_points.argtypes = [ctypes.c_int, P, I64, P, I64, I64, ctypes.c_double,
                                    P, P, I64, P]
    lib.orc_gemm_points.restype = None
    lib.orc_transpose.argtypes = [P, I64, I64, I64, ctypes.c_int, P, I64]
    lib.orc_transpose.restype = None
    lib.orc_activation.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.orc_activation.restype = ctypes.c_double
    lib.orc_epilogue.argtypes = [P, I64, I64, P, P, P, ctypes.c_int, P, I64]
    lib.orc_epilogue.restype = None
    lib.orc_shuffle_b_bytes.argtypes = [I64, I64, ctypes.c_int]
    lib.orc_shuffle_b_bytes.restype = I64
    lib.orc_shuffle_b.argtypes = [P, I64, I64, I64, ctypes.c_int, P]
    lib.orc_shuffle_b.restype = None
    lib.orc_unshuffle_b.argtypes = [P, I64, I64, ctypes.c_int, P, I64]
    lib.orc_unshuffle_b.restype = None
    lib.orc_dim_eff.argtypes = [I64, I64, I64, I64, I64, P, P, P, P]
    lib.orc_dim_eff.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return min(16, os.cpu_count() or 1)


# ----------------------------------------------------------------- codecs
def bf16_to_f64(bits) -> np.ndarray:
    h = _c(bits, np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().orc_bf16_decode_array(_ptr(h), _ptr(out), h.size)
    return out


def bf16_from_f64(x) -> np.ndarray:
    d = _c(x, np.float64)
    out = np.empty(d.shape, np.uint16)
    _load().orc_bf16_encode_array(_ptr(d), _ptr(out), d.size)
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_from_f64(x) -> np.ndarray:
    d = _c(x, np.float64)
    out = np.empty(d.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(d), _ptr(out), d.size)
    return out


# ------------------------------------------------------------------- GEMM
def gemm_bf16(A_bits, B_bits, threads: int | None = None, return_macs: bool = False):
    """fp64 C = A * B^T for bf16 bit arrays A [M, K] and B [N, K] (row-major).

    With ``return_macs`` also returns the number of multiply-adds performed."""
    A = _c(A_bits, np.uint16)
    B = _c(B_bits, np.uint16)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    C = np.zeros((M, N), np.float64)
    macs = _load().orc_gemm_bf16(_ptr(A), K, _ptr(B), K, M, N, K, _ptr(C), N,
                                 threads or default_threads())
    return (C, int(macs)) if return_macs else C


def gemm_e4m3(A_codes, B_codes, sa: float, sb: float, threads: int | None = None,
              return_macs: bool = False):
    """fp64 C = (A * B^T) * sa * sb for e4m3 code arrays A [M, K], B [N, K]."""
    A = _c(A_codes, np.uint8)
    B = _c(B_codes, np.uint8)
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    C = np.zeros((M, N), np.float64)
    macs = _load().orc_gemm_e4m3(_ptr(A), K, _ptr(B), K, M, N, K, float(sa), float(sb), _ptr(C),
                                 N, threads or default_threads())
    return (C, int(macs)) if return_macs else C


def gemm_points(dtype: int, A, B, ms, ns, scale: float = 1.0) -> np.ndarray:
    """fp64 C[ms[i], ns[i]] only; A [M, K], B [N, K] as bf16 bits or e4m3 codes."""
    npdt = np.uint16 if dtype == ORC_BF16 else np.uint8
    A = _c(A, npdt)
    B = _c(B, npdt)
    K = A.shape[1]
    assert B.shape[1] == K
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ms.shape == ns.shape
    assert (ms >= 0).all() and (ms < A.shape[0]).all()
    assert (ns >= 0).all() and (ns < B.shape[0]).all()
    out = np.zeros(ms.shape, np.float64)
    _load().orc_gemm_points(dtype, _ptr(A), K, _ptr(B), K, K, float(scale), _ptr(ms), _ptr(ns),
                            ms.size, _ptr(out))
    return out


# ----------------------------------------------------------- B preshuffle
def shuffle_b_bytes(N: int, K: int, elem_bytes: int) -> int:
    return int(_load().orc_shuffle_b_bytes(N, K, elem_bytes))


def shuffle_b(B, elem_bytes: int) -> np.ndarray:
    """Preshuffled bytes of row-major B [N, K] (bf16 bits or e4m3 codes)."""
    B = np.ascontiguousarray(B)
    N, K = B.shape
    assert B.itemsize == elem_bytes
    out = np.empty(shuffle_b_bytes(N, K, elem_bytes), np.uint8)
    _load().orc_shuffle_b(_ptr(B), K, N, K, elem_bytes, _ptr(out))
    return out


def unshuffle_b(Bs, N: int, K: int, elem_bytes: int) -> np.ndarray:
    Bs = _c(Bs, np.uint8)
    assert Bs.size == shuffle_b_bytes(N, K, elem_bytes)
    dt = np.uint16 if elem_bytes == 2 else np.uint8
    out = np.zeros((N, K), dt)
    _load().orc_unshuffle_b(_ptr(Bs), N, K, elem_bytes, _ptr(out), K)
    return out


# --------------------------------------------------- dimension efficiency
def dim_eff(M: int, N: int, mt_m: int, mt_n: int, num_cus: int):
    """(num_tiles, tile_eff, wq_eff, dim_eff) of a macro tile on num_cus CUs."""
    t = ctypes.c_int64()
    te = ctypes.c_double()
    we = ctypes.c_double()
    de = ctypes.c_double()
    _load().orc_dim_eff(M, N, mt_m, mt_n, num_cus, ctypes.addressof(t), ctypes.addressof(te),
                        ctypes.addressof(we), ctypes.addressof(de))
    return t.value, te.value, we.value, de.value


# activation codes of orc_activation (the same numbering as the library's)
ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3, 4


def activation(act: int, x) -> np.ndarray:
    """orc_activation elementwise on an array (fp64)."""
    lib = _load()
    x = np.asarray(x, np.float64)
    return np.vectorize(lambda v: lib.orc_activation(act, float(v)), otypes=[np.float64])(x)


def epilogue(C, scale_m=None, scale_n=None, bias=None, act: int = ACT_NONE, mul=None):
    """orc_epilogue on a copy of the fp64 product C [M, N]: scales (fp32
    arrays), bias (bf16 bits [N]), activation, mul (bf16 bits [M, >= N])."""
    lib = _load()
    out = np.ascontiguousarray(C, np.float64).copy()
    M, N = out.shape
    sm = None if scale_m is None else _c(scale_m, np.float32)
    sn = None if scale_n is None else _c(scale_n, np.float32)
    bs = None if bias is None else _c(bias, np.uint16)
    ml = None if mul is None else _c(mul, np.uint16)
    lib.orc_epilogue(_ptr(out), M, N, None if sm is None else _ptr(sm),
                     None if sn is None else _ptr(sn), None if bs is None else _ptr(bs), act,
                     None if ml is None else _ptr(ml), 0 if ml is None else ml.shape[1])
    return out


def transpose(X) -> np.ndarray:
    """orc_transpose of a 2-D uint8 / uint16 array: a new array X^T."""
    lib = _load()
    X = np.ascontiguousarray(X)
    rows, cols = X.shape
    out = np.empty((cols, rows), X.dtype)
    lib.orc_transpose(_ptr(X), cols, rows, cols, X.dtype.itemsize, _ptr(out), rows)
    return out


def shuffle_b_t(Bt, elem_bytes: int) -> np.ndarray:
    """The preshuffled layout of B given Bt = B^T ([K, N]): orc_shuffle_b of
    orc_transpose(Bt)."""
    return shuffle_b(transpose(Bt), elem_bytes)
