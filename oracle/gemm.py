"""Float64 GEMM reference (test infrastructure only).

D(m,n) = C(m,n) + sum_{k<K} A(m,k) * B(n,k), with A (M,K), B (N,K), C/D
(M,N) as fixed on the TiledMMA page ("读懂 CuTe 的 make_tiled_mma：一条 MMA
怎样铺成一块矩阵", section "先固定矩阵和方向").  The C triple loop lives in
``gemm_ref.c``; ``gemm_f64_py`` is the same definition in pure Python for tiny
shapes (used to pin the C version).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction
from typing import Optional

import numpy as np

from . import fp16

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_ref.c")
_LIB_PATH = os.path.join(_HERE, "libgemm_ref.so")
_lib = None

C_NONE, C_F16, C_F32 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile gemm_ref.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_gemm_f64.argtypes = [i64, i64, i64, vp, i64, ci, vp, i64,
                                        vp, ci, i64, vp, i64, i64, i64, ci]
        lib.oracle_gemm_f64.restype = ci
        lib.oracle_gemm_f64_sampled.argtypes = [i64, i64, i64, vp, i64, ci, vp,
                                                i64, vp, ci, i64, i64, vp, vp,
                                                vp, ci]
        lib.oracle_gemm_f64_sampled.restype = ci
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ci
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _bits(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16
    return np.ascontiguousarray(x)


def _c_args(C: Optional[np.ndarray]):
    if C is None:
        return None, C_NONE, 0
    C = np.ascontiguousarray(C)
    if C.dtype == np.float16:
        return C.view(np.uint16), C_F16, C.shape[1]
    if C.dtype == np.float32:
        return C, C_F32, C.shape[1]
    raise TypeError(C.dtype)


def gemm_f64(M: int, N: int, K: int, A: np.ndarray, lda: int, a_mmajor: bool,
             B: np.ndarray, ldb: int, C: Optional[np.ndarray] = None,
             rows: Optional[tuple] = None, nthreads: int = 0) -> np.ndarray:
    """Float64 D for rows [m0, m1) (default all).  A and B are fp16 buffers
    (flat or 2-D) addressed through lda/ldb; C is (M, ldc) fp16/fp32 or None.
    Returns an (M, N) float64 array (rows outside [m0, m1) are NaN)."""
    lib = _load()
    A = _bits(np.asarray(A))
    B = _bits(np.asarray(B))
    Cb, ck, ldc = _c_args(C)
    D = np.full((M, N), np.nan, dtype=np.float64)
    m0, m1 = rows if rows is not None else (0, M)
    rc = lib.oracle_gemm_f64(M, N, K, A.ctypes.data, lda, int(bool(a_mmajor)),
                             B.ctypes.data, ldb,
                             None if Cb is None else Cb.ctypes.data, ck, ldc,
                             D.ctypes.data, N, m0, m1, nthreads)
    if rc != 0:
        raise MemoryError("oracle_gemm_f64 failed")
    return D


def gemm_f64_sampled(M: int, N: int, K: int, A, lda: int, a_mmajor: bool,
                     B, ldb: int, C, ms: np.ndarray, ns: np.ndarray,
                     nthreads: int = 0) -> np.ndarray:
    lib = _load()
    A = _bits(np.asarray(A))
    B = _bits(np.asarray(B))
    Cb, ck, ldc = _c_args(C)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape[0], dtype=np.float64)
    rc = lib.oracle_gemm_f64_sampled(M, N, K, A.ctypes.data, lda,
                                     int(bool(a_mmajor)), B.ctypes.data, ldb,
                                     None if Cb is None else Cb.ctypes.data, ck,
                                     ldc, ms.shape[0], ms.ctypes.data,
                                     ns.ctypes.data, out.ctypes.data, nthreads)
    if rc != 0:
        raise IndexError("sample index outside the matrix")
    return out


def gemm_f64_py(M, N, K, A_at, B_at, C_at=None, exact=False):
    """Pure-Python definition for tiny shapes.  ``A_at(m,k)``, ``B_at(n,k)``,
    ``C_at(m,n)`` return floats; with ``exact`` the sum is kept as a
    Fraction (no rounding at all)."""
    out = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            c = C_at(m, n) if C_at else 0.0
            s = Fraction(c) if exact else c
            for k in range(K):
                if exact:
                    s += Fraction(A_at(m, k)) * Fraction(B_at(n, k))
                else:
                    s += A_at(m, k) * B_at(n, k)
            out[m][n] = s
    return out


def operand_accessors(A, lda, a_mmajor, B, ldb, C=None):
    """Element accessors over raw fp16 buffers (exact decode)."""
    Af = fp16.decode_array(_bits(np.asarray(A)).reshape(-1))
    Bf = fp16.decode_array(_bits(np.asarray(B)).reshape(-1))

    def A_at(m, k):
        return float(Af[m + k * lda] if a_mmajor else Af[m * lda + k])

    def B_at(n, k):
        return float(Bf[n * ldb + k])

    C_at = None
    if C is not None:
        if C.dtype == np.float16:
            Cf = fp16.decode_array(C)
        else:
            Cf = C.astype(np.float64)

        def C_at(m, n):
            return float(Cf[m, n])

    return A_at, B_at, C_at
