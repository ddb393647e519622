"""CPU oracle for dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

The arithmetic lives in ``oracle_gemm.c`` (plain C, fp64 accumulation, the
GEMM definition written out).  This module builds that file with gcc when the
shared library is missing or older than its source, and marshals numpy
arrays.  Matrices are passed as 2-D numpy arrays holding the *stored* bits:

* ``"f32"``  -> ``np.float32``
* ``"f16"``  -> ``np.float16`` or ``np.uint16`` (the binary16 bit pattern)
* ``"bf16"`` -> ``np.uint16`` (the bfloat16 bit pattern)
* ``"f64"``  -> ``np.float64``

A row stride larger than the row length is the leading dimension (a numpy
slice of a wider array).  The inner stride must be one element.

Parity status of every function is pinned by ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
_ITEM = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8}
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle_gemm.c into liboracle.so (no fast-math: IEEE arithmetic)."""
    stale = (not os.path.exists(_LIB_PATH)) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c11", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
            lib.oracle_gemm_rows.argtypes = [ci, ci, i64, i64, i64, dbl, vp, ci, i64, vp, ci, i64,
                                             dbl, vp, ci, i64, vp, i64, i64, ci]
            lib.oracle_gemm_rows.restype = ci
            lib.oracle_gemm_element.argtypes = [ci, ci, i64, dbl, vp, ci, i64, vp, ci, i64, dbl,
                                                vp, ci, i64, i64, i64]
            lib.oracle_gemm_element.restype = dbl
            lib.oracle_round_array.argtypes = [vp, i64, ci, vp]
            lib.oracle_round_array.restype = None
            lib.oracle_widen_array.argtypes = [vp, i64, ci, vp]
            lib.oracle_widen_array.restype = None
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _mat(x, dtype):
    """Return (array, leading dimension) for a stored matrix."""
    if x is None:
        return None, 0
    x = np.asarray(x)
    if dtype in ("f16", "bf16") and x.dtype == np.float16:
        x = x.view(np.uint16)
    want = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}[dtype]
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} matrix must be stored as {want}, got {x.dtype}")
    if x.ndim != 2:
        raise ValueError("oracle: matrices are 2-D")
    item = x.itemsize
    if x.size == 0:
        return x, max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != item:
        raise ValueError("oracle: inner stride must be one element")
    if x.strides[0] % item:
        raise ValueError("oracle: row stride must be a whole number of elements")
    ld = x.strides[0] // item if x.shape[0] > 1 else max(x.shape[1], 1)
    return x, ld


def gemm(A, B, *, a_dtype="f32", b_dtype=None, trans_a=False, trans_b=False, alpha=1.0,
         beta=0.0, C=None, c_dtype="f32", M=None, N=None, K=None, rows=None, threads=None):
    """fp64 result of alpha*op(A)@op(B) + beta*C as an (rows x N) float64 array.

    ``A`` is stored M x K (or K x M when ``trans_a``); ``B`` is stored K x N
    (or N x K when ``trans_b``).  ``rows=(r0, r1)`` evaluates only those rows
    of the result.  Shapes may be given explicitly for empty matrices.
    """
    b_dtype = b_dtype or a_dtype
    lib = _load()
    A, lda = _mat(A, a_dtype)
    B, ldb = _mat(B, b_dtype)
    if M is None:
        M = A.shape[1] if trans_a else A.shape[0]
    if K is None:
        K = A.shape[0] if trans_a else A.shape[1]
    if N is None:
        N = B.shape[0] if trans_b else B.shape[1]
    if A is not None and K > 0 and M > 0:
        assert (A.shape == (K, M)) if trans_a else (A.shape == (M, K)), "A shape"
    if B is not None and K > 0 and N > 0:
        assert (B.shape == (N, K)) if trans_b else (B.shape == (K, N)), "B shape"
    Cm, ldc = (None, 0)
    if beta != 0.0:
        Cm, ldc = _mat(C, c_dtype)
        if Cm is None:
            assert M * N == 0, "beta != 0 needs C"
        else:
            assert Cm.shape == (M, N), "C shape"
    r0, r1 = rows if rows is not None else (0, M)
    out = np.empty((r1 - r0, N), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.oracle_gemm_rows(int(trans_a), int(trans_b), M, N, K, float(alpha), ptr(A),
                              _CODES[a_dtype], lda, ptr(B), _CODES[b_dtype], ldb, float(beta),
                              ptr(Cm), _CODES[c_dtype], ldc, out.ctypes.data, r0, r1,
                              threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_rows failed ({rc})")
    return out


def element(A, B, i, j, *, a_dtype="f32", b_dtype=None, trans_a=False, trans_b=False,
            alpha=1.0, beta=0.0, C=None, c_dtype="f32", K=None):
    """fp64 value of one output element C[i][j] (same arithmetic as gemm)."""
    b_dtype = b_dtype or a_dtype
    lib = _load()
    A, lda = _mat(A, a_dtype)
    B, ldb = _mat(B, b_dtype)
    if K is None:
        K = A.shape[0] if trans_a else A.shape[1]
    Cm, ldc = (None, 0)
    if beta != 0.0:
        Cm, ldc = _mat(C, c_dtype)
    return lib.oracle_gemm_element(int(trans_a), int(trans_b), K, float(alpha), A.ctypes.data,
                                   _CODES[a_dtype], lda, B.ctypes.data, _CODES[b_dtype], ldb,
                                   float(beta), None if Cm is None else Cm.ctypes.data,
                                   _CODES[c_dtype], ldc, int(i), int(j))


def round_to(x, dtype):
    """Correctly rounded (nearest-even) narrowing of fp64 values.

    Returns float32 values for "f32" and uint16 bit patterns for "f16"/"bf16".
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float32 if dtype == "f32" else
                   (np.float64 if dtype == "f64" else np.uint16))
    lib.oracle_round_array(x.ctypes.data, x.size, _CODES[dtype], out.ctypes.data)
    return out


def widen(bits, dtype):
    """Exact fp64 values of stored f32/f16/bf16 data."""
    lib = _load()
    want = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}[dtype]
    bits = np.asarray(bits)
    if bits.dtype == np.float16:
        bits = bits.view(np.uint16)
    bits = np.ascontiguousarray(bits, dtype=want)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_widen_array(bits.ctypes.data, bits.size, _CODES[dtype], out.ctypes.data)
    return out


def row_norms(A, dtype, trans=False):
    """2-norms of the rows of op(A) (fp64, from the stored values)."""
    a = widen(A, dtype)
    if trans:
        a = a.T
    return np.sqrt(np.sum(a * a, axis=1))


def col_norms(B, dtype, trans=False):
    """2-norms of the columns of op(B) (fp64, from the stored values)."""
    b = widen(B, dtype)
    if trans:
        b = b.T
    return np.sqrt(np.sum(b * b, axis=0))
