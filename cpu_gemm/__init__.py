"""Cache-blocked CPU GEMM (fp32 accumulation, all cores): the second CPU
baseline ``bench.py`` reports beside the oracle.  It is neither the oracle
nor part of the GPU path; its results serve only as a timing reference.

Compiled with gcc for the host it runs on (``-O3 -march=native``) on first
use, into ``cpu_gemm/_build/`` under a name keyed by the source and the
host's CPU flags, so a library built on one machine is never loaded on
another.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "blocked_gemm.c")
TYPES = {"f32": 0, "f16": 1, "bf16": 2}
_lock = threading.Lock()
_lib = None


def _host_key() -> str:
    h = hashlib.sha256(open(SRC, "rb").read())
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith(("flags", "model name")):
                    h.update(line.encode())
    except OSError:
        pass
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        out = os.path.join(HERE, "_build", f"libblocked_{_host_key()}.so")
        if not os.path.exists(out):
            os.makedirs(os.path.dirname(out), exist_ok=True)
            tmp = out + f".tmp{os.getpid()}"
            subprocess.run(["gcc", "-O3", "-march=native", "-ffp-contract=fast", "-fPIC", "-shared",
                            "-pthread", SRC, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, out)
        lib = ctypes.CDLL(out)
        i, i64, f, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.blocked_gemm.argtypes = [i, i, i, i, i, f, vp, i, i64, vp, i, i64, f, vp, i64, vp, i64, i, i, i]
        lib.blocked_gemm.restype = i
        _lib = lib
        return lib


def gemm_rows(A, B, *, in_dtype, ta, tb, M, N, K, alpha=1.0, beta=0.0, Cin=None, rows=None,
              threads=None) -> np.ndarray:
    """Rows [r0, r1) of C = alpha * op(A) op(B) + beta * Cin as fp32.

    A, B: C-contiguous numpy arrays of the stored matrices (float32, or uint16
    bit patterns for f16 / bf16); Cin: fp32 M x N (read only when beta != 0)."""
    lib = load()
    r0, r1 = rows if rows is not None else (0, M)
    threads = threads or len(os.sched_getaffinity(0))
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    out = np.zeros((max(r1 - r0, 0), N), dtype=np.float32)
    cin_ptr, ldcin = None, N
    if beta != 0.0:
        Cin = np.ascontiguousarray(Cin, dtype=np.float32)
        cin_ptr, ldcin = Cin.ctypes.data, Cin.shape[1]
    # row m of C lives at out[m - r0]
    c_ptr = out.ctypes.data - r0 * N * 4
    rc = lib.blocked_gemm(int(ta), int(tb), M, N, K, float(alpha), A.ctypes.data, TYPES[in_dtype],
                          A.shape[1], B.ctypes.data, TYPES[in_dtype], B.shape[1], float(beta),
                          cin_ptr, ldcin, c_ptr, N, r0, r1, threads)
    if rc != 0:
        raise MemoryError("blocked_gemm could not allocate its buffers")
    return out
