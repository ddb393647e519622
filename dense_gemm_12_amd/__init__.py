"""dense_gemm_12_amd -- dense GEMM for AMD MI355X (gfx950).

A thin ctypes binding over ``libmgemm.so`` (C ABI in ``include/mgemm.h``).
The functions ``gemm_f32``, ``gemm_f16`` and ``gemm_bf16`` (and their
``*_cfg`` forms) take the C ABI's arguments one for one: device pointers as
integers, sizes, leading dimensions, and a HIP stream handle.  ``gemm`` is a
convenience over torch tensors that only reads pointers, strides and the
current stream.  Every step of the computation runs in the HIP kernels; there
is no fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmgemm.so")
TUNE_TABLE = os.path.join(HERE, "tune_gfx950.txt")

MG_OK, MG_EINVAL, MG_EUNSUPPORTED, MG_EHIP, MG_ESCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 32 << 20
MG_N, MG_T = 0, 1
MG_F32, MG_F16, MG_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": MG_F32, "f16": MG_F16, "bf16": MG_BF16}

# Every exported symbol of include/mgemm.h.
EXPORTS = (
    "gemm_f32", "gemm_f16", "gemm_bf16", "gemm_f32_cfg", "gemm_f16_cfg", "gemm_bf16_cfg",
    "gemm_ex", "gemm_ex_noalloc", "mg_workspace_size", "gemm_f32_split16", "mg_split16_workspace_size", "mg_chosen_config_ws",
    "mg_num_configs", "mg_config_name", "mg_chosen_config", "mg_load_tune_table",
    "mg_tune_table_size", "mg_config_occupancy", "mg_status_str", "mg_last_hip_error", "mg_version",
)


class MgemmError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        text = lib.mg_status_str(status).decode() if lib is not None else str(status)
        hip = lib.mg_last_hip_error() if (lib is not None and status == MG_EHIP) else 0
        super().__init__(f"{where}: {text} (status {status}{', hip error %d' % hip if hip else ''})")
        self.status = status


_lock = threading.Lock()
_lib = None


def load(path: str | None = None):
    """Load libmgemm.so (never builds it; build with ``python -m dense_gemm_12_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = path or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"libmgemm.so not built at {path}; run python -m dense_gemm_12_amd.build")
        lib = ctypes.CDLL(path)
        ci, i64, f, vp, cp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_char_p
        gemm32 = [ci, ci, i64, i64, i64, f, vp, i64, vp, i64, f, vp, i64, vp]
        gemm16 = [ci, ci, i64, i64, i64, f, vp, i64, vp, i64, f, vp, ci, i64, vp]
        lib.gemm_f32.argtypes = gemm32
        lib.gemm_f16.argtypes = gemm16
        lib.gemm_bf16.argtypes = gemm16
        lib.gemm_f32_cfg.argtypes = [ci] + gemm32
        lib.gemm_f16_cfg.argtypes = [ci] + gemm16
        lib.gemm_bf16_cfg.argtypes = [ci] + gemm16
        for name in ("gemm_f32", "gemm_f16", "gemm_bf16", "gemm_f32_cfg", "gemm_f16_cfg",
                     "gemm_bf16_cfg"):
            getattr(lib, name).restype = ci
        lib.gemm_ex.argtypes = [ci, ci, ci, ci, i64, i64, i64, f, vp, i64, vp, i64, f, vp, i64, vp,
                                ctypes.c_size_t, ci, ci, vp]
        lib.gemm_ex.restype = ci
        lib.gemm_ex_noalloc.argtypes = [ci, ci, ci, ci, i64, i64, i64, f, vp, i64, vp, i64, f, vp, i64, ci,
                                        ci, vp]
        lib.gemm_ex_noalloc.restype = ci
        lib.mg_workspace_size.argtypes = [ci, ci, ci, ci, i64, i64, i64, i64, i64]
        lib.mg_workspace_size.restype = ctypes.c_size_t
        lib.gemm_f32_split16.argtypes = [ci, ci, i64, i64, i64, f, vp, i64, vp, i64, f, vp, i64, vp,
                                         ctypes.c_size_t, vp]
        lib.gemm_f32_split16.restype = ci
        lib.mg_split16_workspace_size.argtypes = [i64, i64, i64]
        lib.mg_split16_workspace_size.restype = ctypes.c_size_t
        lib.mg_chosen_config_ws.argtypes = [ci, ci, ci, ci, i64, i64, i64, i64, i64]
        lib.mg_chosen_config_ws.restype = ci
        lib.mg_num_configs.argtypes = [ci]
        lib.mg_num_configs.restype = ci
        lib.mg_config_name.argtypes = [ci, ci]
        lib.mg_config_name.restype = cp
        lib.mg_chosen_config.argtypes = [ci, ci, ci, ci, i64, i64, i64]
        lib.mg_chosen_config.restype = ci
        lib.mg_load_tune_table.argtypes = [cp]
        lib.mg_load_tune_table.restype = ci
        lib.mg_tune_table_size.argtypes = []
        lib.mg_tune_table_size.restype = ci
        lib.mg_config_occupancy.argtypes = [ci, ci]
        lib.mg_config_occupancy.restype = ci
        lib.mg_status_str.argtypes = [ci]
        lib.mg_status_str.restype = cp
        lib.mg_last_hip_error.argtypes = []
        lib.mg_last_hip_error.restype = ci
        lib.mg_version.argtypes = []
        lib.mg_version.restype = cp
        if os.path.exists(TUNE_TABLE) and not os.environ.get("MGEMM_NO_TUNE_TABLE"):
            st = lib.mg_load_tune_table(TUNE_TABLE.encode())
            if st != MG_OK:
                raise MgemmError(st, f"mg_load_tune_table({TUNE_TABLE})", lib)
        _lib = lib
        return lib


def _check(st: int, where: str):
    if st != MG_OK:
        raise MgemmError(st, where, _lib)


# ---- the C ABI, one for one ------------------------------------------------

def gemm_f32(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    _check(load().gemm_f32(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream), "gemm_f32")


def gemm_f16(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=None):
    _check(load().gemm_f16(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream),
           "gemm_f16")


def gemm_bf16(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=None):
    _check(load().gemm_bf16(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream),
           "gemm_bf16")


def gemm_f32_cfg(config, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    _check(load().gemm_f32_cfg(config, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               stream), "gemm_f32_cfg")


def gemm_f16_cfg(config, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=None):
    _check(load().gemm_f16_cfg(config, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type,
                               ldc, stream), "gemm_f16_cfg")


def gemm_bf16_cfg(config, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream=None):
    _check(load().gemm_bf16_cfg(config, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type,
                                ldc, stream), "gemm_bf16_cfg")


def gemm_ex(in_type, c_type, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
            workspace_bytes, config=-1, splits=0, stream=None):
    _check(load().gemm_ex(in_type, c_type, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                          workspace, workspace_bytes, config, splits, stream), "gemm_ex")


def gemm_ex_noalloc(in_type, c_type, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, config=-1,
                    splits=0, stream=None):
    _check(load().gemm_ex_noalloc(in_type, c_type, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                  config, splits, stream), "gemm_ex_noalloc")


def workspace_size(in_type, c_type, ta, tb, M, N, K, lda, ldb) -> int:
    """Bytes of split-K workspace gemm_ex(splits=0) uses (codes as in the C ABI)."""
    return load().mg_workspace_size(in_type, c_type, ta, tb, M, N, K, lda, ldb)


def gemm_f32_split16(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes,
                     stream=None):
    _check(load().gemm_f32_split16(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                                   workspace_bytes, stream), "gemm_f32_split16")


def split16_workspace_size(M, N, K) -> int:
    return load().mg_split16_workspace_size(M, N, K)


def num_configs(in_type: str) -> int:
    return load().mg_num_configs(DTYPE_CODES[in_type])


def config_name(in_type: str, config: int) -> str:
    n = load().mg_config_name(DTYPE_CODES[in_type], config)
    return n.decode() if n is not None else None


def config_id(in_type: str, name: str) -> int:
    for i in range(num_configs(in_type)):
        if config_name(in_type, i) == name:
            return i
    raise KeyError(name)


def config_occupancy(in_type: str, config: int) -> int:
    """Workgroups of a configuration per CU on the current device (-1 if unknown)."""
    return load().mg_config_occupancy(DTYPE_CODES[in_type], config)


def chosen_config(in_type, c_type, ta, tb, M, N, K) -> int:
    return load().mg_chosen_config(DTYPE_CODES[in_type], DTYPE_CODES[c_type], ta, tb, M, N, K)


def chosen_config_ws(in_type, c_type, ta, tb, M, N, K, lda, ldb) -> int:
    return load().mg_chosen_config_ws(DTYPE_CODES[in_type], DTYPE_CODES[c_type], ta, tb, M, N, K, lda, ldb)


def load_tune_table(path: str):
    _check(load().mg_load_tune_table(path.encode()), "mg_load_tune_table")


# ---- torch convenience -------------------------------------------------------

def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("matrices are 2-D")
    if t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("inner stride must be 1 (row-major storage)")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, trans_a: bool = False,
         trans_b: bool = False, config: int = -1, stream=None, workspace=None, splits: int = 0,
         split16: bool = False):
    """C <- alpha * op(A) @ op(B) + beta * C on C's device, in place.

    A, B, C are 2-D CUDA tensors holding the *stored* matrices (A is K x M when
    trans_a; B is N x K when trans_b).  Input dtypes: float32, float16 or
    bfloat16 (A and B alike); C is float32 or the input dtype.  Runs on the
    current stream unless ``stream`` (a torch.cuda.Stream) is given.

    With ``workspace`` (a CUDA tensor used as raw bytes, see
    ``workspace_size``) the call goes through ``gemm_ex`` and may split K
    (``splits``: 0 = the planner's choice, 1 = never, n = that many ranges).

    ``split16`` (fp32 only) runs ``gemm_f32_split16``: fp32 through the fp16
    matrix cores; ``workspace`` must then hold ``split16_workspace_size``
    bytes (a buffer of that size is taken from torch's allocator if None).
    """
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    # every buffer the kernels touch must live on C's GPU: a host pointer
    # handed to a kernel faults the device
    for name, t in (("A", A), ("B", B), ("workspace", workspace)):
        if t is not None and (not t.is_cuda or t.device != C.device):
            raise ValueError(f"{name} must be a CUDA tensor on {C.device}, got {t.device}")
    if not C.is_cuda:
        raise ValueError(f"C must be a CUDA tensor, got {C.device}")
    M = A.shape[1] if trans_a else A.shape[0]
    K = A.shape[0] if trans_a else A.shape[1]
    N = B.shape[0] if trans_b else B.shape[1]
    Kb = B.shape[1] if trans_b else B.shape[0]
    if Kb != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: op(A) {M}x{K}, op(B) {Kb}x{N}, C {tuple(C.shape)}")
    s = (stream or torch.cuda.current_stream(C.device)).cuda_stream
    ta, tb = (MG_T if trans_a else MG_N), (MG_T if trans_b else MG_N)
    args = (M, N, K, float(alpha), A.data_ptr(), _ld(A), B.data_ptr(), _ld(B), float(beta))
    if split16:
        if A.dtype != torch.float32 or C.dtype != torch.float32:
            raise TypeError("split16 computes fp32 GEMMs")
        need = split16_workspace_size(M, N, K)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=C.device)
        gemm_f32_split16(ta, tb, *args, C.data_ptr(), _ld(C), workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), s)
        return C
    if workspace is not None or splits not in (0, 1):
        codes = {torch.float32: MG_F32, torch.float16: MG_F16, torch.bfloat16: MG_BF16}
        if A.dtype not in codes or C.dtype not in codes:
            raise TypeError(f"unsupported dtypes {A.dtype} -> {C.dtype}")
        wp = workspace.data_ptr() if workspace is not None else None
        wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
        gemm_ex(codes[A.dtype], codes[C.dtype], ta, tb, *args, C.data_ptr(), _ld(C), wp, wb,
                config, splits, s)
        return C
    if A.dtype == torch.float32:
        if C.dtype != torch.float32:
            raise TypeError("fp32 GEMM writes fp32 C")
        gemm_f32_cfg(config, ta, tb, *args, C.data_ptr(), _ld(C), s)
        return C
    ctype = {torch.float32: MG_F32, torch.float16: MG_F16, torch.bfloat16: MG_BF16}.get(C.dtype)
    if A.dtype == torch.float16:
        gemm_f16_cfg(config, ta, tb, *args, C.data_ptr(), ctype if ctype is not None else -1,
                     _ld(C), s)
    elif A.dtype == torch.bfloat16:
        gemm_bf16_cfg(config, ta, tb, *args, C.data_ptr(), ctype if ctype is not None else -1,
                      _ld(C), s)
    else:
        raise TypeError(f"unsupported input dtype {A.dtype}")
    return C
