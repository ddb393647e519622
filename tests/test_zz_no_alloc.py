"""gemm_ex_noalloc (the split-K / repacking entry point with the library's
fixed scratch array instead of a workspace), called through the C ABI, gives
the same bits as gemm_ex with a workspace of the same size, on two calls in a
row (the second smaller, so stale scratch contents from the first are
present), and matches the oracle: bit-exact on integer data, within the
bound on random data.  A forced split count that needs more than the scratch
is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import gemm_inputs as gi
from gpu_helpers import assert_bit_exact, assert_within, bits, log, oracle_full, out_as_f64

pytestmark = pytest.mark.gpu

CASES = [
    # (in, c, M, N, K, ta, tb, alpha, beta, dist, seed): repacked A (odd K) + split-K, then smaller ones
    ("bf16", "f32", 127, 4096, 4095, False, False, 1.0, 1.0, "uniform", 5000),
    ("bf16", "f32", 100, 1000, 2999, False, False, 1.5, 0.5, "int2", 5100),
    ("f32", "f32", 256, 256, 256, False, False, 1.0, 0.0, "uniform", 5200),
    ("f16", "f16", 64, 192, 1000, True, True, 1.0, 0.0, "int2", 5300),
]


def _inputs(case):
    in_dtype, c_dtype, M, N, K, ta, tb, alpha, beta, dist, seed = case
    A = gi.draw(*((K, M) if ta else (M, K)), dist, seed, in_dtype)
    B = gi.draw(*((N, K) if tb else (K, N)), dist, seed + 1, in_dtype)
    C = gi.draw(M, N, dist if dist == "int2" else "uniform", seed + 2, c_dtype)
    return A, B, C


def _call(mg, fn, case, Ad, Bd, Cd, ws=None, splits=0):
    in_dtype, c_dtype, M, N, K, ta, tb, alpha, beta, *_ = case
    lib = mg.load()
    codes = mg.DTYPE_CODES
    args = [codes[in_dtype], codes[c_dtype], int(ta), int(tb), M, N, K, alpha, Ad.data_ptr(), Ad.stride(0),
            Bd.data_ptr(), Bd.stride(0), beta, Cd.data_ptr(), Cd.stride(0)]
    s = torch.cuda.current_stream().cuda_stream
    if fn == "gemm_ex":
        st = lib.gemm_ex(*args, ws.data_ptr(), ws.numel(), -1, splits, s)
    else:
        st = lib.gemm_ex_noalloc(*args, -1, splits, s)
    return st


def test_noalloc_matches_gemm_ex_and_oracle_two_calls_in_a_row(gpu_lib):
    mg = gpu_lib
    dev = torch.device("cuda:0")
    ws = torch.empty(mg.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=dev)
    for case in CASES:
        in_dtype, c_dtype, M, N, K, ta, tb, alpha, beta, dist, seed = case
        log(f"noalloc case {case}")
        A, B, C = _inputs(case)
        Ad, Bd = A.to(dev), B.to(dev)
        C_na, C_ex = C.to(dev), C.to(dev)
        assert _call(mg, "noalloc", case, Ad, Bd, C_na) == mg.MG_OK
        ws.fill_(0xFF)  # the workspace path must not depend on its contents either
        assert _call(mg, "gemm_ex", case, Ad, Bd, C_ex, ws=ws) == mg.MG_OK
        torch.cuda.synchronize()
        got = C_na.cpu()
        assert torch.equal(bits_t(got), bits_t(C_ex.cpu())), f"{case}: differs from gemm_ex"
        kw = dict(alpha=alpha, beta=beta, ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype)
        ref = oracle_full(A, B, C, **kw)
        if dist == "int2":
            assert_bit_exact(got, ref, c_dtype, f"noalloc {case}")
        else:
            assert_within(out_as_f64(got, c_dtype), ref, A=A, B=B, Cin=C, what=f"noalloc {case}", **kw)


def bits_t(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def test_noalloc_refuses_a_split_beyond_the_scratch(gpu_lib):
    mg = gpu_lib
    dev = torch.device("cuda:0")
    case = ("f32", "f32", 1024, 1024, 4096, False, False, 1.0, 0.0, "int2", 5400)
    A, B, C = _inputs(case)
    Ad, Bd, Cd = A.to(dev), B.to(dev), C.to(dev)
    # 16 splits x 1024 x 1024 x 4 bytes = 64 MiB of partials > 32 MiB
    assert _call(mg, "noalloc", case, Ad, Bd, Cd, splits=16) == mg.MG_ESCRATCH
    torch.cuda.synchronize()
    assert torch.equal(Cd.cpu(), C), "C must be untouched on an error"
    # 8 splits fit (32 MiB) and run
    assert _call(mg, "noalloc", case, Ad, Bd, Cd, splits=8) == mg.MG_OK
    torch.cuda.synchronize()
    ref = oracle_full(A, B, C, alpha=1.0, beta=0.0, ta=False, tb=False, in_dtype="f32", c_dtype="f32")
    assert_bit_exact(Cd.cpu(), ref, "f32", "noalloc forced 8 splits")
