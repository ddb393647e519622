"""The whole-matrix checker the large-shape parity tests rely on
(``gpu_helpers.freivalds_stream``) and the row/column sample plan, exercised
on the CPU: correctly rounded oracle results pass, and errors planted in
them -- an all-zero C, C left as C_in, one zeroed tile, a dropped k term, a
negated row, a transposed operand, a missing beta term, a NaN -- fail.  The
shapes mirror the workloads (16-bit TN with fp16 C at K = 2048, bf16 NN with
fp32 C and beta = 1, fp32 NN with alpha = 1.5, beta = 0.5) at sizes the oracle
finishes in about a second."""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import bits, freivalds_stream, sample_plan

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _case(in_dtype, c_dtype, M, N, K, ta, tb, alpha, beta, seed, dist):
    sa = (K, M) if ta else (M, K)
    sb = (N, K) if tb else (K, N)
    A = gi.draw(*sa, dist, seed, in_dtype, scale_k=K)
    B = gi.draw(*sb, dist, seed + 1, in_dtype, scale_k=K)
    Cin = gi.draw(M, N, "uniform" if dist != "int2" else "int2", seed + 2, c_dtype) if beta else None
    ref = oracle.gemm(bits(A), bits(B), a_dtype=in_dtype, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta,
                      C=None if Cin is None else bits(Cin), c_dtype=c_dtype)
    return A, B, Cin, ref


def _as_tensor(x64, c_dtype):
    r = oracle.round_to(x64, c_dtype)
    if c_dtype == "f32":
        return torch.from_numpy(r.copy())
    return torch.from_numpy(r.view(np.int16).copy()).view(TORCH[c_dtype])


CASES = {
    # name: (in, c, M, N, K, ta, tb, alpha, beta, dist)
    "fp16_tn_k2048": ("f16", "f16", 320, 288, 2048, False, True, 1.0, 0.0, "normal_k"),
    "bf16_nn_beta1": ("bf16", "f32", 256, 320, 1024, False, False, 1.0, 1.0, "uniform"),
    "fp32_nn_ab": ("f32", "f32", 192, 160, 700, False, False, 1.5, 0.5, "uniform"),
    "fp16_tt": ("f16", "f32", 160, 192, 512, True, True, 1.0, 0.0, "normal_k"),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    in_dtype, c_dtype, M, N, K, ta, tb, alpha, beta, dist = CASES[request.param]
    A, B, Cin, ref = _case(in_dtype, c_dtype, M, N, K, ta, tb, alpha, beta, 1500, dist)
    kw = dict(alpha=alpha, beta=beta, ta=ta, tb=tb, in_dtype=in_dtype, c_dtype=c_dtype)
    return request.param, A, B, Cin, ref, kw


def _fails(C, A, B, Cin, kw):
    with pytest.raises(AssertionError):
        freivalds_stream(C, A, B, Cin, **kw)


def test_correct_result_passes(case):
    name, A, B, Cin, ref, kw = case
    freivalds_stream(_as_tensor(ref, kw["c_dtype"]), A, B, Cin, **kw)
    freivalds_stream(_as_tensor(ref, kw["c_dtype"]), A, B, Cin, chunk=37, seed=5, **kw)


def test_planted_errors_fail(case):
    name, A, B, Cin, ref, kw = case
    c = kw["c_dtype"]
    M, N = ref.shape
    _fails(_as_tensor(np.zeros_like(ref), c), A, B, Cin, kw)                  # all-zero C
    tile = ref.copy()
    tile[128:256, 128:256] = 0.0                                               # one unwritten tile
    _fails(_as_tensor(tile, c), A, B, Cin, kw)
    neg = ref.copy()
    neg[M // 3] = -neg[M // 3]                                                 # one negated row
    _fails(_as_tensor(neg, c), A, B, Cin, kw)
    nan = ref.copy()
    nan[5, 7] = np.nan
    _fails(_as_tensor(nan, c), A, B, Cin, kw)
    if Cin is not None:
        _fails(Cin.clone(), A, B, Cin, kw)                                     # C left as C_in
        no_beta = oracle.gemm(bits(A), bits(B), a_dtype=kw["in_dtype"], trans_a=kw["ta"], trans_b=kw["tb"],
                              alpha=kw["alpha"])
        _fails(_as_tensor(no_beta, c), A, B, Cin, kw)                          # beta term missing


def test_transposed_operand_fails():
    """op(B) read transposed (a square problem, so the shapes still fit)."""
    A, B, Cin, ref = _case("f16", "f16", 256, 256, 256, False, True, 1.0, 0.0, 1600, "normal_k")
    kw = dict(alpha=1.0, beta=0.0, ta=False, tb=True, in_dtype="f16", c_dtype="f16")
    wrong = oracle.gemm(bits(A), bits(B), a_dtype="f16", trans_a=False, trans_b=False)
    freivalds_stream(_as_tensor(ref, "f16"), A, B, Cin, **kw)
    _fails(_as_tensor(wrong, "f16"), A, B, Cin, kw)


def test_dropped_k_term_fails_on_random_fp32_and_exact_integer_data():
    A, B, Cin, ref = _case("f32", "f32", 96, 80, 300, False, False, 1.5, 0.5, 1700, "uniform")
    kw = dict(alpha=1.5, beta=0.5, ta=False, tb=False, in_dtype="f32", c_dtype="f32")
    dropped = oracle.gemm(bits(A)[:, :-1], bits(B)[:-1], alpha=1.5, beta=0.5, C=bits(Cin))
    _fails(_as_tensor(dropped, "f32"), A, B, Cin, kw)
    # integer data (the bit-exact twins): exact mode catches any single change
    A, B, Cin, ref = _case("bf16", "f32", 160, 96, 2048, False, False, 1.0, 1.0, 1800, "int2")
    kw = dict(alpha=1.0, beta=1.0, ta=False, tb=False, in_dtype="bf16", c_dtype="f32", exact=True)
    freivalds_stream(_as_tensor(ref, "f32"), A, B, Cin, **kw)
    dropped = oracle.gemm(bits(A)[:, 1:], bits(B)[1:], a_dtype="bf16", alpha=1.0, beta=1.0, C=bits(Cin))
    _fails(_as_tensor(dropped, "f32"), A, B, Cin, kw)
    one = ref.copy()
    one[17, 33] += 1.0
    _fails(_as_tensor(one, "f32"), A, B, Cin, kw)


def test_sample_plan_touches_every_128_band():
    for M, N in [(16384, 16384), (4096, 11008), (127, 4096), (4092, 4092)]:
        rows, cols, blocks = sample_plan(M, N, seed=11)
        assert {r // 128 for r in rows} == set(range((M + 127) // 128))
        assert {c // 128 for c in cols} == set(range((N + 127) // 128))
        assert rows[-1] == M - 1 and cols[-1] == N - 1 and rows[0] == 0 and cols[0] == 0
        assert len(blocks) == 4
